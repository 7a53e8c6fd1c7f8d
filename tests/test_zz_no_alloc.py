"""The allocation-free decode entry point (static device scratch) through the
C ABI: two calls in a row, the second on a smaller input, each against the
workspace entry point's output on the same inputs (bit for bit: the same
kernels on the same partial-state layout) and against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import variable_length_flashattention_amd as rra
from gpu_helpers import OUT_TOL, dev_bf16, dev_i32, host_f64, say
from variable_length_flashattention_amd import inputs as I

pytestmark = pytest.mark.gpu


def decode_both(c):
    q, kp, vp = dev_bf16(c.q), dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    bt, cl = dev_i32(c.block_table), dev_i32(c.context_lens)
    args = (c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks, c.scale)
    out_ws = torch.empty_like(q)
    out_ws.view(torch.int16).fill_(0x7FC0)
    need = rra.rra_paged_decode_workspace_bytes(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    say(f"  launch rra_paged_decode_attn case={c.name} S={c.num_seqs} Hq={c.num_q_heads} Hkv={c.num_kv_heads} "
        f"D={c.head_dim} BS={c.block_size}")
    rra.rra_paged_decode_attn(q, kp, vp, bt, cl, out_ws, *args, ws, ws.numel())
    torch.cuda.synchronize()
    out_na = torch.empty_like(q)
    out_na.view(torch.int16).fill_(0x7FC0)
    say(f"  launch rra_paged_decode_attn_noalloc case={c.name} (workspace need {need} bytes)")
    rra.rra_paged_decode_attn_noalloc(q, kp, vp, bt, cl, out_na, *args)
    torch.cuda.synchronize()
    return host_f64(out_ws), host_f64(out_na)


def check(c):
    got_ws, got_na = decode_both(c)
    assert np.array_equal(got_na, got_ws), f"{c.name}: no-alloc output differs from the workspace entry point"
    ref = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale)
    err = float(np.max(np.abs(got_na - ref)))
    say(f"  {c.name}: max|dout| vs oracle {err:.3e}")
    assert np.all(np.isfinite(got_na)) and err <= OUT_TOL


def test_noalloc_two_calls_second_smaller():
    # first: the paged decode workload at full size (64 seqs, ctx U[1,8192],
    # 32 q / 8 kv heads, head_dim 128); second: a smaller one with a
    # different layout of the scratch (head_dim 64, 2 kv heads, 5 seqs,
    # one of them empty), which must not see the first call's partial states
    check(I.paged_decode())
    check(I.decode_case("small_after", [1, 37, 300, 0, 17], 8, 2, 64, 16, seed=5555))


def test_noalloc_many_sequences():
    """Above 256 sequences the token-group offsets also live in the scratch."""
    rng = np.random.Generator(np.random.PCG64(812))
    check(I.decode_case("many", rng.integers(0, 300, 700).tolist(), 8, 2, 128, 16, seed=813))
    check(I.decode_case("small_after_many", [5, 0, 33], 4, 4, 256, 8, seed=814))
