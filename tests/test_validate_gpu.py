"""The debug check of sequence offsets (RRA_VALIDATE=1 in the environment),
on the GPU.  With the check on, good offsets run as usual and match the
oracle; offsets that break a precondition of the forward's sequence offsets
("Varlen Flash Attention Implementation Plan", Task 1) are rejected with
RRA_ERR_INVALID_ARG before any other kernel runs, so none of the bad calls
below reaches an attention kernel."""
import numpy as np
import pytest
import torch

import oracle as O
import variable_length_flashattention_amd as rra
from gpu_helpers import compare, dev_bf16, dev_i32, run_varlen, say
from variable_length_flashattention_amd import inputs as I
from variable_length_flashattention_amd.binding import RRA_ERR_INVALID_ARG

pytestmark = pytest.mark.gpu


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("RRA_VALIDATE", "1")


def small_case():
    return I.varlen_case("validate", [5, 130, 64], [7, 130, 70], 2, 64, seed=91, causal=True)


def expect_invalid(fn, *args):
    with pytest.raises(rra.RraError) as e:
        fn(*args)
    assert e.value.status == RRA_ERR_INVALID_ARG


def fwd_args(c, cu_q, cu_k, max_q):
    q, k, v = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    return (q, k, v, out, lse, dev_i32(cu_q), dev_i32(cu_k), max_q, len(cu_q) - 1, q.shape[1], q.shape[2], c.scale,
            True)


def test_good_offsets_pass(validate):
    c = small_case()
    say("  validated forward, good offsets")
    out, lse = run_varlen(c)
    ro, rl = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True)
    compare(out, lse, ro, rl, "validated forward")


@pytest.mark.parametrize("what", ["max_seqlen_q", "q_decreasing", "q_start", "k_decreasing", "k_start"])
def test_bad_forward_offsets(validate, what):
    c = small_case()
    cu_q, cu_k, max_q = c.cu_q.copy(), c.cu_k.copy(), c.max_seqlen_q
    if what == "max_seqlen_q":
        max_q = 100                      # a sequence has 130 query rows
    elif what == "q_decreasing":
        cu_q[1], cu_q[2] = cu_q[2], cu_q[1]
    elif what == "q_start":
        cu_q = cu_q + 1
    elif what == "k_decreasing":
        cu_k[2] = cu_k[1] - 1
    else:
        cu_k = cu_k + 3
    say(f"  validated forward, bad offsets: {what}")
    expect_invalid(rra.rra_varlen_attn_fwd, *fwd_args(c, cu_q, cu_k, max_q))


def test_bad_paged_lengths(validate):
    c = I.paged_prefill_case("validate_paged", [40, 9], [50, 20], 2, 128, 16, seed=17, causal=True,
                             num_kv_heads=2, spare_blocks=1)
    cap = c.max_blocks * c.block_size
    for bad in (cap + 1, -1):
        lens = c.seqlens_k.copy()
        lens[1] = bad
        q = dev_bf16(c.q)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        say(f"  validated paged forward, key length {bad} (capacity {cap})")
        expect_invalid(rra.rra_varlen_attn_fwd_paged, q, dev_bf16(c.k_pool), dev_bf16(c.v_pool), out, lse,
                       dev_i32(c.cu_q), dev_i32(lens), dev_i32(c.block_table), c.max_seqlen_q, c.batch, c.num_heads,
                       c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks, c.scale, True)


@pytest.mark.parametrize("what", ["max_seqlen_k", "total_q"])
def test_bad_backward_offsets(validate, what):
    c = small_case()
    q, k, v = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v)
    Tq, H, D = q.shape
    out, dout = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros((Tq, H), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    max_k = int(np.diff(c.cu_k).max())
    total_q = Tq
    if what == "max_seqlen_k":
        max_k -= 1
    else:
        total_q -= 1
    ws_bytes = rra.rra_varlen_attn_bwd_workspace_bytes(total_q, H)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    say(f"  validated backward, bad {what}")
    expect_invalid(rra.rra_varlen_attn_bwd, q, k, v, out, lse, dout, dq, dk, dv, dev_i32(c.cu_q), dev_i32(c.cu_k),
                   total_q, c.max_seqlen_q, max_k, c.batch, H, H, D, c.scale, True, ws, ws_bytes)


def test_bad_pack_offsets(validate):
    lengths = [3, 9, 4]
    cu = I.cu_from_lengths(lengths)
    row_bytes = 64
    padded = torch.zeros((len(lengths), 9, row_bytes), dtype=torch.uint8, device="cuda")
    packed = torch.zeros((int(cu[-1]), row_bytes), dtype=torch.uint8, device="cuda")
    say("  validated pack, max_seqlen below a length")
    expect_invalid(rra.rra_pack_rows, padded, packed, dev_i32(cu), len(lengths), 8, row_bytes)
    expect_invalid(rra.rra_unpack_rows, packed, padded, dev_i32(cu), len(lengths), 8, row_bytes)
    say("  validated pack, good offsets")
    rra.rra_pack_rows(padded, packed, dev_i32(cu), len(lengths), 9, row_bytes)
    torch.cuda.synchronize()
