"""GPU parity of the forward pass with paged keys and values (chunked
prefill) against the fp64 oracle, and against the packed forward pass on the
same keys gathered into a contiguous buffer."""
import numpy as np
import pytest
import torch

import oracle as O
import variable_length_flashattention_amd as rra
from gpu_helpers import compare, dev_bf16, dev_i32, host_f64, run_varlen, say
from variable_length_flashattention_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_paged(c, causal=None):
    """Launch rra_varlen_attn_fwd_paged; out/lse pre-filled with NaN so
    unwritten rows show.  Returns (out f64 [Tq,H,D], lse f64 [Tq,H])."""
    causal = c.causal if causal is None else causal
    q = dev_bf16(c.q)
    out = torch.empty_like(q)
    out.view(torch.int16).fill_(0x7FC0)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    say(f"  launch rra_varlen_attn_fwd_paged case={c.name} seed={c.seed} Tq={q.shape[0]} H={c.num_heads} "
        f"Hkv={c.num_kv_heads} D={c.head_dim} BS={c.block_size} maxb={c.max_blocks} B={c.batch} causal={causal}")
    rra.rra_varlen_attn_fwd_paged(q, dev_bf16(c.k_pool), dev_bf16(c.v_pool), out, lse, dev_i32(c.cu_q),
                                  dev_i32(c.seqlens_k), dev_i32(c.block_table), c.max_seqlen_q, c.batch, c.num_heads,
                                  c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks, c.scale, causal)
    torch.cuda.synchronize()
    return host_f64(out), lse.cpu().numpy().astype(np.float64)


CASES = [
    # name, Lq, Lk, H, Hkv, D, BS
    ("bs16_d128", [1, 17, 64, 300], [1, 40, 64, 333], 4, 4, 128, 16),
    ("bs8_d64", [129, 5, 70], [200, 5, 70], 2, 2, 64, 8),
    ("bs8_d256", [65, 3], [97, 40], 2, 1, 256, 8),
    ("bs32_gqa", [256, 100, 7], [300, 612, 519], 8, 2, 128, 32),
    ("bs64_d256", [40, 200], [40, 260], 4, 2, 256, 64),
    ("bs128_chunk", [128, 33], [1000, 700], 4, 4, 128, 128),
    ("bs1024", [70, 1], [1500, 1024], 2, 2, 64, 1024),
    ("k_shorter", [40, 200, 129], [5, 64, 1], 2, 2, 128, 16),   # fully masked rows under causal
    ("empty_seqs", [0, 50, 0, 20], [10, 0, 0, 45], 2, 2, 128, 16),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_cases(case, causal):
    name, lq, lk, H, Hkv, D, BS = case
    c = I.paged_prefill_case(name, lq, lk, H, D, BS, seed=len(name) * 13 + sum(lq) + sum(lk), causal=causal,
                             num_kv_heads=Hkv, spare_blocks=3)
    out, lse = run_paged(c)
    ref_out, ref_lse = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale,
                                           causal)
    compare(out, lse, ref_out, ref_lse, f"{name} causal={causal}")


def test_paged_table_with_spare_columns():
    """A block table wider than any sequence needs (unused entries hold -1
    and are never read)."""
    c = I.paged_prefill_case("wide_table", [90, 12], [150, 40], 2, 128, 16, seed=77, causal=True, max_blocks=40)
    out, lse = run_paged(c)
    ref_out, ref_lse = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale,
                                           True)
    compare(out, lse, ref_out, ref_lse, "wide table")


@pytest.mark.parametrize("block_size", [16, 256])
def test_chunked_full_size(block_size):
    """The skewed/chunked shape (Lq {8192,1024,128,7}, Lk {8192,3072,128,519},
    16 heads, head_dim 128, bottom-right causal) with paged K/V (the pool's
    unused slots hold NaN): bit for bit the packed forward pass on the same
    K/V, and every (token, head) row against the oracle."""
    c = I.chunked_paged(block_size)
    out, lse = run_paged(c)
    pout, plse = run_varlen(c.dense, causal=True)
    assert np.array_equal(out, pout) and np.array_equal(lse, plse), "paged differs from packed"
    ro, rl = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale, True)
    compare(out, lse, ro, rl, f"chunked paged bs{block_size}, every row")


def test_paged_convenience_wrapper():
    c = I.paged_prefill_case("wrapper", [33, 64], [50, 64], 4, 64, 16, seed=5, causal=True, num_kv_heads=2)
    out, lse = rra.varlen_attn_fwd_paged(dev_bf16(c.q), dev_bf16(c.k_pool), dev_bf16(c.v_pool), dev_i32(c.cu_q),
                                         dev_i32(c.seqlens_k), dev_i32(c.block_table), c.max_seqlen_q, c.scale, True)
    torch.cuda.synchronize()
    ref_out, ref_lse = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale,
                                           True)
    compare(host_f64(out), lse.cpu().numpy().astype(np.float64), ref_out, ref_lse, "wrapper")
