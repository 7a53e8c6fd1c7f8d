"""Integer work on the GPU, bit-exact: the forward kernel's work-item decoder
against the oracle's work list, and the decode kernel's block-table addressing
against the oracle's gather."""
import numpy as np
import pytest
import torch

import oracle as O
import variable_length_flashattention_amd as rra
from gpu_helpers import dev_bf16, dev_i32, say
from variable_length_flashattention_amd import inputs as I

pytestmark = pytest.mark.gpu


def device_tile_map(cu, H, D):
    B = len(cu) - 1
    maxq = int(np.max(np.diff(cu))) if B else 0
    bq = rra.rra_varlen_block_q(D, maxq)
    cap = max(1, B * (-(-maxq // bq)) * H)
    items = torch.full((cap * 3,), -7, dtype=torch.int32, device="cuda")
    say(f"  launch rra_debug_varlen_tile_map B={B} H={H} D={D} maxq={maxq}")
    n = rra.rra_debug_varlen_tile_map(dev_i32(cu), B, H, maxq, D, items, cap)
    return items.cpu().numpy().reshape(-1, 3)[:n], bq


@pytest.mark.parametrize("seed,B,maxlen,H,D", [
    (1, 16, 2048, 32, 128), (2, 4, 9000, 16, 128), (3, 1024, 128, 8, 64), (4, 100, 700, 3, 256),
    (5, 9500, 40, 1, 128),  # more sequences than the kernel caches in LDS
    (6, 7, 1, 5, 64),
])
def test_tile_map_bit_exact(seed, B, maxlen, H, D):
    rng = np.random.Generator(np.random.PCG64(seed))
    L = rng.integers(0, maxlen + 1, size=B)
    cu = I.cu_from_lengths(L)
    got, bq = device_tile_map(cu, H, D)
    ref = O.varlen_tile_map(cu, H, bq)
    n = len(ref)
    assert np.array_equal(got[:n], ref)
    assert np.all(got[n:] == -1)


def test_tile_map_configs():
    for c in (I.tiny(True), I.mixed(), I.skewed(), I.many_short(64, True)):
        got, bq = device_tile_map(c.cu_q, c.num_heads, c.head_dim)
        ref = O.varlen_tile_map(c.cu_q, c.num_heads, bq)
        assert np.array_equal(got[:len(ref)], ref) and np.all(got[len(ref):] == -1), c.name


@pytest.mark.parametrize("ctx,BS,Hkv,D", [
    ([5, 0, 37, 16, 17], 16, 2, 128), ([1, 2, 3, 100], 1, 1, 64), ([300, 9], 8, 4, 256), ([1000, 64], 32, 2, 128),
])
def test_gather_bit_exact(ctx, BS, Hkv, D):
    c = I.decode_case("g", ctx, Hkv, Hkv, D, BS, seed=sum(ctx))
    dense = torch.full((c.num_seqs, c.max_blocks * BS, Hkv, D), -1, dtype=torch.int16, device="cuda")
    say(f"  launch rra_debug_paged_gather ctx={ctx} BS={BS} Hkv={Hkv} D={D}")
    rra.rra_debug_paged_gather(dev_bf16(c.k_pool), dev_i32(c.block_table), dev_i32(c.context_lens), dense,
                               c.num_seqs, Hkv, D, BS, c.max_blocks)
    got = dense.cpu().numpy().view(np.uint16)
    ref = O.paged_gather(c.k_pool, c.block_table, c.context_lens, fill=0xFFFF)
    assert np.array_equal(got, ref)
