"""Integer work on the GPU, bit-exact: the forward kernel's work-item decoder
against the oracle's work list, and the decode kernel's block-table addressing
against the oracle's gather."""
import numpy as np
import pytest
import torch

import oracle as O
import variable_length_flashattention_amd as rra
from gpu_helpers import dev_bf16, dev_i32, say, device_sort_grain
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
    return items.cpu().numpy().reshape(-1, 3)[:n], bq, device_sort_grain(B, maxq, bq, D)


@pytest.mark.parametrize("seed,B,maxlen,H,D,sorted_", [
    (1, 16, 2048, 32, 128, False), (2, 4, 9000, 16, 128, False), (3, 1024, 128, 8, 64, True),
    (4, 100, 700, 3, 256, True),
    (5, 9500, 40, 1, 128, False),   # more sequences than the kernel caches in LDS
    (6, 7, 1, 5, 64, False),
    (7, 1200, 100, 2, 64, False),   # cached, but no room for the permutation
    (8, 140, 2100, 2, 256, False),  # cached, more than 64 sort keys
    (9, 600, 300, 3, 256, True),    # keys 1..12 across ten 64-sequence chunks
    (10, 64, 500, 2, 128, True),    # the smallest sorted batch
    (11, 63, 500, 2, 128, False),
])
def test_tile_map_bit_exact(seed, B, maxlen, H, D, sorted_):
    rng = np.random.Generator(np.random.PCG64(seed))
    L = rng.integers(0, maxlen + 1, size=B)
    cu = I.cu_from_lengths(L)
    got, bq, grain = device_tile_map(cu, H, D)
    assert (grain > 0) == sorted_
    ref = O.varlen_tile_map(cu, H, bq, grain)
    n = len(ref)
    assert np.array_equal(got[:n], ref)
    assert np.all(got[n:] == -1)


def test_tile_map_configs():
    for c in (I.tiny(True), I.mixed(), I.skewed(), I.many_short(64, True), I.many_short(256, True)):
        got, bq, grain = device_tile_map(c.cu_q, c.num_heads, c.head_dim)
        ref = O.varlen_tile_map(c.cu_q, c.num_heads, bq, grain)
        assert np.array_equal(got[:len(ref)], ref) and np.all(got[len(ref):] == -1), c.name


def device_gather(c, Hq):
    """Run the decode split kernel in its gather mode through the C ABI;
    returns (k_dense, v_dense) as uint16 arrays, unwritten rows 0xFFFF."""
    S, BS, Hkv, D = c.num_seqs, c.block_size, c.num_kv_heads, c.head_dim
    shape = (S, c.max_blocks * BS, Hkv, D)
    kd = torch.full(shape, -1, dtype=torch.int16, device="cuda")
    vd = torch.full(shape, -1, dtype=torch.int16, device="cuda")
    need = rra.rra_paged_decode_workspace_bytes(S, Hq, Hkv, D)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    say(f"  launch rra_debug_paged_gather S={S} Hq={Hq} Hkv={Hkv} D={D} BS={BS} max_blocks={c.max_blocks} "
        f"max_ctx={int(c.context_lens.max())}")
    rra.rra_debug_paged_gather(dev_bf16(c.k_pool), dev_bf16(c.v_pool), dev_i32(c.block_table),
                               dev_i32(c.context_lens), kd, vd, S, Hq, Hkv, D, BS, c.max_blocks, ws, ws.numel())
    torch.cuda.synchronize()
    return kd.cpu().numpy().view(np.uint16), vd.cpu().numpy().view(np.uint16)


def check_gather(c, Hq):
    kd, vd = device_gather(c, Hq)
    assert np.array_equal(kd, O.paged_gather(c.k_pool, c.block_table, c.context_lens, fill=0xFFFF)), "K loads"
    assert np.array_equal(vd, O.paged_gather(c.v_pool, c.block_table, c.context_lens, fill=0xFFFF)), "V loads"


# Block sizes below 16 hold 4 table entries per lane (windows of 256 blocks;
# entries 64 and up are fetched from the second to fourth register), 16 and
# above one per lane (windows of 64 blocks).  Contexts longer than one window
# make a piece span several windows.
GATHER_CASES = [
    # ctx, BS, Hq, Hkv, D
    ([5, 0, 37, 16, 17], 16, 2, 2, 128),
    ([1, 2, 3, 100], 1, 1, 1, 64),
    ([300, 9, 70, 1], 1, 4, 2, 128),          # 300 blocks: rel >= 64, >= 128, >= 192 and a second window
    ([1100, 3, 257, 1024], 4, 8, 2, 64),      # 275 blocks of 4
    ([600, 513, 4, 2100], 8, 4, 4, 256),      # 75 and 263 blocks of 8
    ([300, 9], 8, 8, 4, 256),
    ([1000, 64, 4097, 1], 16, 32, 8, 128),    # 257 blocks of 16: five windows of 64
    ([5000, 63, 64, 65, 1], 64, 16, 2, 64),   # 79 blocks of 64
    ([1000, 64], 32, 2, 2, 128),
]


@pytest.mark.parametrize("ctx,BS,Hq,Hkv,D", GATHER_CASES)
def test_gather_bit_exact(ctx, BS, Hq, Hkv, D):
    c = I.decode_case("g", ctx, Hq, Hkv, D, BS, seed=sum(ctx) + BS)
    check_gather(c, Hq)


def test_gather_many_sequences():
    """More sequences than the split kernel keeps offsets for in registers:
    the offsets kernel writes them into the workspace and waves search them."""
    rng = np.random.Generator(np.random.PCG64(4242))
    ctx = rng.integers(0, 200, size=700)
    for BS in (4, 16):
        c = I.decode_case("g_many", ctx, 8, 2, 128, BS, seed=4243 + BS)
        check_gather(c, 8)


def test_gather_decode_workload():
    """The paged decode workload at full size (64 sequences, contexts U[1,8192],
    Hq=32, Hkv=8, head_dim 128, 16-token blocks), in the benchmark's launch
    configuration: every K and V row the split kernel loads, bit for bit."""
    check_gather(I.paged_decode(), 32)
