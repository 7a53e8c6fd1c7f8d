"""Seeded random shapes against the oracle: batch sizes, ragged lengths
(including empty sequences and k shorter or longer than q), head counts and
grouped-query ratios, head dims, block sizes and mask modes drawn from a
fixed list of seeds, for every entry point."""
import numpy as np
import pytest
import torch

import oracle as O
import variable_length_flashattention_amd as rra
from gpu_helpers import OUT_TOL, compare, dev_bf16, dev_i32, device_sort_grain, host_f64, run_varlen, say
from variable_length_flashattention_amd import inputs as I

pytestmark = pytest.mark.gpu

SEEDS = list(range(24))


def draw(seed):
    rng = np.random.Generator(np.random.PCG64(9000 + seed))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    H = Hkv * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 7))
    lq = rng.integers(0, 300, size=B)
    lk = np.where(rng.random(B) < 0.5, lq, rng.integers(0, 400, size=B))
    causal = bool(rng.integers(0, 2))
    return rng, D, H, Hkv, lq, lk, causal


@pytest.mark.parametrize("seed", SEEDS)
def test_forward_random(seed):
    rng, D, H, Hkv, lq, lk, causal = draw(seed)
    c = I.varlen_case(f"rand{seed}", lq, lk, H, D, seed=seed, causal=causal, num_kv_heads=Hkv)
    out, lse = run_varlen(c)
    ro, rl = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal)
    compare(out, lse, ro, rl, f"random forward {seed}")


@pytest.mark.parametrize("seed", SEEDS)
def test_paged_forward_random(seed):
    rng, D, H, Hkv, lq, lk, causal = draw(seed)
    BS = int(rng.choice([8, 16, 32, 128]))
    c = I.paged_prefill_case(f"prand{seed}", lq, lk, H, D, BS, seed=seed, causal=causal, num_kv_heads=Hkv,
                             spare_blocks=2)
    q = dev_bf16(c.q)
    say(f"  launch rra_varlen_attn_fwd_paged seed={seed} B={c.batch} H={H} Hkv={Hkv} D={D} BS={BS} causal={causal}")
    out, lse = rra.varlen_attn_fwd_paged(q, dev_bf16(c.k_pool), dev_bf16(c.v_pool), dev_i32(c.cu_q),
                                         dev_i32(c.seqlens_k), dev_i32(c.block_table), c.max_seqlen_q, c.scale,
                                         causal)
    torch.cuda.synchronize()
    ro, rl = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale, causal)
    compare(host_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"random paged forward {seed}")


def draw_many(seed):
    """Batches of 64-400 sequences (the forward kernel's length-sorted work
    list): lengths U[0,300] with empty sequences, k lengths equal to q or
    drawn apart (some 0), 1-2 kv heads."""
    rng = np.random.Generator(np.random.PCG64(9500 + seed))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2]))
    H = Hkv * int(rng.choice([1, 2]))
    B = int(rng.integers(64, 401))
    lq = rng.integers(0, 301, size=B)
    lq[rng.random(B) < 0.05] = 0
    lk = np.where(rng.random(B) < 0.7, lq, rng.integers(0, 400, size=B))
    causal = bool(rng.integers(0, 2))
    return rng, D, H, Hkv, lq, lk, causal


MANY_SEEDS = list(range(8))


@pytest.mark.parametrize("seed", MANY_SEEDS)
def test_forward_random_sorted(seed):
    rng, D, H, Hkv, lq, lk, causal = draw_many(seed)
    assert device_sort_grain(len(lq), int(lq.max()), 128, D) > 0  # the sorted kernel runs
    c = I.varlen_case(f"many{seed}", lq, lk, H, D, seed=seed, causal=causal, num_kv_heads=Hkv)
    out, lse = run_varlen(c)
    ro, rl = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal)
    compare(out, lse, ro, rl, f"random forward, sorted work list {seed}")


@pytest.mark.parametrize("seed", MANY_SEEDS[:4])
def test_paged_forward_random_sorted(seed):
    rng, D, H, Hkv, lq, lk, causal = draw_many(seed)
    assert device_sort_grain(len(lq), int(lq.max()), 128, D) > 0
    BS = int(rng.choice([8, 16, 64]))
    c = I.paged_prefill_case(f"pmany{seed}", lq, lk, H, D, BS, seed=seed, causal=causal, num_kv_heads=Hkv,
                             spare_blocks=2)
    q = dev_bf16(c.q)
    say(f"  launch rra_varlen_attn_fwd_paged (sorted) seed={seed} B={c.batch} H={H} Hkv={Hkv} D={D} BS={BS} "
        f"causal={causal}")
    out, lse = rra.varlen_attn_fwd_paged(q, dev_bf16(c.k_pool), dev_bf16(c.v_pool), dev_i32(c.cu_q),
                                         dev_i32(c.seqlens_k), dev_i32(c.block_table), c.max_seqlen_q, c.scale,
                                         causal)
    torch.cuda.synchronize()
    ro, rl = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale, causal)
    compare(host_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, f"random paged forward, sorted {seed}")


@pytest.mark.parametrize("seed", SEEDS)
def test_backward_random(seed):
    rng, D, H, Hkv, lq, lk, causal = draw(seed)
    c = I.varlen_case(f"brand{seed}", lq, lk, H, D, seed=seed, causal=causal, num_kv_heads=Hkv)
    g = I.normal_bf16(rng, c.q.shape)
    q, k, v, dout = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v), dev_bf16(g)
    cu_q, cu_k = dev_i32(c.cu_q), dev_i32(c.cu_k)
    say(f"  launch forward+backward seed={seed} B={c.batch} H={H} Hkv={Hkv} D={D} causal={causal}")
    out, lse = rra.varlen_attn_fwd(q, k, v, cu_q, cu_k, c.max_seqlen_q, c.scale, causal)
    max_k = int(np.max(np.diff(c.cu_k)))
    dq, dk, dv = rra.varlen_attn_bwd(q, k, v, out, lse, dout, cu_q, cu_k, c.max_seqlen_q, max_k, c.scale, causal)
    torch.cuda.synchronize()
    refs = O.varlen_attn_bwd(c.q, c.k, c.v, g, c.cu_q, c.cu_k, c.scale, causal)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        gg = host_f64(got)
        assert np.all(np.isfinite(gg)), name
        ratio = float(np.max(np.abs(gg - ref) / (3e-2 + 1e-2 * np.abs(ref)))) if ref.size else 0.0
        say(f"  random backward {seed} {name}: error / bound = {ratio:.3f}")
        assert ratio <= 1.0, (name, ratio)


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_random(seed):
    rng = np.random.Generator(np.random.PCG64(9500 + seed))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 8]))
    Hq = Hkv * int(rng.choice([1, 4, 8, 32]))
    BS = int(rng.choice([1, 4, 16, 64]))
    S = int(rng.choice([1, 3, 40, 300]))
    ctx = rng.integers(0, {1: 3000, 3: 1000, 40: 200, 300: 100}[S], size=S)
    c = I.decode_case(f"drand{seed}", ctx, Hq, Hkv, D, BS, seed=seed)
    q = dev_bf16(c.q)
    say(f"  launch rra_paged_decode_attn seed={seed} S={S} Hq={Hq} Hkv={Hkv} D={D} BS={BS}")
    out = rra.paged_decode_attn(q, dev_bf16(c.k_pool), dev_bf16(c.v_pool), dev_i32(c.block_table),
                                dev_i32(c.context_lens), c.scale)
    torch.cuda.synchronize()
    ref = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale)
    got = host_f64(out)
    assert np.all(np.isfinite(got))
    e = float(np.max(np.abs(got - ref)))
    say(f"  random decode {seed}: max|dout|={e:.3e}")
    assert e <= OUT_TOL


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_decode_steps_random(seed):
    """The stateful decode over random tiles of blocks equals the oracle's
    step and finalize."""
    from oracle_pins import split_into_tiles
    rng = np.random.Generator(np.random.PCG64(9700 + seed))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 4, 16]))
    BS = int(rng.choice([1, 8, 16, 32]))
    S = int(rng.choice([1, 5, 70, 280]))
    ctx = rng.integers(0, {1: 2000, 5: 600, 70: 150, 280: 60}[S], size=S)
    c = I.decode_case(f"srand{seed}", ctx, Hq, Hkv, D, BS, seed=seed)
    tiles = split_into_tiles(c, rng, max_cap=int(rng.integers(1, 9)))
    q, kp, vp = dev_bf16(c.q), dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    say(f"  launch stateful decode seed={seed} S={S} Hq={Hq} Hkv={Hkv} D={D} BS={BS} steps={len(tiles)}")
    st = rra.decode_state_init(S, Hq, D, "cuda")
    ref = O.decode_state_init(S, Hq, D)
    for tb, cnt, tok in tiles:
        rra.paged_decode_step(st, q, kp, vp, dev_i32(tb), dev_i32(cnt), c.scale, token_counts=dev_i32(tok))
        O.paged_decode_step(ref, c.q, c.k_pool, c.v_pool, tb, cnt, c.scale, token_counts=tok)
    out = rra.paged_decode_finalize(st)
    torch.cuda.synchronize()
    got, want = host_f64(out), O.paged_decode_finalize(ref)
    assert np.all(np.isfinite(got))
    e = float(np.max(np.abs(got - want))) if got.size else 0.0
    say(f"  random stateful decode {seed}: {len(tiles)} steps, max|dout|={e:.3e}")
    assert e <= OUT_TOL
