"""Checks that pin the CPU oracle to facts fixed by the pages and by
mathematics, independently of the oracle's own code.

Every ``pin_*`` function takes a loaded oracle library handle (the real one,
or a deliberately broken copy in the mutation test) and raises AssertionError
when the oracle disagrees.  Sources: "Varlen Flash Attention Implementation
Plan" (Task 1 kernel, Task 2 CPU simulation and tests) and
"spark_storage/attention_ref.rs" (step_tile_ref, finalize_ref).
"""
from __future__ import annotations

import math

import numpy as np

import oracle as O
from golden_cases import check as golden_check
from golden_cases import golden_files
from golden_cases import load as golden_load
from variable_length_flashattention_amd.inputs import (bf16_bits, bf16_to_f32, cu_from_lengths, decode_case,
                                                       paged_prefill_case, varlen_case)


# --- an independent brute force ------------------------------------------------

def brute_force_varlen(q, k, v, cu_q, cu_k, scale, causal):
    """softmax over the whole packed [Tq x Tk] score matrix with a block
    diagonal (same-sequence) mask and the bottom-right causal rule, summed with
    math.fsum.  Written against the definition, not the oracle's loops.  k, v
    may have fewer heads than q: query head h uses kv head h // (H // Hkv),
    the contiguous grouping of the decode page."""
    qf, kf, vf = (bf16_to_f32(x).astype(np.float64) for x in (q, k, v))
    Tq, H, D = qf.shape
    Tk = kf.shape[0]
    R = H // kf.shape[1]
    B = len(cu_q) - 1
    seq_q = np.full(Tq, -1)
    seq_k = np.full(Tk, -1)
    for b in range(B):
        seq_q[cu_q[b]:cu_q[b + 1]] = b
        seq_k[cu_k[b]:cu_k[b + 1]] = b
    out = np.full((Tq, H, D), np.nan)
    lse = np.full((Tq, H), np.nan)
    for tq in range(Tq):
        b = seq_q[tq]
        if b < 0:
            continue
        i = tq - cu_q[b]
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for h in range(H):
            logits = []
            for tk in range(Tk):
                if seq_k[tk] != b:
                    continue
                j = tk - cu_k[b]
                if causal and j > i + Lk - Lq:
                    continue
                logits.append((scale * math.fsum(qf[tq, h, d] * kf[tk, h // R, d] for d in range(D)), tk))
            if not logits:
                out[tq, h] = 0.0
                lse[tq, h] = -math.inf
                continue
            M = max(s for s, _ in logits)
            w = [(math.exp(s - M), tk) for s, tk in logits]
            Z = math.fsum(x for x, _ in w)
            for d in range(D):
                out[tq, h, d] = math.fsum(x * vf[tk, h // R, d] for x, tk in w) / Z
            lse[tq, h] = M + math.log(Z)
    return out, lse


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    with np.errstate(invalid="ignore"):
        same_special = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))) | (np.isnan(a) & np.isnan(b))
        ok = same_special | (np.abs(a - b) <= tol * (1.0 + np.abs(b)))
    assert np.all(ok), f"{what}: max diff {np.nanmax(np.where(ok, 0, np.abs(a - b)))}"


def _random_case(rng, B, H, D, max_len, allow_short_k=True, Hkv=None):
    lq = rng.integers(0, max_len + 1, size=B)
    if allow_short_k:
        lk = rng.integers(0, max_len + 1, size=B)
    else:
        lk = lq + rng.integers(0, 4, size=B)
    return varlen_case("rand", lq, lk, H, D, int(rng.integers(1 << 30)), False, rng=rng, num_kv_heads=Hkv)


# --- prefill pins -----------------------------------------------------------------

def pin_bruteforce_tiny(lib):
    """Oracle == brute force on tiny random packs (empty sequences, Lk < Lq,
    Lk > Lq, fully masked rows), both causal modes, within 1e-12."""
    rng = np.random.Generator(np.random.PCG64(11))
    for trial in range(10):
        c = _random_case(rng, B=int(rng.integers(1, 5)), H=int(rng.integers(1, 3)), D=int(rng.choice([4, 8, 16])),
                         max_len=9)
        for causal in (False, True):
            o1, l1 = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
            o2, l2 = brute_force_varlen(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal)
            _close(o1, o2, 1e-12, f"out trial {trial} causal {causal}")
            _close(l1, l2, 1e-12, f"lse trial {trial} causal {causal}")


def pin_golden_plan_examples(lib):
    """Worked examples of the plan page's CPU tests (tests/golden/plan_*.json)."""
    def run(q, k, v, cu, scale, causal):
        return O.varlen_attn(q, k, v, cu, cu, scale, causal, lib=lib)
    files = golden_files("plan_")
    assert len(files) == 6
    for f in files:
        golden_check(golden_load(f), run)


def pin_constant_values(lib):
    """V == c everywhere gives out == c on every row that sees a key."""
    rng = np.random.Generator(np.random.PCG64(12))
    c = varlen_case("c", [5, 9, 1], [7, 9, 3], 2, 8, 3, False, rng=rng)
    v = bf16_bits(np.full(c.v.shape, -1.75, np.float32))
    for causal in (False, True):
        out, lse = O.varlen_attn(c.q, c.k, v, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
        _close(out, np.full(out.shape, -1.75), 1e-13, f"V==c causal {causal}")


def pin_single_key(lib):
    """One visible key j gives out == v_j and lse == scale * q.k_j."""
    rng = np.random.Generator(np.random.PCG64(13))
    c = varlen_case("c", [3, 4], [1, 1], 2, 8, 4, False, rng=rng)
    out, lse = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, False, lib=lib)
    qf, kf, vf = (bf16_to_f32(x).astype(np.float64) for x in (c.q, c.k, c.v))
    for b in range(2):
        for t in range(c.cu_q[b], c.cu_q[b + 1]):
            for h in range(2):
                kt = c.cu_k[b]
                _close(out[t, h], vf[kt, h], 1e-14, "single key out")
                _close(lse[t, h], c.scale * float(np.dot(qf[t, h], kf[kt, h])), 1e-13, "single key lse")


def pin_zero_query_uniform(lib):
    """q == 0 gives uniform weights: out = mean of the visible v rows and
    lse = ln(#visible).  With Lk > Lq the causal count is i + Lk - Lq + 1
    (bottom-right); with Lk < Lq rows i < Lq - Lk see nothing (out 0, lse -inf)."""
    rng = np.random.Generator(np.random.PCG64(14))
    c = varlen_case("c", [4, 6], [7, 3], 1, 4, 5, False, rng=rng)
    q0 = np.zeros_like(c.q)
    vf = bf16_to_f32(c.v).astype(np.float64)
    for causal in (False, True):
        out, lse = O.varlen_attn(q0, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
        for b in range(2):
            Lq, Lk = c.cu_q[b + 1] - c.cu_q[b], c.cu_k[b + 1] - c.cu_k[b]
            for i in range(Lq):
                n = Lk if not causal else max(0, min(Lk, i + Lk - Lq + 1))
                t = c.cu_q[b] + i
                if n == 0:
                    assert np.all(out[t] == 0.0) and np.all(lse[t] == -np.inf), (b, i)
                    continue
                keys = slice(c.cu_k[b], c.cu_k[b] + n)
                _close(out[t, 0], vf[keys, 0].mean(axis=0), 1e-14, f"uniform out b{b} i{i}")
                _close(lse[t, 0], math.log(n), 1e-14, f"uniform lse b{b} i{i}")


def pin_packed_equals_per_sequence(lib):
    """Varlen output equals the output of each sequence run on its own."""
    rng = np.random.Generator(np.random.PCG64(15))
    c = varlen_case("c", [5, 0, 12, 3], [5, 2, 12, 8], 2, 16, 6, False, rng=rng)
    for causal in (False, True):
        out, lse = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
        for b in range(c.batch):
            qs, qe, ks, ke = c.cu_q[b], c.cu_q[b + 1], c.cu_k[b], c.cu_k[b + 1]
            if qe == qs:
                continue
            cu1 = np.array([0, qe - qs], np.int32)
            cuk1 = np.array([0, ke - ks], np.int32)
            o1, l1 = O.varlen_attn(c.q[qs:qe], c.k[ks:ke], c.v[ks:ke], cu1, cuk1, c.scale, causal, lib=lib)
            assert np.array_equal(o1, out[qs:qe]) and np.array_equal(l1, lse[qs:qe]), (b, causal)


def pin_key_permutation(lib):
    """Without a causal mask the result does not depend on key order within a sequence."""
    rng = np.random.Generator(np.random.PCG64(16))
    c = varlen_case("c", [6, 9], [10, 4], 2, 8, 7, False, rng=rng)
    out, lse = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, False, lib=lib)
    perm = np.arange(c.k.shape[0])
    for b in range(c.batch):
        perm[c.cu_k[b]:c.cu_k[b + 1]] = rng.permutation(np.arange(c.cu_k[b], c.cu_k[b + 1]))
    o2, l2 = O.varlen_attn(c.q, c.k[perm], c.v[perm], c.cu_q, c.cu_k, c.scale, False, lib=lib)
    _close(o2, out, 1e-13, "key permutation out")
    _close(l2, lse, 1e-13, "key permutation lse")


def pin_sequence_isolation_and_order(lib):
    """Changing another sequence leaves a sequence's rows bit-identical;
    reversing the sequence order reverses the rows."""
    rng = np.random.Generator(np.random.PCG64(17))
    c = varlen_case("c", [4, 7, 3], [4, 9, 3], 2, 8, 8, True, rng=rng)
    out, lse = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True, lib=lib)
    k2, v2 = c.k.copy(), c.v.copy()
    k2[c.cu_k[0]:c.cu_k[1]] = bf16_bits(rng.standard_normal(k2[c.cu_k[0]:c.cu_k[1]].shape).astype(np.float32))
    v2[c.cu_k[2]:c.cu_k[3]] = bf16_bits(rng.standard_normal(v2[c.cu_k[2]:c.cu_k[3]].shape).astype(np.float32))
    o2, l2 = O.varlen_attn(c.q, k2, v2, c.cu_q, c.cu_k, c.scale, True, lib=lib)
    s = slice(c.cu_q[1], c.cu_q[2])
    assert np.array_equal(o2[s], out[s]) and np.array_equal(l2[s], lse[s])
    # reversed order
    lq, lk = np.diff(c.cu_q)[::-1], np.diff(c.cu_k)[::-1]
    qr = np.concatenate([c.q[c.cu_q[b]:c.cu_q[b + 1]] for b in reversed(range(3))])
    kr = np.concatenate([c.k[c.cu_k[b]:c.cu_k[b + 1]] for b in reversed(range(3))])
    vr = np.concatenate([c.v[c.cu_k[b]:c.cu_k[b + 1]] for b in reversed(range(3))])
    o3, l3 = O.varlen_attn(qr, kr, vr, cu_from_lengths(lq), cu_from_lengths(lk), c.scale, True, lib=lib)
    orr = np.concatenate([out[c.cu_q[b]:c.cu_q[b + 1]] for b in reversed(range(3))])
    lrr = np.concatenate([lse[c.cu_q[b]:c.cu_q[b + 1]] for b in reversed(range(3))])
    assert np.array_equal(o3, orr) and np.array_equal(l3, lrr)


def pin_scale_homogeneity(lib):
    """softmax(scale * q.k): doubling q (exact in bf16) and halving the scale
    changes nothing, while doubling only the scale does."""
    rng = np.random.Generator(np.random.PCG64(18))
    c = varlen_case("c", [5, 8], [6, 8], 2, 8, 9, False, rng=rng)
    out, lse = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, True, lib=lib)
    q2 = bf16_bits(bf16_to_f32(c.q) * 2.0)
    o2, l2 = O.varlen_attn(q2, c.k, c.v, c.cu_q, c.cu_k, c.scale / 2, True, lib=lib)
    _close(o2, out, 1e-13, "scale homogeneity out")
    _close(l2, lse, 1e-13, "scale homogeneity lse")


def pin_sampled_rows_match_full(lib):
    """The sampled-row entry point returns exactly the rows of the full pass."""
    rng = np.random.Generator(np.random.PCG64(19))
    c = varlen_case("c", [7, 0, 20, 5], [9, 3, 20, 5], 3, 16, 10, True, rng=rng)
    for causal in (False, True):
        out, lse = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
        rows = np.array([[t, h] for t in range(0, int(c.cu_q[-1]), 3) for h in range(3)], np.int32)
        o2, l2 = O.varlen_attn_rows(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, rows, lib=lib)
        assert np.array_equal(o2, out[rows[:, 0], rows[:, 1]]) and np.array_equal(l2, lse[rows[:, 0], rows[:, 1]])


# --- decode pins --------------------------------------------------------------------

def _small_decode(seed, ctx, Hq=4, Hkv=2, D=8, BS=4, max_blocks=None):
    return decode_case("d", ctx, Hq, Hkv, D, BS, seed, max_blocks=max_blocks)


def pin_gqa_prefill(lib):
    """Grouped-query prefill (query head h reads kv head h // (H // Hkv), the
    grouping of step_tile_ref in "spark_storage/attention_ref.rs"): equals the
    brute force on tiny packs, and equals plain multi-head attention on K/V
    whose heads are repeated H // Hkv times, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(23))
    for trial, (H, Hkv) in enumerate([(4, 2), (4, 1), (6, 3), (6, 2)]):
        c = _random_case(rng, B=3, H=H, D=8, max_len=7, Hkv=Hkv)
        for causal in (False, True):
            o1, l1 = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
            o2, l2 = brute_force_varlen(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal)
            _close(o1, o2, 1e-12, f"gqa out trial {trial} causal {causal}")
            _close(l1, l2, 1e-12, f"gqa lse trial {trial} causal {causal}")
            R = H // Hkv
            o3, l3 = O.varlen_attn(c.q, np.repeat(c.k, R, axis=1), np.repeat(c.v, R, axis=1), c.cu_q, c.cu_k,
                                   c.scale, causal, lib=lib)
            assert np.array_equal(o1, o3, equal_nan=True) and np.array_equal(l1, l3, equal_nan=True), \
                f"gqa vs repeated heads, trial {trial}"


def _gather_pool(pool, block_table, lengths):
    """Packed [sum Lk, Hkv, D] rows of each sequence's keys, read from the pool
    by numpy fancy indexing (token j of sequence b: slot j % BS of block
    block_table[b, j // BS])."""
    BS = pool.shape[1]
    parts = []
    for b, L in enumerate(lengths):
        j = np.arange(int(L))
        parts.append(pool[block_table[b, j // BS], j % BS])
    return np.concatenate(parts) if parts else pool[:0, 0]


def pin_paged_prefill(lib):
    """Paged keys and values (chunked prefill).  (1) Equals the packed forward
    pass on K/V gathered from the pool by numpy indexing, bit for bit, and the
    brute force within 1e-12, over block sizes 1..16, GQA, Lk < Lq, Lk > Lq
    and empty sequences; pool slots past the keys hold NaN and never leak.
    (2) The bottom-right reading: a chunk holding the last Lq queries of a
    sequence, with all L keys visible to it, gives exactly the rows L-Lq..L-1
    of the causal self-attention over the whole sequence."""
    rng = np.random.Generator(np.random.PCG64(41))
    for trial, (BS, H, Hkv) in enumerate([(1, 2, 2), (2, 4, 2), (4, 2, 1), (8, 3, 3), (16, 4, 4), (4, 6, 2)]):
        B = int(rng.integers(1, 5))
        lq = rng.integers(0, 10, size=B)
        lk = rng.integers(0, 14, size=B)
        c = paged_prefill_case("p", lq, lk, H, 8, BS, int(rng.integers(1 << 30)), True, num_kv_heads=Hkv,
                               spare_blocks=int(rng.integers(0, 3)))
        kg = _gather_pool(c.k_pool, c.block_table, c.seqlens_k)
        vg = _gather_pool(c.v_pool, c.block_table, c.seqlens_k)
        assert np.array_equal(kg, c.dense.k) and np.array_equal(vg, c.dense.v)  # the generator's own layout
        cu_k = cu_from_lengths(c.seqlens_k)
        for causal in (False, True):
            o1, l1 = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale,
                                         causal, lib=lib)
            o2, l2 = O.varlen_attn(c.q, kg, vg, c.cu_q, cu_k, c.scale, causal, lib=lib)
            assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True), \
                f"paged vs gathered, trial {trial} causal {causal}"
            o3, l3 = brute_force_varlen(c.q, kg, vg, c.cu_q, cu_k, c.scale, causal)
            _close(o1, o3, 1e-12, f"paged out trial {trial} causal {causal}")
            _close(l1, l3, 1e-12, f"paged lse trial {trial} causal {causal}")
            assert not np.any(np.isnan(o1)) and not np.any(np.isnan(l1)), f"NaN leaked, trial {trial}"
            rows = np.array([[t, t % H] for t in range(int(c.cu_q[-1]))], dtype=np.int32).reshape(-1, 2)
            if len(rows):
                o4, l4 = O.varlen_attn_paged(c.q, c.k_pool, c.v_pool, c.cu_q, c.seqlens_k, c.block_table, c.scale,
                                             causal, rows=rows, lib=lib)
                assert np.array_equal(o4, o1[rows[:, 0], rows[:, 1]]) and \
                    np.array_equal(l4, l1[rows[:, 0], rows[:, 1]]), f"paged sampled rows, trial {trial}"
    # chunked prefill: the last Lq queries of each sequence against all L keys
    L = [13, 7, 20]
    chunk = [5, 7, 1]
    full = paged_prefill_case("full", L, L, 2, 8, 4, 43, True)
    of, lf = O.varlen_attn_paged(full.q, full.k_pool, full.v_pool, full.cu_q, full.seqlens_k, full.block_table,
                                 full.scale, True, lib=lib)
    sel = np.concatenate([np.arange(full.cu_q[b] + L[b] - chunk[b], full.cu_q[b + 1]) for b in range(3)])
    oc, lc = O.varlen_attn_paged(full.q[sel], full.k_pool, full.v_pool, cu_from_lengths(chunk), full.seqlens_k,
                                 full.block_table, full.scale, True, lib=lib)
    assert np.array_equal(oc, of[sel]) and np.array_equal(lc, lf[sel]), "chunk rows differ from the full prefill"


def _torch_attention_grads(q, k, v, dout, cu_q, cu_k, scale, causal):
    """dq, dk, dv by torch autograd (CPU, float64) of a dense masked softmax
    attention per sequence; kv head h // (H // Hkv) via repeat_interleave."""
    import torch
    qf, kf, vf, gf = (torch.from_numpy(bf16_to_f32(x).astype(np.float64)) for x in (q, k, v, dout))
    qf.requires_grad_(True)
    kf.requires_grad_(True)
    vf.requires_grad_(True)
    R = qf.shape[1] // kf.shape[1]
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(len(cu_q) - 1):
        qs, ks, vs = qf[cu_q[b]:cu_q[b + 1]], kf[cu_k[b]:cu_k[b + 1]], vf[cu_k[b]:cu_k[b + 1]]
        Lq, Lk = qs.shape[0], ks.shape[0]
        if Lq == 0 or Lk == 0:
            continue
        kr = ks.repeat_interleave(R, dim=1).transpose(0, 1)    # [H, Lk, D]
        vr = vs.repeat_interleave(R, dim=1).transpose(0, 1)
        s = scale * torch.matmul(qs.transpose(0, 1), kr.transpose(1, 2))  # [H, Lq, Lk]
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lk)[None, :]
        vis = (j <= i + Lk - Lq) if causal else torch.ones(Lq, Lk, dtype=torch.bool)
        s = s.masked_fill(~vis, float("-inf"))
        has = vis.any(dim=1)                                     # rows with a visible key
        p = torch.softmax(s[:, has], dim=-1)
        o = torch.matmul(p, vr)                                  # [H, rows, D]
        loss = loss + (o * gf[cu_q[b]:cu_q[b + 1]].transpose(0, 1)[:, has]).sum()
    loss.backward()
    z = lambda t: t.grad.numpy() if t.grad is not None else np.zeros(t.shape)
    return z(qf), z(kf), z(vf)


def _f64_forward_loss(qf, kf, vf, gf, cu_q, cu_k, scale, causal):
    """sum(out * dout) of the forward definition on float64 inputs (numpy)."""
    R = qf.shape[1] // kf.shape[1]
    total = 0.0
    for b in range(len(cu_q) - 1):
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(Lq):
            for h in range(qf.shape[1]):
                js = [j for j in range(Lk) if not causal or j <= i + Lk - Lq]
                if not js:
                    continue
                x = np.array([scale * np.dot(qf[cu_q[b] + i, h], kf[cu_k[b] + j, h // R]) for j in js])
                w = np.exp(x - x.max())
                w /= w.sum()
                o = sum(wj * vf[cu_k[b] + j, h // R] for wj, j in zip(w, js))
                total += float(np.dot(o, gf[cu_q[b] + i, h]))
    return total


def pin_backward(lib):
    """Gradients of sum(out * dout): (1) equal torch autograd of a dense masked
    softmax attention (float64, CPU) within 1e-10 over empty sequences,
    Lk < Lq, Lk > Lq, both causal modes and grouped-query K/V; (2) equal
    central finite differences of the float64 forward definition; (3) the
    closed forms sum_j dK_j = 0 (softmax rows sum to one, so the dS rows sum
    to zero) and sum_j dV_j = sum of dO over rows with a visible key, per
    (sequence, kv head)."""
    rng = np.random.Generator(np.random.PCG64(51))
    for trial, (H, Hkv) in enumerate([(2, 2), (4, 2), (3, 1), (2, 2), (4, 4)]):
        c = _random_case(rng, B=int(rng.integers(1, 4)), H=H, D=8, max_len=8, Hkv=Hkv)
        dout = normal_bf16_like(rng, c.q.shape)
        for causal in (False, True):
            dq, dk, dv = O.varlen_attn_bwd(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
            tq, tk, tv = _torch_attention_grads(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal)
            _close(dq, tq, 1e-10, f"dq trial {trial} causal {causal}")
            _close(dk, tk, 1e-10, f"dk trial {trial} causal {causal}")
            _close(dv, tv, 1e-10, f"dv trial {trial} causal {causal}")
            gf = bf16_to_f32(dout).astype(np.float64)
            R = H // Hkv
            for b in range(c.batch):
                ks, ke = c.cu_k[b], c.cu_k[b + 1]
                if ke == ks:
                    continue
                Lq, Lk = c.cu_q[b + 1] - c.cu_q[b], ke - ks
                assert np.all(np.abs(dk[ks:ke].sum(axis=0)) <= 1e-12 * (1 + np.abs(dk[ks:ke]).sum(axis=0))), \
                    f"sum of dK, trial {trial}"
                for kh in range(Hkv):
                    want = np.zeros(c.head_dim)
                    for i in range(Lq):
                        if not causal or i + Lk - Lq >= 0:
                            want += gf[c.cu_q[b] + i, kh * R:(kh + 1) * R].sum(axis=0)
                    _close(dv[ks:ke, kh].sum(axis=0), want, 1e-12, f"sum of dV, trial {trial}")
    # finite differences on one small case
    c = _random_case(np.random.Generator(np.random.PCG64(52)), B=2, H=2, D=4, max_len=5, Hkv=1)
    dout = normal_bf16_like(rng, c.q.shape)
    qf, kf, vf, gf = (bf16_to_f32(x).astype(np.float64) for x in (c.q, c.k, c.v, dout))
    for causal in (False, True):
        grads = O.varlen_attn_bwd(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
        for which, (arr, g) in enumerate(zip((qf, kf, vf), grads)):
            if arr.shape[0] == 0:
                continue
            for _ in range(4):
                idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
                eps = 1e-6
                arr[idx] += eps
                up = _f64_forward_loss(qf, kf, vf, gf, c.cu_q, c.cu_k, c.scale, causal)
                arr[idx] -= 2 * eps
                dn = _f64_forward_loss(qf, kf, vf, gf, c.cu_q, c.cu_k, c.scale, causal)
                arr[idx] += eps
                fd = (up - dn) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(fd)), f"finite difference {which} {idx}: {fd} vs {g[idx]}"


def _softmax_probs(q, k, cu_q, cu_k, scale, causal):
    """Dense per-sequence probabilities P[b] (numpy float64, [H, Lq, Lk],
    rows without a visible key all 0), straight from the definition."""
    qf, kf = bf16_to_f32(q).astype(np.float64), bf16_to_f32(k).astype(np.float64)
    R = qf.shape[1] // kf.shape[1]
    probs = []
    for b in range(len(cu_q) - 1):
        qs, ks = qf[cu_q[b]:cu_q[b + 1]], np.repeat(kf[cu_k[b]:cu_k[b + 1]], R, axis=1)
        Lq, Lk = qs.shape[0], ks.shape[0]
        s = scale * np.einsum("ihd,jhd->hij", qs, ks)
        vis = (np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + Lk - Lq) if causal else np.ones((Lq, Lk), bool)
        s = np.where(vis[None], s, -np.inf)
        m = np.max(s, axis=2, keepdims=True) if Lk else np.zeros((qs.shape[1], Lq, 1))
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m)
        z = e.sum(axis=2, keepdims=True)
        probs.append(np.divide(e, z, out=np.zeros_like(e), where=z > 0))
    return probs


def pin_backward_given_out(lib):
    """The backward with the softmax Jacobian's row term taken from a given
    out: (1) with the exact forward out it equals the exact gradients
    (dO_i . out_i = sum_j P_ij dP_ij) within 1e-12; (2) with out + delta it
    differs from them by the closed form of a shifted row term:
    dq_i -= scale (dO_i . delta_i) sum_j P_ij k_j, dk_j -= scale sum_i P_ij
    (dO_i . delta_i) q_i, and dv is unchanged (it has no row term)."""
    rng = np.random.Generator(np.random.PCG64(53))
    for trial, (H, Hkv) in enumerate([(2, 2), (4, 2), (3, 1)]):
        c = _random_case(rng, B=int(rng.integers(1, 4)), H=H, D=8, max_len=8, Hkv=Hkv)
        dout = normal_bf16_like(rng, c.q.shape)
        for causal in (False, True):
            exact = O.varlen_attn_bwd(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
            out, _ = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal, lib=lib)
            out0 = np.nan_to_num(out)
            same = O.varlen_attn_bwd(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal, out=out0, lib=lib)
            for name, a, b in zip(("dq", "dk", "dv"), same, exact):
                _close(a, b, 1e-12, f"given exact out, {name}, trial {trial} causal {causal}")
            delta = rng.standard_normal(out0.shape)
            shifted = O.varlen_attn_bwd(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal, out=out0 + delta,
                                        lib=lib)
            gf = bf16_to_f32(dout).astype(np.float64)
            qf, kf = bf16_to_f32(c.q).astype(np.float64), bf16_to_f32(c.k).astype(np.float64)
            R = H // Hkv
            want_dq, want_dk = exact[0].copy(), exact[1].copy()
            for b, P in enumerate(_softmax_probs(c.q, c.k, c.cu_q, c.cu_k, c.scale, causal)):
                qs, qe, ks, ke = c.cu_q[b], c.cu_q[b + 1], c.cu_k[b], c.cu_k[b + 1]
                t = np.einsum("ihd,ihd->hi", gf[qs:qe], delta[qs:qe])          # dO_i . delta_i, [H, Lq]
                kr = np.repeat(kf[ks:ke], R, axis=1)                            # [Lk, H, D]
                want_dq[qs:qe] -= c.scale * np.einsum("hi,hij,jhd->ihd", t, P, kr)
                dk_h = c.scale * np.einsum("hij,hi,ihd->jhd", P, t, qf[qs:qe])  # per query head
                want_dk[ks:ke] -= dk_h.reshape(ke - ks, Hkv, R, c.head_dim).sum(axis=2)
            _close(shifted[0], want_dq, 1e-11, f"shifted out, dq, trial {trial} causal {causal}")
            _close(shifted[1], want_dk, 1e-11, f"shifted out, dk, trial {trial} causal {causal}")
            _close(shifted[2], exact[2], 1e-12, f"shifted out, dv, trial {trial} causal {causal}")


def normal_bf16_like(rng, shape):
    return bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def pin_decode_direct_equals_recurrence(lib):
    """The direct softmax definition and the decode page's per-token (m, l, o)
    recurrence with state carried across tiles agree to fp64 rounding."""
    c = _small_decode(21, [1, 5, 16, 17, 0, 33], max_blocks=10)
    out = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale, lib=lib)
    for cap in (1, 3, 100):
        r = O.paged_decode_recurrent(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale, cap, lib=lib)
        _close(r, out, 1e-12, f"recurrence tile_capacity {cap}")


def pin_decode_equals_varlen_single_query(lib):
    """Decode equals the packed forward pass with one query per sequence on the
    gathered K/V rows, q head qh reading kv head qh // (Hq / Hkv)."""
    c = _small_decode(22, [3, 9, 14, 1], Hq=6, Hkv=2, D=16, BS=4)
    out = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale, lib=lib)
    R = c.num_q_heads // c.num_kv_heads
    ks, vs = [], []
    for s in range(c.num_seqs):
        t = np.arange(c.context_lens[s])
        blk = c.block_table[s, t // c.block_size]
        kk = c.k_pool[blk, t % c.block_size]         # [ctx, Hkv, D]
        vv = c.v_pool[blk, t % c.block_size]
        ks.append(np.repeat(kk, R, axis=1))          # head qh -> kv head qh // R
        vs.append(np.repeat(vv, R, axis=1))
    cu_q = np.arange(c.num_seqs + 1, dtype=np.int32)
    cu_k = cu_from_lengths(c.context_lens)
    o2, _ = O.varlen_attn(c.q, np.concatenate(ks), np.concatenate(vs), cu_q, cu_k, c.scale, False, lib=lib)
    _close(out, o2, 1e-12, "decode vs varlen")


def split_into_tiles(case, rng, max_cap):
    """Cut every sequence's block list into consecutive tiles of random sizes
    (1..max_cap blocks, possibly empty for a sequence); returns a list of
    (tile_blocks [S, max_cap], tile_block_counts [S], token_counts [S])."""
    S, BS = case.num_seqs, case.block_size
    nblk = [(int(c) + BS - 1) // BS for c in case.context_lens]
    pos = [0] * S
    tiles = []
    while any(pos[s] < nblk[s] for s in range(S)):
        tb = np.full((S, max_cap), -1, dtype=np.int32)
        cnt = np.zeros(S, dtype=np.int32)
        tok = np.zeros(S, dtype=np.int32)
        for s in range(S):
            take = min(int(rng.integers(0, max_cap + 1)), nblk[s] - pos[s])
            tb[s, :take] = case.block_table[s, pos[s]:pos[s] + take]
            cnt[s] = take
            t0, t1 = pos[s] * BS, min((pos[s] + take) * BS, int(case.context_lens[s]))
            tok[s] = max(0, t1 - t0)
            pos[s] += take
        tiles.append((tb, cnt, tok))
    return tiles


def pin_decode_step(lib):
    """The stateful interface (AttnState, step_tile_ref, finalize_ref): folding
    any cut of the context into tiles, step after step from (-inf, 0, 0), then
    finalizing equals the direct softmax definition; m + ln l is the
    log-sum-exp of the scaled scores; a state that saw no token finalizes to 0."""
    rng = np.random.Generator(np.random.PCG64(31))
    c = _small_decode(31, [0, 1, 5, 16, 17, 40], Hq=4, Hkv=2, D=8, BS=4)
    ref = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale, lib=lib)
    for trial in range(3):
        st = O.decode_state_init(c.num_seqs, c.num_q_heads, c.head_dim)
        for tb, cnt, tok in split_into_tiles(c, rng, max_cap=3):
            O.paged_decode_step(st, c.q, c.k_pool, c.v_pool, tb, cnt, c.scale, token_counts=tok, lib=lib)
        out = O.paged_decode_finalize(st, lib=lib)
        _close(out, ref, 1e-12, f"step trial {trial}")
        # log-sum-exp of the scaled scores, from the gathered rows
        qf = bf16_to_f32(c.q).astype(np.float64)
        R = c.num_q_heads // c.num_kv_heads
        for s in range(c.num_seqs):
            ctx = int(c.context_lens[s])
            t = np.arange(ctx)
            kk = bf16_to_f32(c.k_pool[c.block_table[s, t // c.block_size], t % c.block_size]).astype(np.float64)
            for qh in range(c.num_q_heads):
                if ctx == 0:
                    assert st[0][s, qh] == -np.inf and st[1][s, qh] == 0.0 and np.all(out[s, qh] == 0.0)
                    continue
                x = c.scale * (kk[:, qh // R, :] @ qf[s, qh])
                lse = x.max() + math.log(math.fsum(np.exp(x - x.max())))
                _close(st[0][s, qh] + math.log(st[1][s, qh]), lse, 1e-12, f"step lse s={s} qh={qh}")
    # without token counts every token of the listed blocks counts
    st = O.decode_state_init(c.num_seqs, c.num_q_heads, c.head_dim)
    full = c.context_lens - c.context_lens % c.block_size  # whole blocks only
    nb = full // c.block_size
    O.paged_decode_step(st, c.q, c.k_pool, c.v_pool, c.block_table, nb, c.scale, lib=lib)
    ref_full = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, full.astype(np.int32), c.scale, lib=lib)
    _close(O.paged_decode_finalize(st, lib=lib), ref_full, 1e-12, "step over whole blocks")


def pin_decode_closed_forms(lib):
    """ctx 0 -> 0; ctx 1 -> v_0; V constant per kv head kh -> every q head of
    the group qh // (Hq/Hkv) == kh gets that constant."""
    c = _small_decode(23, [0, 1, 7, 12], Hq=8, Hkv=2, D=8, BS=4)
    out = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale, lib=lib)
    assert np.all(out[0] == 0.0)
    v0 = bf16_to_f32(c.v_pool[c.block_table[1, 0], 0]).astype(np.float64)  # [Hkv, D]
    for qh in range(8):
        _close(out[1, qh], v0[qh // 4], 1e-14, "ctx 1")
    vconst = np.zeros(c.v_pool.shape, np.float32)
    for kh in range(2):
        vconst[:, :, kh, :] = kh + 1.0
    out2 = O.paged_decode(c.q, c.k_pool, bf16_bits(vconst), c.block_table, c.context_lens, c.scale, lib=lib)
    for s in (1, 2, 3):
        for qh in range(8):
            _close(out2[s, qh], np.full(8, qh // 4 + 1.0), 1e-13, "gqa grouping")


def pin_decode_ignores_tail(lib):
    """Pool rows past the context length (inside the last block) and table
    entries past the last used block never reach the result."""
    c = _small_decode(24, [5, 6, 3], Hq=4, Hkv=2, D=8, BS=4, max_blocks=4)
    out = O.paged_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale, lib=lib)
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    bt = c.block_table.copy()
    for s in range(c.num_seqs):
        ctx = int(c.context_lens[s])
        last = c.block_table[s, (ctx - 1) // c.block_size]
        for slot in range(ctx % c.block_size or c.block_size, c.block_size):
            kp[last, slot] = 0x7FC0  # NaN
            vp[last, slot] = 0x7FC0
        bt[s, (ctx + c.block_size - 1) // c.block_size:] = 1 << 30
    out2 = O.paged_decode(c.q, kp, vp, bt, c.context_lens, c.scale, lib=lib)
    assert np.array_equal(out, out2)
    out3 = O.paged_decode_recurrent(c.q, kp, vp, bt, c.context_lens, c.scale, 2, lib=lib)
    _close(out3, out, 1e-12, "recurrence tail")


def pin_decode_gather(lib):
    """The gather hook equals numpy fancy indexing of the block table."""
    c = _small_decode(25, [5, 0, 9, 16], Hq=4, Hkv=2, D=8, BS=4, max_blocks=5)
    dense = O.paged_gather(c.k_pool, c.block_table, c.context_lens, lib=lib)
    for s in range(c.num_seqs):
        for t in range(c.max_blocks * c.block_size):
            if t < c.context_lens[s]:
                ref = c.k_pool[c.block_table[s, t // c.block_size], t % c.block_size]
                assert np.array_equal(dense[s, t], ref), (s, t)
            else:
                assert np.all(dense[s, t] == 0xFFFF)


# --- tile-map pins --------------------------------------------------------------------

def brute_force_tile_map(cu_q, H, BQ, grain=0):
    """All (b, qt, h) with qt < ceil(L_b / BQ), sorted by qt descending, then
    (with a grain) ceil(L_b / grain) descending, then b, then h."""
    items = []
    for b in range(len(cu_q) - 1):
        L = int(cu_q[b + 1]) - int(cu_q[b])
        n = -(-L // BQ)
        key = -(-L // grain) if grain else 0
        for qt in range(n):
            for h in range(H):
                items.append((-qt, -key, b, h))
    items.sort()
    return np.array([(b, -nqt, h) for nqt, _, b, h in items], np.int32).reshape(-1, 3)


def pin_tile_map(lib):
    rng = np.random.Generator(np.random.PCG64(26))
    for trial in range(40):
        B = int(rng.integers(0, 20))
        L = rng.integers(0, 700, size=B)
        cu = cu_from_lengths(L)
        H = int(rng.integers(1, 5))
        BQ = int(rng.choice([16, 64, 128]))
        grain = int(rng.choice([0, BQ // 4, BQ // 2, BQ]))
        got = O.varlen_tile_map(cu, H, BQ, grain, lib=lib)
        ref = brute_force_tile_map(cu, H, BQ, grain)
        assert np.array_equal(got, ref), (trial, B, H, BQ, grain)
    # a hand-checked case: lengths 5, 130, 64, 200 with BQ = 128, grain 64:
    # level 1 holds tiles of b = 1 (key 3) and b = 3 (key 4): b = 3 first;
    # level 0: keys 1, 3, 1, 4 -> b = 3, 1, 0, 2
    got = O.varlen_tile_map(cu_from_lengths([5, 130, 64, 200]), 1, 128, 64, lib=lib)
    assert got.tolist() == [[3, 1, 0], [1, 1, 0], [3, 0, 0], [1, 0, 0], [0, 0, 0], [2, 0, 0]]


ALL_PINS = [
    pin_bruteforce_tiny,
    pin_golden_plan_examples,
    pin_constant_values,
    pin_single_key,
    pin_zero_query_uniform,
    pin_packed_equals_per_sequence,
    pin_key_permutation,
    pin_sequence_isolation_and_order,
    pin_scale_homogeneity,
    pin_sampled_rows_match_full,
    pin_gqa_prefill,
    pin_paged_prefill,
    pin_backward,
    pin_backward_given_out,
    pin_decode_direct_equals_recurrence,
    pin_decode_equals_varlen_single_query,
    pin_decode_step,
    pin_decode_closed_forms,
    pin_decode_ignores_tail,
    pin_decode_gather,
    pin_tile_map,
]
