"""GPU parity of the backward pass (dq, dk, dv) against the fp64 oracle.

The GPU backward takes the GPU forward's out and lse, as a training step
would; the oracle recomputes everything in double from q, k, v and dout.
Tolerance on the bf16 gradients: |d - ref| <= BWD_ATOL + BWD_RTOL * |ref|.
The relative part covers the bf16 rounding of the stored gradient (2^-9
relative) plus the bf16 rounding of P and dS as MMA operands, whose errors
add up over the rows of a long sequence in proportion to the gradient's own
size.  The absolute part covers the row term dsum_i = dO_i . out_i, which
the backward forms from the forward's stored bf16 out: its rounding (and
the forward's own error) shifts every dS_ij of the row by P_ij * dsum error,
most where a row has only a few keys and P is large (tests/
test_backward_bound.py shows on the CPU that the bf16 rounding of out alone
moves the exact gradient past 2e-2 on 2000 sequences of 0-6 keys).  The
decomposition is pinned here too: fed the oracle's own forward (out rounded
to bf16, lse to fp32), the GPU backward must match the oracle's chain rule
with the row term from that same bf16 out within the tighter
ROW_TERM_ATOL + BWD_RTOL * |ref|."""
import numpy as np
import pytest
import torch

import oracle as O
import variable_length_flashattention_amd as rra
from gpu_helpers import dev_bf16, dev_i32, host_f64, say
from variable_length_flashattention_amd import inputs as I

pytestmark = pytest.mark.gpu

BWD_ATOL = 3e-2
BWD_RTOL = 1e-2
ROW_TERM_ATOL = 2e-2


def run_bwd(c, dout_bits, causal):
    """GPU forward then backward; gradients pre-filled with NaN so unwritten
    rows show.  Returns (dq, dk, dv) as float64."""
    q, k, v = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v)
    cu_q, cu_k = dev_i32(c.cu_q), dev_i32(c.cu_k)
    dout = dev_bf16(dout_bits)
    Hkv = c.num_kv_heads
    max_k = int(np.max(np.diff(c.cu_k))) if c.batch else 0
    say(f"  launch forward+backward case={c.name} seed={c.seed} Tq={q.shape[0]} Tk={k.shape[0]} H={c.num_heads} "
        f"Hkv={Hkv} D={c.head_dim} B={c.batch} causal={causal}")
    out, lse = rra.varlen_attn_fwd(q, k, v, cu_q, cu_k, c.max_seqlen_q, c.scale, causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for t in (dq, dk, dv):
        t.view(torch.int16).fill_(0x7FC0)
    rra.varlen_attn_bwd(q, k, v, out, lse, dout, cu_q, cu_k, c.max_seqlen_q, max_k, c.scale, causal, dq=dq, dk=dk,
                        dv=dv)
    torch.cuda.synchronize()
    return host_f64(dq), host_f64(dk), host_f64(dv)


def run_bwd_given_forward(c, dout_bits, causal, out_bits, lse):
    """GPU backward only, on a given forward result (out bf16 bits, lse
    float32).  Returns (dq, dk, dv) as float64."""
    q, k, v = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v)
    cu_q, cu_k = dev_i32(c.cu_q), dev_i32(c.cu_k)
    max_k = int(np.max(np.diff(c.cu_k))) if c.batch else 0
    say(f"  launch backward on the oracle's forward case={c.name} seed={c.seed} Tq={q.shape[0]} Tk={k.shape[0]} "
        f"H={c.num_heads} Hkv={c.num_kv_heads} D={c.head_dim} B={c.batch} causal={causal}")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for t in (dq, dk, dv):
        t.view(torch.int16).fill_(0x7FC0)
    rra.varlen_attn_bwd(q, k, v, dev_bf16(out_bits), torch.from_numpy(lse).cuda(), dev_bf16(dout_bits), cu_q, cu_k,
                        c.max_seqlen_q, max_k, c.scale, causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return host_f64(dq), host_f64(dk), host_f64(dv)


def compare_grads(got, ref, what, atol=BWD_ATOL):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert g.shape == r.shape, (what, name)
        assert np.all(np.isfinite(g)), f"{what}: {name} has non-finite or unwritten entries"
        err = np.abs(g - r)
        bound = atol + BWD_RTOL * np.abs(r)
        worst = float(np.max(err / bound)) if err.size else 0.0
        say(f"  {what} {name}: max|d|={float(err.max()) if err.size else 0.0:.3e} "
            f"max|ref|={float(np.abs(r).max()) if r.size else 0.0:.2f} worst/bound={worst:.3f}")
        assert worst <= 1.0, f"{what}: {name} off by {worst:.3f} x the bound"


def dout_for(c, seed):
    return I.normal_bf16(np.random.Generator(np.random.PCG64(seed)), c.q.shape)


CASES = [
    # name, Lq, Lk, H, Hkv, D
    ("tiny", [1, 17, 64], [1, 17, 64], 2, 2, 64),
    ("ragged_d128", [300, 129, 5], [300, 129, 5], 4, 4, 128),
    ("k_longer", [100, 33], [333, 200], 2, 2, 128),     # chunk: bottom-right rows
    ("k_shorter", [200, 64], [70, 1], 2, 2, 128),       # rows without visible keys under causal
    ("empty_seqs", [0, 40, 20, 0], [30, 0, 45, 0], 2, 2, 128),
    ("gqa_4to1", [150, 260], [150, 260], 8, 2, 128),
    ("d256", [140, 33], [140, 300], 2, 1, 256),
    ("d64_many", list(range(1, 40, 3)), list(range(1, 40, 3)), 4, 2, 64),
    ("long_d64", [3000, 7], [3000, 700], 2, 1, 64),      # 94 query tiles, 24 key blocks
    # more sequences than the LDS work tables hold (both kernels decode items from global memory)
    ("many_seqs_global", np.random.Generator(np.random.PCG64(63)).integers(0, 7, 2000).tolist(),
     np.random.Generator(np.random.PCG64(64)).integers(0, 7, 2000).tolist(), 2, 1, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_cases(case, causal):
    name, lq, lk, H, Hkv, D = case
    c = I.varlen_case(name, lq, lk, H, D, seed=len(name) * 7 + sum(lq), causal=causal, num_kv_heads=Hkv)
    dout = dout_for(c, c.seed + 1)
    got = run_bwd(c, dout, causal)
    ref = O.varlen_attn_bwd(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal)
    compare_grads(got, ref, f"{name} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_row_term(case, causal):
    """The GPU backward fed the oracle's forward (out rounded once to bf16,
    lse to fp32) against the oracle's chain rule whose row term dout_i . out_i
    uses that same bf16 out: within ROW_TERM_ATOL + BWD_RTOL * |ref|."""
    name, lq, lk, H, Hkv, D = case
    c = I.varlen_case(name, lq, lk, H, D, seed=len(name) * 7 + sum(lq), causal=causal, num_kv_heads=Hkv)
    dout = dout_for(c, c.seed + 1)
    out, lse = O.varlen_attn(c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, causal)
    out_bits = I.bf16_bits(np.nan_to_num(out).astype(np.float32))
    lse32 = np.ascontiguousarray(np.nan_to_num(lse, nan=0.0, neginf=-np.inf).astype(np.float32))
    got = run_bwd_given_forward(c, dout, causal, out_bits, lse32)
    ref = O.varlen_attn_bwd(c.q, c.k, c.v, dout, c.cu_q, c.cu_k, c.scale, causal,
                            out=I.bf16_to_f32(out_bits).astype(np.float64))
    compare_grads(got, ref, f"{name} causal={causal} (row term from the bf16 out)", atol=ROW_TERM_ATOL)


def test_backward_deterministic():
    c = I.varlen_case("det", [500, 77], [500, 300], 4, 128, seed=9, causal=True, num_kv_heads=2)
    dout = dout_for(c, 10)
    a = run_bwd(c, dout, True)
    b = run_bwd(c, dout, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_mixed_full_size():
    """The mixed workload (16 sequences up to 2048, 32 heads, head_dim 128,
    causal) at its full launch: every gradient written and finite; the
    closed forms sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per (sequence,
    head); and exact parity on the three shortest sequences (sequences are
    independent, so the oracle runs on them alone) and on the longest."""
    c = I.mixed()
    dout = dout_for(c, 2002)
    dq, dk, dv = run_bwd(c, dout, True)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.all(np.isfinite(g)), f"{name} has non-finite or unwritten entries"
    g = I.bf16_to_f32(dout).astype(np.float64)
    worst_k = worst_v = 0.0
    for b in range(c.batch):
        s, e = int(c.cu_k[b]), int(c.cu_k[b + 1])
        sk = dk[s:e].sum(axis=0)
        scale_k = np.abs(dk[s:e]).sum(axis=0) + 1.0
        worst_k = max(worst_k, float(np.max(np.abs(sk) / scale_k)))
        sv, want = dv[s:e].sum(axis=0), g[s:e].sum(axis=0)  # q = k lengths: every row sees a key
        worst_v = max(worst_v, float(np.max(np.abs(sv - want) / (np.abs(dv[s:e]).sum(axis=0) + 1.0))))
    say(f"  mixed: sum dK relative {worst_k:.2e}, sum dV - sum dO relative {worst_v:.2e}")
    assert worst_k <= 2e-2 and worst_v <= 2e-2
    lens = np.diff(c.cu_q)
    order = np.argsort(lens, kind="stable")
    pick = list(order[:3]) + [order[-1]]
    for b in pick:
        qs, qe, ks, ke = int(c.cu_q[b]), int(c.cu_q[b + 1]), int(c.cu_k[b]), int(c.cu_k[b + 1])
        ref = O.varlen_attn_bwd(c.q[qs:qe], c.k[ks:ke], c.v[ks:ke], dout[qs:qe], [0, qe - qs], [0, ke - ks], c.scale,
                                True)
        compare_grads((dq[qs:qe], dk[ks:ke], dv[ks:ke]), ref, f"mixed sequence {b} (length {qe - qs})")
