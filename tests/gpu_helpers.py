"""Helpers for the GPU tests: move bf16 bit arrays to the device, run the
library through its C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np

from variable_length_flashattention_amd.inputs import bf16_to_f32

OUT_TOL = 2e-2   # max |out - oracle| (bf16 output)
LSE_TOL = 1e-3   # max |lse - oracle| (fp32)


def say(msg):
    print(msg, flush=True)


def dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def dev_i32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host_f64(t):
    import torch
    return bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def run_varlen(case, causal=None, poison=True):
    """Launch rra_varlen_attn_fwd on the case; out/lse pre-filled with NaN so
    unwritten rows show.  Returns (out f64 [Tq,H,D], lse f64 [Tq,H])."""
    import torch
    import variable_length_flashattention_amd as rra
    causal = case.causal if causal is None else causal
    q, k, v = dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v)
    cu_q, cu_k = dev_i32(case.cu_q), dev_i32(case.cu_k)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if poison:
        out.view(torch.int16).fill_(0x7FC0)  # bf16 NaN
        lse.fill_(float("nan"))
    say(f"  launch rra_varlen_attn_fwd case={case.name} seed={case.seed} Tq={q.shape[0]} Tk={k.shape[0]} "
        f"H={q.shape[1]} Hkv={k.shape[1]} D={q.shape[2]} B={case.batch} causal={causal}")
    if k.shape[1] == q.shape[1]:
        rra.rra_varlen_attn_fwd(q, k, v, out, lse, cu_q, cu_k, case.max_seqlen_q, case.batch, q.shape[1],
                                q.shape[2], case.scale, causal)
    else:
        rra.rra_varlen_attn_fwd_gqa(q, k, v, out, lse, cu_q, cu_k, case.max_seqlen_q, case.batch, q.shape[1],
                                    k.shape[1], q.shape[2], case.scale, causal)
    torch.cuda.synchronize()
    return host_f64(out), lse.cpu().numpy().astype(np.float64)


def compare(out, lse, ref_out, ref_lse, what):
    """Element-wise comparison at the stated tolerances; -inf lse must match
    exactly and the corresponding out row must be exactly 0."""
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ninf), f"{what}: -inf lse pattern differs"
    assert np.all(out[ninf] == 0.0), f"{what}: rows without visible keys must be 0"
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert np.all(np.isfinite(lse[~ninf])), f"{what}: non-finite lse"
    eo = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    el = float(np.max(np.abs(lse[~ninf] - ref_lse[~ninf]))) if np.any(~ninf) else 0.0
    say(f"  {what}: max|dout|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= OUT_TOL, f"{what}: max|dout| {eo}"
    assert el <= LSE_TOL, f"{what}: max|dlse| {el}"
    return eo, el


SCHED_INTS = 3584  # LDS ints of the kernels' work-list tables
SORT_SCRATCH = 256
SORT_MIN_BATCH = 64


def device_sort_grain(B, maxq, bq, D):
    """The grain by which the forward's work list orders sequences inside a
    level (0: ascending b): its key tile, for batches of at least 64
    sequences whose tables fit in LDS with the permutation and have at most
    64 distinct sort keys."""
    grain = 64 if D <= 128 else 32
    levels = -(-maxq // bq)
    cached = 2 * (B + 1) + 2 * (levels + 1) <= SCHED_INTS
    keys = levels * (bq // grain)
    fits = 3 * (B + 1) + 2 * (levels + 1) + SORT_SCRATCH <= SCHED_INTS
    return grain if cached and B >= SORT_MIN_BATCH and 1 <= keys <= 64 and fits else 0
