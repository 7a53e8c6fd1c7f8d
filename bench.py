"""Benchmark of the varlen attention forward (and the paged decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

A step is one rra_varlen_attn_fwd call on the mixed-length workload
(16 sequences with lengths uniform in [1, 2048] from seed 2001, 32 heads,
head_dim 128, bf16, causal), inputs resident in HBM.  The value is that
workload's algorithmic TFLOP/s: 4 * head_dim * heads * (visible query/key
pairs), causal pairs counted exactly.  The paged GQA decode (64 sequences,
context lengths uniform in [1, 8192], Hq=32/Hkv=8, head_dim 128, 16-token
blocks) is timed the same way and reported in GB/s of compulsory HBM bytes.
The other synthetic workloads are timed once each for context.  Per-launch
durations come from HIP events recorded on the stream the kernels run on.
Rank 0 prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quick", action="store_true", help="skip the context workloads")
    p.add_argument("--only", default="", choices=["", "mixed", "decode", "decode_steps", "skewed", "many_short_d64",
                                                  "many_short_d256", "chunked_paged_bs16", "backward"],
                   help="time only this workload (for profiling runs)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="first run one plain device-to-device copy of BYTES bytes (a known-size reference "
                        "for the HBM byte counters)")
    return p.parse_args()


VARLEN_SOURCES = ("varlen_fwd.hip", "tile_map.h", "rra_device.h", "rra_internal.h", "rra_api.hip")
DECODE_SOURCES = ("paged_decode.hip", "rra_device.h", "rra_internal.h", "rra_api.hip")
BWD_SOURCES = ("varlen_bwd.hip", "tile_map.h", "rra_device.h", "rra_internal.h", "rra_api.hip")


def kernel_source_hash(files=None):
    """sha256 prefix over the kernel sources (all of csrc/, or the named files)
    and the compiler flags they are built with."""
    from variable_length_flashattention_amd import build as B
    h = hashlib.sha256(" ".join(B.FLAGS).encode())
    csrc = os.path.join(ROOT, "variable_length_flashattention_amd", "csrc")
    for f in sorted(files if files is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


SETTLE_S = 0.5  # seconds of untimed back-to-back launches before the warm-up steps
COLD_COPIES = 4  # input copies cycled by the HBM-bound many-short runs (4 x 273 MB > the 256 MiB MALL)
DECODE_COPIES = 2  # the decode's pools are 1.07 GB each: two copies keep every launch cold


def time_launches(torch, fn, steps, warmup, settle_s=SETTLE_S):
    """Settle, warm up, then time exactly `steps` back-to-back launches: wall
    time bracketed by synchronize, and one HIP event pair around the whole
    timed region on the current stream (the stream the library launches on).
    The settle phase runs the same launches untimed for `settle_s` seconds:
    the GPU's clocks ramp up over the first ~0.1 s of sustained work (the
    mixed forward runs ~25 % slower in its first 50 launches than after 200),
    and the figure wanted is the sustained rate.
    Returns (wall seconds, event seconds per launch)."""
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) * 1e-3 / steps


class VarlenRun:
    """rra_varlen_attn_fwd (or _gqa) on a case.  With copies > 1 the inputs
    and outputs exist that many times at different addresses and each launch
    uses the next copy, so that no launch finds its inputs in the caches (the
    256 MiB MALL included) from the launch before: a cold measurement."""
    def __init__(self, torch, case, copies=1):
        import variable_length_flashattention_amd as rra
        self.rra, self.case = rra, case
        self.sets = []
        for _ in range(copies):
            q, k, v = dev_bf16(torch, case.q), dev_bf16(torch, case.k), dev_bf16(torch, case.v)
            out = torch.empty_like(q)
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
            self.sets.append((q, k, v, out, lse))
        self.q, self.k, self.v, self.out, self.lse = self.sets[0]
        self.cu_q = torch.from_numpy(case.cu_q).cuda()
        self.cu_k = torch.from_numpy(case.cu_k).cuda()
        self.i = 0

    def __call__(self):
        c = self.case
        q, k, v, out, lse = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        if c.num_kv_heads == c.num_heads:
            self.rra.rra_varlen_attn_fwd(q, k, v, out, lse, self.cu_q, self.cu_k, c.max_seqlen_q, c.batch,
                                         c.num_heads, c.head_dim, c.scale, c.causal)
        else:
            self.rra.rra_varlen_attn_fwd_gqa(q, k, v, out, lse, self.cu_q, self.cu_k, c.max_seqlen_q, c.batch,
                                             c.num_heads, c.num_kv_heads, c.head_dim, c.scale, c.causal)


class BwdRun:
    """The backward pass (rra_varlen_attn_bwd) on the forward's out and lse
    for a fixed upstream gradient."""
    def __init__(self, torch, case, seed=2002):
        import variable_length_flashattention_amd as rra
        self.rra, self.case = rra, case
        self.q, self.k, self.v = dev_bf16(torch, case.q), dev_bf16(torch, case.k), dev_bf16(torch, case.v)
        self.cu_q = torch.from_numpy(case.cu_q).cuda()
        self.cu_k = torch.from_numpy(case.cu_k).cuda()
        self.dout = dev_bf16(torch, I_normal(case.q.shape, seed))
        self.out, self.lse = rra.varlen_attn_fwd(self.q, self.k, self.v, self.cu_q, self.cu_k, case.max_seqlen_q,
                                                 case.scale, case.causal)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.tq = int(case.cu_q[-1])
        self.max_k = int(np.max(np.diff(case.cu_k)))
        need = rra.rra_varlen_attn_bwd_workspace_bytes(self.tq, case.num_heads)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def __call__(self):
        c = self.case
        self.rra.rra_varlen_attn_bwd(self.q, self.k, self.v, self.out, self.lse, self.dout, self.dq, self.dk,
                                     self.dv, self.cu_q, self.cu_k, self.tq, c.max_seqlen_q, self.max_k, c.batch,
                                     c.num_heads, c.num_kv_heads, c.head_dim, c.scale, c.causal, self.ws,
                                     self.ws.numel())


def I_normal(shape, seed):
    from variable_length_flashattention_amd import inputs as I
    return I.normal_bf16(np.random.Generator(np.random.PCG64(seed)), shape)


class PagedRun:
    """The forward pass with paged K/V (rra_varlen_attn_fwd_paged)."""
    def __init__(self, torch, case):
        import variable_length_flashattention_amd as rra
        self.rra, self.case = rra, case
        self.q = dev_bf16(torch, case.q)
        self.kp, self.vp = dev_bf16(torch, case.k_pool), dev_bf16(torch, case.v_pool)
        self.cu_q = torch.from_numpy(case.cu_q).cuda()
        self.lk = torch.from_numpy(case.seqlens_k).cuda()
        self.bt = torch.from_numpy(case.block_table).cuda()
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")

    def __call__(self):
        c = self.case
        self.rra.rra_varlen_attn_fwd_paged(self.q, self.kp, self.vp, self.out, self.lse, self.cu_q, self.lk, self.bt,
                                           c.max_seqlen_q, c.batch, c.num_heads, c.num_kv_heads, c.head_dim,
                                           c.block_size, c.max_blocks, c.scale, c.causal)


class DecodeRun:
    """rra_paged_decode_attn on a case; with copies > 1 each launch uses the
    next copy of q, the pools, out and the workspace (cold, as VarlenRun)."""
    def __init__(self, torch, case, copies=1):
        import variable_length_flashattention_amd as rra
        self.rra, self.case = rra, case
        self.bt = torch.from_numpy(case.block_table).cuda()
        self.cl = torch.from_numpy(case.context_lens).cuda()
        need = rra.rra_paged_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                                    case.head_dim)
        self.sets = []
        for _ in range(copies):
            q = dev_bf16(torch, case.q)
            kp, vp = dev_bf16(torch, case.k_pool), dev_bf16(torch, case.v_pool)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            self.sets.append((q, kp, vp, torch.empty_like(q), ws))
        self.i = 0

    def __call__(self):
        c = self.case
        q, kp, vp, out, ws = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.rra.rra_paged_decode_attn(q, kp, vp, self.bt, self.cl, out, c.num_seqs, c.num_q_heads,
                                       c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks, c.scale, ws,
                                       ws.numel())


class DecodeStepsRun:
    """The stateful decode on the decode workload: state init, the context of
    every sequence folded in n_tiles consecutive tiles of blocks (one
    rra_paged_decode_step each), then finalize."""
    def __init__(self, torch, case, n_tiles=4, copies=1):
        import variable_length_flashattention_amd as rra
        self.rra, self.case = rra, case
        S, BS = case.num_seqs, case.block_size
        self.q = dev_bf16(torch, case.q)
        self.pools = [(dev_bf16(torch, case.k_pool), dev_bf16(torch, case.v_pool)) for _ in range(copies)]
        self.ip = 0
        nblk = (case.context_lens.astype(np.int64) + BS - 1) // BS
        cut = [np.minimum(nblk, (nblk * j + n_tiles - 1) // n_tiles) for j in range(n_tiles + 1)]
        self.cap = max(1, max(int((cut[j + 1] - cut[j]).max()) for j in range(n_tiles)))
        self.tiles = []
        for j in range(n_tiles):
            tb = np.full((S, self.cap), -1, dtype=np.int32)
            cnt = (cut[j + 1] - cut[j]).astype(np.int32)
            for s_ in range(S):
                tb[s_, :cnt[s_]] = case.block_table[s_, cut[j][s_]:cut[j + 1][s_]]
            tok = np.maximum(np.minimum(cut[j + 1] * BS, case.context_lens) - cut[j] * BS, 0).astype(np.int32)
            self.tiles.append(tuple(torch.from_numpy(x).cuda() for x in (tb, cnt, tok)))
        Hq, D = case.num_q_heads, case.head_dim
        self.m = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
        self.l = torch.empty_like(self.m)
        self.o = torch.empty((S, Hq, D), dtype=torch.float32, device="cuda")
        self.out = torch.empty_like(self.q)
        need = rra.rra_paged_decode_workspace_bytes(S, Hq, case.num_kv_heads, D)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def __call__(self):
        c, r = self.case, self.rra
        S, Hq, D = c.num_seqs, c.num_q_heads, c.head_dim
        kp, vp = self.pools[self.ip]
        self.ip = (self.ip + 1) % len(self.pools)
        r.rra_paged_decode_state_init(self.m, self.l, self.o, S, Hq, D)
        for tb, cnt, tok in self.tiles:
            r.rra_paged_decode_step(self.m, self.l, self.o, self.q, kp, vp, tb, cnt, tok, S, Hq,
                                    c.num_kv_heads, D, c.block_size, self.cap, c.scale, self.ws, self.ws.numel())
        r.rra_paged_decode_finalize(self.l, self.o, self.out, S, Hq, D)


def cpu_baseline(case, n_rows=655360, seed=7):
    """The fp64 oracle, as it stands, on a bounded random sample of the same
    workload's (token, head) rows; reported in the metric's unit."""
    import oracle as O
    rng = np.random.Generator(np.random.PCG64(seed))
    Tq = int(case.cu_q[-1])
    rows = np.stack([rng.integers(0, Tq, n_rows), rng.integers(0, case.num_heads, n_rows)], 1).astype(np.int32)
    b = np.searchsorted(case.cu_q, rows[:, 0], side="right") - 1
    i = rows[:, 0] - case.cu_q[b]
    Lq, Lk = np.diff(case.cu_q)[b], np.diff(case.cu_k)[b]
    vis = np.clip(i + Lk - Lq + 1, 0, Lk) if case.causal else Lk
    flops = 4.0 * case.head_dim * float(np.sum(vis))
    threads = O.default_threads()
    t0 = time.perf_counter()
    O.varlen_attn_rows(case.q, case.k, case.v, case.cu_q, case.cu_k, case.scale, case.causal, rows, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} random (token, head) rows of the mixed workload (seed {seed}); "
                      f"{flops / 1e9:.2f} GFLOP in {dt:.2f} s, fp64"}


# profiles/<record>_hbm_traffic.json for the context workloads that have one
TRAFFIC_RECORDS = {"skewed": "varlen_fwd_skewed", "chunked_paged_bs16": "varlen_fwd_paged_chunked_bs16",
                   "many_short_d64_causal": "varlen_fwd_many_short_d64",
                   "many_short_d256_causal": "varlen_fwd_many_short_d256"}


def load_traffic(name, src_hash):
    """HBM bytes per launch measured with rocprofv3 counters (scaled by a copy
    kernel calibration), if the record matches the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards across GPUs only on paper)", file=sys.stderr)
        sys.exit(2)
    import torch
    from variable_length_flashattention_amd import inputs as I
    import variable_length_flashattention_amd as rra
    rra.load_library()
    src_hash = kernel_source_hash()
    if args.copy_calibration:
        n = args.copy_calibration // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only and args.only != "mixed":
        case = {"decode": None, "decode_steps": "steps", "skewed": I.skewed(), "many_short_d64": I.many_short(64, True),
                "many_short_d256": I.many_short(256, True), "chunked_paged_bs16": "paged",
                "backward": "backward"}[args.only]
        if case == "backward":
            case = I.mixed()
            r = BwdRun(torch, case)
            nbytes, flops = 2 * I.varlen_bytes(case), int(2.5 * I.varlen_flops(case))
        elif case == "paged":
            case = I.chunked_paged(16)
            r = PagedRun(torch, case)
            nbytes, flops = I.varlen_bytes(case.dense), I.varlen_flops(case.dense)
        elif case is None or case == "steps":
            steps = case == "steps"
            case = I.paged_decode()
            r = (DecodeStepsRun if steps else DecodeRun)(torch, case, copies=DECODE_COPIES)
            nbytes, flops = I.decode_bytes(case), I.decode_flops(case)
        else:
            hbm_bound = args.only.startswith("many_short")
            r = VarlenRun(torch, case, copies=COLD_COPIES if hbm_bound else 1)
            nbytes, flops = I.varlen_bytes(case), I.varlen_flops(case)
        _, t = time_launches(torch, r, args.steps, args.warmup)
        print(json.dumps({"only": args.only, "avg_us": round(t * 1e6, 2), "TFLOP/s": round(flops / t / 1e12, 2),
                          "GB/s": round(nbytes / t / 1e9, 1), "kernel_source_hash": src_hash,
                          "varlen_source_hash": kernel_source_hash(VARLEN_SOURCES),
                          "decode_source_hash": kernel_source_hash(DECODE_SOURCES),
                          "bwd_source_hash": kernel_source_hash(BWD_SOURCES)}), flush=True)
        return

    mixed = I.mixed()
    flops = I.varlen_flops(mixed)
    run = VarlenRun(torch, mixed)
    wall, avg_launch = time_launches(torch, run, args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / avg_launch / 1e12
    lines = {
        "metric": "varlen attn fwd TFLOP/s + % bf16 MFMA peak; paged decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mixed-length varlen prefill: 16 sequences, lengths U[1,2048] (seed 2001), "
                               "q=k lengths, 32 heads, head_dim 128, bf16, causal",
                   "batch": mixed.batch, "tokens": int(mixed.cu_q[-1]), "num_heads": 32, "head_dim": 128,
                   "causal": True, "seed": 2001, "flops_per_step": flops, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic("varlen_fwd_mixed", kernel_source_hash(VARLEN_SOURCES)),
                     "kernel": "varlen_fwd_kernel<128, true, false, false>", "avg_launch_us": round(avg_launch * 1e6, 2),
                     "algorithmic_bytes": I.varlen_bytes(mixed)},
    }

    if args.only == "mixed":
        lines["kernel_source_hash"] = src_hash
        lines["varlen_source_hash"] = kernel_source_hash(VARLEN_SOURCES)
        print(json.dumps(lines), flush=True)
        return

    # paged decode (second row of the metric)
    dec = I.paged_decode()
    drun = DecodeRun(torch, dec, copies=DECODE_COPIES)
    _, d_avg = time_launches(torch, drun, args.steps, args.warmup)
    dbytes = I.decode_bytes(dec)
    lines["decode"] = {"workload": "paged GQA decode: 64 seqs, ctx U[1,8192] (seed 5001), Hq=32, Hkv=8, "
                                   "head_dim 128, 16-token blocks, permuted block table",
                       "GB/s": round(dbytes / d_avg / 1e9, 1), "frac_of_hbm_peak": round(dbytes / d_avg / 1e9 / PEAK_HBM_GBS, 4),
                       "avg_call_us": round(d_avg * 1e6, 2), "bytes_per_call": dbytes,
                       "traffic": load_traffic("paged_decode", kernel_source_hash(DECODE_SOURCES)),
                       "context_tokens": int(dec.context_lens.sum()),
                       "cold": True, "copies": DECODE_COPIES,
                       "note": "range-split + combine kernels per call (an offsets kernel too above 256 sequences); "
                               "consecutive launches use different copies of q and the pools (cold)"}
    del drun
    srun = DecodeStepsRun(torch, dec, copies=DECODE_COPIES)
    _, s_avg = time_launches(torch, srun, args.steps, args.warmup)
    lines["decode"]["stateful_4_steps"] = {
        "GB/s": round(dbytes / s_avg / 1e9, 1), "frac_of_hbm_peak": round(dbytes / s_avg / 1e9 / PEAK_HBM_GBS, 4),
        "avg_us": round(s_avg * 1e6, 2),
        "cold": True, "copies": DECODE_COPIES,
        "note": "state init + 4 rra_paged_decode_step calls (each context cut into 4 tiles of blocks) + finalize"}
    del srun
    torch.cuda.empty_cache()

    # backward of the mixed workload (5 matmuls' worth of algorithmic flops:
    # 2.5x the forward's)
    brun = BwdRun(torch, mixed)
    _, b_avg = time_launches(torch, brun, args.steps, args.warmup)
    lines["backward"] = {"workload": "backward of the mixed workload (dq, dk, dv from out, lse, dout)",
                         "TFLOP/s": round(2.5 * flops / b_avg / 1e12, 2),
                         "frac_mfma_peak": round(2.5 * flops / b_avg / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "avg_call_us": round(b_avg * 1e6, 2),
                         "traffic": load_traffic("varlen_bwd_mixed", kernel_source_hash(BWD_SOURCES)),
                         "note": "dq (+ dsum) and dk/dv kernels per call; flops = 2.5 x forward (S, dP, dV, dK, dQ)"}
    del brun
    torch.cuda.empty_cache()

    if not args.quick:
        ctx = {}
        for name, case, bound in [
            ("tiny_causal", I.tiny(True), "latency"), ("tiny_noncausal", I.tiny(False), "latency"),
            ("skewed", I.skewed(), "mfma"),
            ("chunked_paged_bs16", I.chunked_paged(16), "mfma"),
            ("chunked_paged_bs256", I.chunked_paged(256), "mfma"),
            ("mixed_gqa_32q_8kv", I.mixed_gqa(), "mfma"),
            ("many_short_d64_causal", I.many_short(64, True), "hbm"),
            ("many_short_d64_noncausal", I.many_short(64, False), "hbm"),
            ("many_short_d256_causal", I.many_short(256, True), "hbm"),
            ("many_short_d256_noncausal", I.many_short(256, False), "hbm"),
        ]:
            # HBM-bound workloads are timed cold (COLD_COPIES input copies in
            # rotation); the others warm, inputs reused from launch to launch
            cold = bound == "hbm"
            if isinstance(case, I.PagedPrefillCase):
                r = PagedRun(torch, case)
            else:
                r = VarlenRun(torch, case, copies=COLD_COPIES if cold else 1)
            _, t = time_launches(torch, r, 20, 3)
            dense = case.dense if isinstance(case, I.PagedPrefillCase) else case
            f, b = I.varlen_flops(dense), I.varlen_bytes(dense)
            ctx[name] = {"avg_us": round(t * 1e6, 2), "TFLOP/s": round(f / t / 1e12, 2),
                         "frac_mfma_peak": round(f / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "GB/s": round(b / t / 1e9, 1), "frac_hbm_peak": round(b / t / 1e9 / PEAK_HBM_GBS, 4),
                         "bound": bound, "cold": cold}
            if name in TRAFFIC_RECORDS:
                ctx[name]["traffic"] = load_traffic(TRAFFIC_RECORDS[name], kernel_source_hash(VARLEN_SOURCES))
            if cold:
                ctx[name]["copies"] = COLD_COPIES
            del r
            torch.cuda.empty_cache()
        lines["other_workloads"] = ctx

    if not args.no_cpu_baseline:
        lines["cpu_baseline"] = cpu_baseline(mixed)
    lines["kernel_source_hash"] = src_hash
    print(json.dumps(lines), flush=True)


if __name__ == "__main__":
    main()
