"""ctypes front end of ``liboracle.so`` (the fp64 CPU oracle).

Test infrastructure only.  Inputs are bf16 bit patterns (``numpy.uint16``)
exactly as they are handed to the GPU; outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain C99, -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", *extra_flags,
           "-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
    i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_varlen_attn.argtypes = [u16p, u16p, u16p, i32p, i32p, i32, i32, i32, f64, i32, f64p, f64p, i32]
    lib.oracle_varlen_attn.restype = ctypes.c_int
    lib.oracle_varlen_attn_rows.argtypes = [u16p, u16p, u16p, i32p, i32p, i32, i32, i32, f64, i32,
                                            i32p, i64, f64p, f64p, i32]
    lib.oracle_varlen_attn_rows.restype = ctypes.c_int
    lib.oracle_varlen_attn_gqa.argtypes = [u16p, u16p, u16p, i32p, i32p, i32, i32, i32, i32, f64, i32, f64p, f64p,
                                           i32]
    lib.oracle_varlen_attn_gqa.restype = ctypes.c_int
    lib.oracle_varlen_attn_rows_gqa.argtypes = [u16p, u16p, u16p, i32p, i32p, i32, i32, i32, i32, f64, i32,
                                                i32p, i64, f64p, f64p, i32]
    lib.oracle_varlen_attn_rows_gqa.restype = ctypes.c_int
    lib.oracle_varlen_attn_paged.argtypes = [u16p, u16p, u16p, i32p, i32p, i32p, i32, i32, i32, i32, i32, i32,
                                             f64, i32, ctypes.c_void_p, i64, f64p, f64p, i32]
    lib.oracle_varlen_attn_paged.restype = ctypes.c_int
    lib.oracle_varlen_attn_bwd.argtypes = [u16p, u16p, u16p, u16p, i32p, i32p, i32, i32, i32, i32, f64, i32, f64p,
                                           f64p, f64p, i32]
    lib.oracle_varlen_attn_bwd.restype = ctypes.c_int
    lib.oracle_varlen_attn_bwd_given_out.argtypes = [u16p, u16p, u16p, u16p, f64p, i32p, i32p, i32, i32, i32, i32,
                                                     f64, i32, f64p, f64p, f64p, i32]
    lib.oracle_varlen_attn_bwd_given_out.restype = ctypes.c_int
    lib.oracle_paged_decode.argtypes = [u16p, u16p, u16p, i32p, i32p, i32, i32, i32, i32, i32, i32, f64, f64p, i32]
    lib.oracle_paged_decode.restype = ctypes.c_int
    lib.oracle_paged_decode_recurrent.argtypes = [u16p, u16p, u16p, i32p, i32p, i32, i32, i32, i32, i32, i32,
                                                  f64, i32, f64p, i32]
    lib.oracle_paged_decode_recurrent.restype = ctypes.c_int
    lib.oracle_paged_decode_step.argtypes = [f64p, f64p, f64p, u16p, u16p, u16p, i32p, i32p, ctypes.c_void_p,
                                             i32, i32, i32, i32, i32, i32, f64, i32]
    lib.oracle_paged_decode_step.restype = ctypes.c_int
    lib.oracle_paged_decode_finalize.argtypes = [f64p, f64p, i32, i32, i32, f64p]
    lib.oracle_paged_decode_finalize.restype = ctypes.c_int
    lib.oracle_paged_gather.argtypes = [u16p, i32p, i32p, i32, i32, i32, i32, i32, u16p]
    lib.oracle_paged_gather.restype = ctypes.c_int
    lib.oracle_varlen_tile_map.argtypes = [i32p, i32, i32, i32, i32, i32p, i64]
    lib.oracle_varlen_tile_map.restype = ctypes.c_int64
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library.  ``path`` selects
    another build of it, e.g. a deliberately broken copy in a test."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def varlen_attn(q, k, v, cu_q, cu_k, scale, causal, nthreads=None, lib=None):
    """Full oracle: q [Tq,H,D], k/v [Tk,Hkv,D] uint16 bf16 bits (Hkv divides
    H; query head h reads kv head h // (H // Hkv)); returns (out [Tq,H,D]
    float64, lse [Tq,H] float64).  Rows of tokens outside every sequence stay
    NaN."""
    lib = lib or load()
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    Tq, H, D = q.shape
    Hkv = k.shape[1]
    out = np.full((Tq, H, D), np.nan)
    lse = np.full((Tq, H), np.nan)
    rc = lib.oracle_varlen_attn_gqa(q, k, v, cu_q, cu_k, len(cu_q) - 1, H, Hkv, D, float(scale),
                                    int(bool(causal)), out, lse, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_varlen_attn rejected its arguments")
    return out, lse


def varlen_attn_rows(q, k, v, cu_q, cu_k, scale, causal, rows, nthreads=None, lib=None):
    """Oracle for selected rows only; ``rows`` is an int array [n, 2] of
    (packed query token, head).  Returns (out [n, D], lse [n])."""
    lib = lib or load()
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _c(rows, np.int32).reshape(-1, 2)
    D = q.shape[2]
    out = np.full((rows.shape[0], D), np.nan)
    lse = np.full((rows.shape[0],), np.nan)
    rc = lib.oracle_varlen_attn_rows_gqa(q, k, v, cu_q, cu_k, len(cu_q) - 1, q.shape[1], k.shape[1], D,
                                         float(scale), int(bool(causal)), rows, rows.shape[0], out, lse,
                                         nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_varlen_attn_rows rejected its arguments")
    return out, lse


def varlen_attn_paged(q, k_pool, v_pool, cu_q, seqlens_k, block_table, scale, causal, rows=None, nthreads=None,
                      lib=None):
    """Oracle with paged keys and values (chunked prefill): q [Tq,H,D]; pools
    [NB,BS,Hkv,D]; seqlens_k [B] keys per sequence; block_table [B, maxb].
    Returns (out [Tq,H,D], lse [Tq,H]), or with ``rows`` ([n, 2] of (packed
    query token, head)) (out [n, D], lse [n])."""
    lib = lib or load()
    q, k_pool, v_pool = _c(q, np.uint16), _c(k_pool, np.uint16), _c(v_pool, np.uint16)
    cu_q, lk, bt = _c(cu_q, np.int32), _c(seqlens_k, np.int32), _c(block_table, np.int32)
    Tq, H, D = q.shape
    _, BS, Hkv, _ = k_pool.shape
    if rows is None:
        out, lse, rp, n = np.full((Tq, H, D), np.nan), np.full((Tq, H), np.nan), None, 0
    else:
        rows = _c(rows, np.int32).reshape(-1, 2)
        out, lse = np.full((rows.shape[0], D), np.nan), np.full((rows.shape[0],), np.nan)
        rp, n = rows.ctypes.data_as(ctypes.c_void_p), rows.shape[0]
    rc = lib.oracle_varlen_attn_paged(q, k_pool, v_pool, cu_q, lk, bt, len(cu_q) - 1, H, Hkv, D, BS, bt.shape[1],
                                      float(scale), int(bool(causal)), rp, n, out, lse,
                                      nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_varlen_attn_paged rejected its arguments")
    return out, lse


def varlen_attn_bwd(q, k, v, dout, cu_q, cu_k, scale, causal, out=None, nthreads=None, lib=None):
    """Gradients of sum(out * dout) of the packed forward pass: q, dout
    [Tq,H,D], k, v [Tk,Hkv,D] bf16 bits.  Returns (dq [Tq,H,D], dk [Tk,Hkv,D],
    dv [Tk,Hkv,D]) float64; rows outside every sequence stay NaN.  With
    ``out`` (float64 [Tq,H,D], e.g. a rounded forward output) the softmax
    Jacobian's row term is dout_i . out_i from those rows instead of its
    exact value."""
    lib = lib or load()
    q, k, v, dout = (_c(x, np.uint16) for x in (q, k, v, dout))
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    Tq, H, D = q.shape
    Tk, Hkv, _ = k.shape
    dq = np.full((Tq, H, D), np.nan)
    dk = np.full((Tk, Hkv, D), np.nan)
    dv = np.full((Tk, Hkv, D), np.nan)
    if out is None:
        rc = lib.oracle_varlen_attn_bwd(q, k, v, dout, cu_q, cu_k, len(cu_q) - 1, H, Hkv, D, float(scale),
                                        int(bool(causal)), dq, dk, dv, nthreads or default_threads())
    else:
        out = _c(out, np.float64)
        if out.shape != (Tq, H, D):
            raise ValueError("out must be float64 [Tq, H, D]")
        rc = lib.oracle_varlen_attn_bwd_given_out(q, k, v, dout, out, cu_q, cu_k, len(cu_q) - 1, H, Hkv, D,
                                                  float(scale), int(bool(causal)), dq, dk, dv,
                                                  nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_varlen_attn_bwd rejected its arguments")
    return dq, dk, dv


def _decode_args(q, k_pool, v_pool, block_table, context_lens):
    q = _c(q, np.uint16)
    k_pool, v_pool = _c(k_pool, np.uint16), _c(v_pool, np.uint16)
    block_table, context_lens = _c(block_table, np.int32), _c(context_lens, np.int32)
    S, Hq, D = q.shape
    _, BS, Hkv, _ = k_pool.shape
    return q, k_pool, v_pool, block_table, context_lens, S, Hq, Hkv, D, BS, block_table.shape[1]


def paged_decode(q, k_pool, v_pool, block_table, context_lens, scale, nthreads=None, lib=None):
    """Direct definition.  q [S,Hq,D]; pools [NB,BS,Hkv,D]; block_table
    [S, max_blocks] int32; context_lens [S] int32.  Returns out [S,Hq,D] f64."""
    lib = lib or load()
    q, k_pool, v_pool, bt, cl, S, Hq, Hkv, D, BS, MB = _decode_args(q, k_pool, v_pool, block_table, context_lens)
    out = np.full((S, Hq, D), np.nan)
    rc = lib.oracle_paged_decode(q, k_pool, v_pool, bt, cl, S, Hq, Hkv, D, BS, MB, float(scale), out,
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_paged_decode rejected its arguments")
    return out


def paged_decode_recurrent(q, k_pool, v_pool, block_table, context_lens, scale, tile_capacity=1,
                           nthreads=None, lib=None):
    """The decode page's per-token (m, l, o) recurrence with the state carried
    across tiles of ``tile_capacity`` blocks, then the l > 0 guarded finalize."""
    lib = lib or load()
    q, k_pool, v_pool, bt, cl, S, Hq, Hkv, D, BS, MB = _decode_args(q, k_pool, v_pool, block_table, context_lens)
    out = np.full((S, Hq, D), np.nan)
    rc = lib.oracle_paged_decode_recurrent(q, k_pool, v_pool, bt, cl, S, Hq, Hkv, D, BS, MB, float(scale),
                                           int(tile_capacity), out, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_paged_decode_recurrent rejected its arguments")
    return out


def decode_state_init(num_seqs, num_q_heads, head_dim):
    """The decode page's initial AttnState: m = -inf, l = 0, o = 0 (fp64 here)."""
    return (np.full((num_seqs, num_q_heads), -np.inf), np.zeros((num_seqs, num_q_heads)),
            np.zeros((num_seqs, num_q_heads, head_dim)))


def paged_decode_step(state, q, k_pool, v_pool, tile_blocks, tile_block_counts, scale, token_counts=None,
                      nthreads=None, lib=None):
    """One step_tile_ref: fold the listed blocks (tile_blocks [S, cap] int32,
    tile_block_counts [S]; token_counts [S] cuts the tile) into the state
    (m, l, o), in place."""
    lib = lib or load()
    m, l, o = state
    q, k_pool, v_pool = _c(q, np.uint16), _c(k_pool, np.uint16), _c(v_pool, np.uint16)
    tb, tc = _c(tile_blocks, np.int32), _c(tile_block_counts, np.int32)
    S, Hq, D = q.shape
    _, BS, Hkv, _ = k_pool.shape
    tok = None if token_counts is None else _c(token_counts, np.int32)
    rc = lib.oracle_paged_decode_step(m, l, o, q, k_pool, v_pool, tb, tc,
                                      None if tok is None else tok.ctypes.data_as(ctypes.c_void_p),
                                      S, Hq, Hkv, D, BS, tb.shape[1], float(scale), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_paged_decode_step rejected its arguments")
    return state


def paged_decode_finalize(state, lib=None):
    """finalize_ref: out = o / l, 0 where l == 0."""
    lib = lib or load()
    m, l, o = state
    S, Hq, D = o.shape
    out = np.full((S, Hq, D), np.nan)
    if lib.oracle_paged_decode_finalize(l, o, S, Hq, D, out) != 0:
        raise ValueError("oracle_paged_decode_finalize rejected its arguments")
    return out


def paged_gather(pool, block_table, context_lens, fill=0xFFFF, lib=None):
    """Dense [S, max_blocks*BS, Hkv, D] copy of each sequence's visible pool
    rows (bf16 bits); rows past the context length hold ``fill``."""
    lib = lib or load()
    pool = _c(pool, np.uint16)
    bt, cl = _c(block_table, np.int32), _c(context_lens, np.int32)
    _, BS, Hkv, D = pool.shape
    S, MB = bt.shape
    dense = np.full((S, MB * BS, Hkv, D), fill, dtype=np.uint16)
    rc = lib.oracle_paged_gather(pool, bt, cl, S, Hkv, D, BS, MB, dense)
    if rc != 0:
        raise ValueError("oracle_paged_gather rejected its arguments")
    return dense


def varlen_tile_map(cu_q, num_heads, block_q, sort_grain=0, lib=None):
    """Canonical work list of the tiled forward pass: int32 [n_items, 3] of
    (sequence, query tile, head), most expensive tile level first; inside a
    level, sequences in ascending b (sort_grain 0) or in descending
    ceil(L / sort_grain), ties in ascending b."""
    lib = lib or load()
    cu_q = _c(cu_q, np.int32)
    B = len(cu_q) - 1
    cap = 0
    for b in range(B):
        cap += -(-(int(cu_q[b + 1]) - int(cu_q[b])) // block_q)
    cap = max(cap * num_heads, 1)
    items = np.zeros((cap, 3), dtype=np.int32)
    n = lib.oracle_varlen_tile_map(cu_q, B, num_heads, block_q, int(sort_grain), items, cap)
    if n < 0:
        raise ValueError("oracle_varlen_tile_map rejected its arguments")
    return items[:n]
