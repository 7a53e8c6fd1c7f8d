"""ctypes binding of librra.so (argument marshalling only).

Every function named ``rra_*`` forwards to the C entry point of the same name
declared in ``include/rra.h``.  Tensor arguments may be torch tensors (their
``data_ptr()`` is passed) or integers (raw device addresses).  ``stream``
defaults to torch's current stream on the current device.  A non-zero status
raises :class:`RraError`.  There is no fallback: if the library is missing the
first call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "librra.so"
_lib = None

RRA_OK = 0
RRA_ERR_INVALID_ARG = 1
RRA_ERR_UNSUPPORTED = 2
RRA_ERR_WORKSPACE = 3
RRA_ERR_HIP = 4
RRA_ERR_SCRATCH = 5


class RraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status} ({rra_status_string(status)})")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load librra.so from the package directory (built in-tree)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()'). "
            "There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.rra_status_string.argtypes = [i32]
    lib.rra_status_string.restype = ctypes.c_char_p
    lib.rra_varlen_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
    lib.rra_varlen_attn_fwd.restype = i32
    lib.rra_varlen_attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.rra_varlen_attn_fwd_gqa.restype = i32
    lib.rra_varlen_attn_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                              f32, i32, vp]
    lib.rra_varlen_attn_fwd_paged.restype = i32
    lib.rra_varlen_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                        f32, i32, vp, sz, vp]
    lib.rra_varlen_attn_bwd.restype = i32
    lib.rra_varlen_attn_bwd_workspace_bytes.argtypes = [i32, i32]
    lib.rra_varlen_attn_bwd_workspace_bytes.restype = sz
    lib.rra_varlen_block_q.argtypes = [i32, i32]
    lib.rra_varlen_block_q.restype = i32
    lib.rra_paged_decode_attn.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.rra_paged_decode_attn.restype = i32
    lib.rra_paged_decode_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.rra_paged_decode_attn_noalloc.restype = i32
    lib.rra_paged_decode_scratch_bytes.argtypes = []
    lib.rra_paged_decode_scratch_bytes.restype = sz
    lib.rra_paged_decode_state_init.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    lib.rra_paged_decode_state_init.restype = i32
    lib.rra_paged_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp,
                                          sz, vp]
    lib.rra_paged_decode_step.restype = i32
    lib.rra_paged_decode_finalize.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    lib.rra_paged_decode_finalize.restype = i32
    lib.rra_paged_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.rra_paged_decode_workspace_bytes.restype = sz
    lib.rra_pack_rows.argtypes = [vp, vp, vp, i32, i32, i64, vp]
    lib.rra_pack_rows.restype = i32
    lib.rra_unpack_rows.argtypes = [vp, vp, vp, i32, i32, i64, vp]
    lib.rra_unpack_rows.restype = i32
    lib.rra_debug_varlen_tile_map.argtypes = [vp, i32, i32, i32, i32, vp, i64, ctypes.POINTER(i64), vp]
    lib.rra_debug_varlen_tile_map.restype = i32
    lib.rra_debug_paged_gather.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.rra_debug_paged_gather.restype = i32
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != RRA_OK:
        raise RraError(fn, status)


def rra_status_string(status: int) -> str:
    return load_library().rra_status_string(int(status)).decode()


def rra_varlen_block_q(head_dim: int, max_seqlen_q: int) -> int:
    return int(load_library().rra_varlen_block_q(int(head_dim), int(max_seqlen_q)))


def rra_varlen_attn_fwd(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, batch, num_heads,
                        head_dim, softmax_scale, causal, stream=None):
    st = load_library().rra_varlen_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        int(max_seqlen_q), int(batch), int(num_heads), int(head_dim), float(softmax_scale), int(bool(causal)),
        _stream(stream))
    _check("rra_varlen_attn_fwd", st)


def rra_varlen_attn_fwd_gqa(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, batch, num_heads,
                            num_kv_heads, head_dim, softmax_scale, causal, stream=None):
    st = load_library().rra_varlen_attn_fwd_gqa(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        int(max_seqlen_q), int(batch), int(num_heads), int(num_kv_heads), int(head_dim), float(softmax_scale),
        int(bool(causal)), _stream(stream))
    _check("rra_varlen_attn_fwd_gqa", st)


def rra_varlen_attn_fwd_paged(q, k_pool, v_pool, out, lse, cu_seqlens_q, seqlens_k, block_table, max_seqlen_q, batch,
                              num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, softmax_scale, causal,
                              stream=None):
    st = load_library().rra_varlen_attn_fwd_paged(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q), _ptr(seqlens_k),
        _ptr(block_table), int(max_seqlen_q), int(batch), int(num_heads), int(num_kv_heads), int(head_dim),
        int(block_size), int(max_blocks_per_seq), float(softmax_scale), int(bool(causal)), _stream(stream))
    _check("rra_varlen_attn_fwd_paged", st)


def rra_varlen_attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, total_q, max_seqlen_q,
                        max_seqlen_k, batch, num_heads, num_kv_heads, head_dim, softmax_scale, causal, workspace,
                        workspace_bytes, stream=None):
    st = load_library().rra_varlen_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(total_q), int(max_seqlen_q), int(max_seqlen_k), int(batch),
        int(num_heads), int(num_kv_heads), int(head_dim), float(softmax_scale), int(bool(causal)), _ptr(workspace),
        int(workspace_bytes), _stream(stream))
    _check("rra_varlen_attn_bwd", st)


def rra_varlen_attn_bwd_workspace_bytes(total_q, num_heads) -> int:
    return int(load_library().rra_varlen_attn_bwd_workspace_bytes(int(total_q), int(num_heads)))


def rra_paged_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim) -> int:
    return int(load_library().rra_paged_decode_workspace_bytes(int(num_seqs), int(num_q_heads), int(num_kv_heads),
                                                               int(head_dim)))


def rra_paged_decode_attn(q, k_pool, v_pool, block_table, context_lens, out, num_seqs, num_q_heads, num_kv_heads,
                          head_dim, block_size, max_blocks_per_seq, softmax_scale, workspace, workspace_bytes,
                          stream=None):
    st = load_library().rra_paged_decode_attn(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(context_lens), _ptr(out), int(num_seqs),
        int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size), int(max_blocks_per_seq),
        float(softmax_scale), _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("rra_paged_decode_attn", st)


def rra_paged_decode_attn_noalloc(q, k_pool, v_pool, block_table, context_lens, out, num_seqs, num_q_heads,
                                  num_kv_heads, head_dim, block_size, max_blocks_per_seq, softmax_scale,
                                  stream=None):
    st = load_library().rra_paged_decode_attn_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(context_lens), _ptr(out), int(num_seqs),
        int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size), int(max_blocks_per_seq),
        float(softmax_scale), _stream(stream))
    _check("rra_paged_decode_attn_noalloc", st)


def rra_paged_decode_scratch_bytes() -> int:
    return int(load_library().rra_paged_decode_scratch_bytes())

def rra_paged_decode_state_init(state_m, state_l, state_o, num_seqs, num_q_heads, head_dim, stream=None):
    st = load_library().rra_paged_decode_state_init(_ptr(state_m), _ptr(state_l), _ptr(state_o), int(num_seqs),
                                                    int(num_q_heads), int(head_dim), _stream(stream))
    _check("rra_paged_decode_state_init", st)


def rra_paged_decode_step(state_m, state_l, state_o, q, k_pool, v_pool, tile_blocks, tile_block_counts,
                          tile_token_counts, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, tile_capacity,
                          softmax_scale, workspace, workspace_bytes, stream=None):
    st = load_library().rra_paged_decode_step(
        _ptr(state_m), _ptr(state_l), _ptr(state_o), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(tile_blocks),
        _ptr(tile_block_counts), _ptr(tile_token_counts), int(num_seqs), int(num_q_heads), int(num_kv_heads),
        int(head_dim), int(block_size), int(tile_capacity), float(softmax_scale), _ptr(workspace),
        int(workspace_bytes), _stream(stream))
    _check("rra_paged_decode_step", st)


def rra_paged_decode_finalize(state_l, state_o, out, num_seqs, num_q_heads, head_dim, stream=None):
    st = load_library().rra_paged_decode_finalize(_ptr(state_l), _ptr(state_o), _ptr(out), int(num_seqs),
                                                  int(num_q_heads), int(head_dim), _stream(stream))
    _check("rra_paged_decode_finalize", st)


def rra_debug_varlen_tile_map(cu_seqlens_q, batch, num_heads, max_seqlen_q, head_dim, items_out, capacity,
                              stream=None) -> int:
    count = ctypes.c_int64(0)
    st = load_library().rra_debug_varlen_tile_map(
        _ptr(cu_seqlens_q), int(batch), int(num_heads), int(max_seqlen_q), int(head_dim), _ptr(items_out),
        int(capacity), ctypes.byref(count), _stream(stream))
    _check("rra_debug_varlen_tile_map", st)
    return int(count.value)


def rra_pack_rows(padded, packed, cu_seqlens, batch, max_seqlen, row_bytes, stream=None):
    st = load_library().rra_pack_rows(_ptr(padded), _ptr(packed), _ptr(cu_seqlens), int(batch), int(max_seqlen),
                                      int(row_bytes), _stream(stream))
    _check("rra_pack_rows", st)


def rra_unpack_rows(packed, padded, cu_seqlens, batch, max_seqlen, row_bytes, stream=None):
    st = load_library().rra_unpack_rows(_ptr(packed), _ptr(padded), _ptr(cu_seqlens), int(batch), int(max_seqlen),
                                        int(row_bytes), _stream(stream))
    _check("rra_unpack_rows", st)


def rra_debug_paged_gather(k_pool, v_pool, block_table, context_lens, k_dense, v_dense, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, max_blocks_per_seq, workspace, workspace_bytes,
                           stream=None):
    st = load_library().rra_debug_paged_gather(
        _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(context_lens), _ptr(k_dense), _ptr(v_dense),
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_blocks_per_seq), _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("rra_debug_paged_gather", st)


# --- allocating conveniences (torch allocates; the library computes) ----------

def varlen_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, softmax_scale, causal, out=None,
                    lse=None, stream=None):
    """q [Tq,H,D], k/v [Tk,Hkv,D] bf16 CUDA tensors (Hkv divides H; Hkv < H
    is grouped-query attention); cu_seqlens int32 CUDA tensors.  Returns
    (out bf16 [Tq,H,D], lse fp32 [Tq,H])."""
    import torch
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    for t in (q, k, v, cu_seqlens_q, cu_seqlens_k):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("all tensors must be contiguous device tensors")
    if q.dim() != 3 or k.shape != v.shape or k.dim() != 3 or q.shape[2] != k.shape[2] or k.shape[1] == 0 \
            or q.shape[1] % k.shape[1] != 0:
        raise ValueError("q must be [Tq,H,D] and k, v [Tk,Hkv,D] with Hkv dividing H")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    Tq, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=q.device)
    rra_varlen_attn_fwd_gqa(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, cu_seqlens_q.numel() - 1,
                            H, k.shape[1], D, softmax_scale, causal, stream)
    return out, lse


def varlen_attn_bwd(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale,
                    causal, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the packed forward pass for the upstream
    gradient dout; q/out/dout [Tq,H,D], k/v [Tk,Hkv,D] bf16, lse [Tq,H] fp32
    (the forward's out and lse), cu_seqlens int32 (all device tensors)."""
    import torch
    for t in (q, k, v, out, dout):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v, out, dout must be contiguous bfloat16 device tensors")
    if q.shape != out.shape or q.shape != dout.shape or k.shape != v.shape or q.shape[1] % k.shape[1] != 0:
        raise ValueError("bad shapes for the backward pass")
    Tq, H, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = rra_varlen_attn_bwd_workspace_bytes(Tq, H)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    rra_varlen_attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, Tq, max_seqlen_q,
                        max_seqlen_k, cu_seqlens_q.numel() - 1, H, k.shape[1], D, softmax_scale, causal, workspace,
                        workspace.numel() * workspace.element_size(), stream)
    return dq, dk, dv


def pack_padded(padded, cu_seqlens, total=None, stream=None):
    """padded [B, Lmax, ...] device tensor, cu_seqlens int32 [B+1] device
    tensor -> packed [total, ...] (total = cu_seqlens[-1], read on the host
    when not given)."""
    import torch
    if not padded.is_contiguous() or not padded.is_cuda:
        raise ValueError("padded must be a contiguous device tensor")
    B, Lmax = padded.shape[:2]
    if cu_seqlens.numel() != B + 1:
        raise ValueError("cu_seqlens must have batch + 1 entries")
    total = int(cu_seqlens[-1].item()) if total is None else int(total)
    packed = torch.empty((total,) + tuple(padded.shape[2:]), dtype=padded.dtype, device=padded.device)
    row_bytes = padded[0, 0].numel() * padded.element_size() if Lmax and B else 4
    rra_pack_rows(padded, packed, cu_seqlens, B, Lmax, row_bytes, stream)
    return packed


def unpack_to_padded(packed, cu_seqlens, max_seqlen, stream=None):
    """packed [total, ...] device tensor -> padded [B, max_seqlen, ...]
    (rows past each sequence's length are zero)."""
    import torch
    if not packed.is_contiguous() or not packed.is_cuda:
        raise ValueError("packed must be a contiguous device tensor")
    B = cu_seqlens.numel() - 1
    padded = torch.empty((B, int(max_seqlen)) + tuple(packed.shape[1:]), dtype=packed.dtype, device=packed.device)
    row_bytes = max(1, int(np.prod(packed.shape[1:], dtype=np.int64))) * packed.element_size()
    rra_unpack_rows(packed, padded, cu_seqlens, B, int(max_seqlen), row_bytes, stream)
    return padded


def varlen_attn_fwd_paged(q, k_pool, v_pool, cu_seqlens_q, seqlens_k, block_table, max_seqlen_q, softmax_scale,
                          causal, out=None, lse=None, stream=None):
    """q [Tq,H,D] bf16 packed by cu_seqlens_q [B+1]; k_pool/v_pool
    [NB,BS,Hkv,D] bf16; seqlens_k [B] and block_table [B,maxb] int32 (all
    device tensors).  Returns (out bf16 [Tq,H,D], lse fp32 [Tq,H])."""
    import torch
    _decode_checks(q, k_pool, v_pool, (cu_seqlens_q, seqlens_k, block_table))
    if q.shape[1] % k_pool.shape[2] != 0 or block_table.dim() != 2 or seqlens_k.numel() != cu_seqlens_q.numel() - 1 \
            or block_table.shape[0] != seqlens_k.numel():
        raise ValueError("bad shapes for a paged forward pass")
    Tq, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=q.device)
    rra_varlen_attn_fwd_paged(q, k_pool, v_pool, out, lse, cu_seqlens_q, seqlens_k, block_table, max_seqlen_q,
                              seqlens_k.numel(), H, k_pool.shape[2], D, k_pool.shape[1], block_table.shape[1],
                              softmax_scale, causal, stream)
    return out, lse


def paged_decode_attn(q, k_pool, v_pool, block_table, context_lens, softmax_scale, out=None, workspace=None,
                      stream=None):
    """q [S,Hq,D] bf16; pools [NB,BS,Hkv,D] bf16; block_table [S,maxb] int32;
    context_lens [S] int32 (all device tensors).  Returns out bf16 [S,Hq,D]."""
    import torch
    _decode_checks(q, k_pool, v_pool, (block_table, context_lens))
    S, Hq, D = q.shape
    _, BS, Hkv, _ = k_pool.shape
    MB = block_table.shape[1]
    if out is None:
        out = torch.empty_like(q)
    need = rra_paged_decode_workspace_bytes(S, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rra_paged_decode_attn(q, k_pool, v_pool, block_table, context_lens, out, S, Hq, Hkv, D, BS, MB, softmax_scale,
                          workspace, workspace.numel() * workspace.element_size(), stream)
    return out


def _decode_checks(q, k_pool, v_pool, index_tensors):
    import torch
    if q.dtype != torch.bfloat16 or k_pool.dtype != torch.bfloat16 or v_pool.dtype != torch.bfloat16:
        raise TypeError("q, k_pool, v_pool must be bfloat16")
    for t in index_tensors:
        if t is not None and t.dtype != torch.int32:
            raise TypeError("block tables and counts must be int32")
    for t in (q, k_pool, v_pool) + tuple(index_tensors):
        if t is not None and (not t.is_contiguous() or not t.is_cuda):
            raise ValueError("all tensors must be contiguous device tensors")
    if q.dim() != 3 or k_pool.dim() != 4 or k_pool.shape != v_pool.shape or q.shape[2] != k_pool.shape[3]:
        raise ValueError("q must be [S,Hq,D] and the pools [NB,BS,Hkv,D]")


def decode_state_init(num_seqs, num_q_heads, head_dim, device, stream=None):
    """A fresh decode state (m, l, o): fp32 device tensors [S,Hq], [S,Hq],
    [S,Hq,D] holding m = -inf, l = 0, o = 0."""
    import torch
    m = torch.empty((num_seqs, num_q_heads), dtype=torch.float32, device=device)
    l = torch.empty_like(m)
    o = torch.empty((num_seqs, num_q_heads, head_dim), dtype=torch.float32, device=device)
    rra_paged_decode_state_init(m, l, o, num_seqs, num_q_heads, head_dim, stream)
    return m, l, o


def paged_decode_step(state, q, k_pool, v_pool, tile_blocks, tile_block_counts, softmax_scale, token_counts=None,
                      workspace=None, stream=None):
    """Fold one tile of paged K/V into state = (m, l, o), in place.
    tile_blocks [S, cap] int32, tile_block_counts [S] int32, token_counts
    [S] int32 or None (device tensors)."""
    import torch
    m, l, o = state
    _decode_checks(q, k_pool, v_pool, (tile_blocks, tile_block_counts, token_counts))
    S, Hq, D = q.shape
    _, BS, Hkv, _ = k_pool.shape
    if m.shape != (S, Hq) or l.shape != (S, Hq) or o.shape != (S, Hq, D) or tile_blocks.dim() != 2:
        raise ValueError("state must be ([S,Hq], [S,Hq], [S,Hq,D]) and tile_blocks [S,cap]")
    need = rra_paged_decode_workspace_bytes(S, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rra_paged_decode_step(m, l, o, q, k_pool, v_pool, tile_blocks, tile_block_counts, token_counts, S, Hq, Hkv, D,
                          BS, tile_blocks.shape[1], softmax_scale, workspace,
                          workspace.numel() * workspace.element_size(), stream)
    return state


def paged_decode_finalize(state, out=None, stream=None):
    """out = o / l (0 where l == 0), bf16 [S,Hq,D]."""
    import torch
    _, l, o = state
    S, Hq, D = o.shape
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=o.device)
    rra_paged_decode_finalize(l, o, out, S, Hq, D, stream)
    return out
