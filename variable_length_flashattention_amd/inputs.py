"""Seeded synthetic workloads (inputs only; none of the attention arithmetic).

Every floating-point tensor is drawn as float32 N(0, 1) from
``numpy.random.Generator(PCG64(seed))`` and rounded once to bf16
(round-to-nearest-even).  The same bf16 bit patterns (``numpy.uint16``) go to
the GPU library and to the CPU oracle.  Draw order: lengths, then q, k, v for
the packed forward pass; context lengths, K pool, V pool, block permutation,
then q for the paged decode.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, mult: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    b = bf16_bits(x)
    if mult != 1.0:  # a power-of-two multiple is exact in bf16
        b = bf16_bits(bf16_to_f32(b) * np.float32(mult))
    return b


@dataclass
class VarlenCase:
    """Packed forward-pass inputs; q [Tq,H,D], k/v [Tk,H,D] as bf16 bits."""
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray
    scale: float
    causal: bool
    seed: int
    recipe: str = ""

    @property
    def batch(self) -> int:
        return len(self.cu_q) - 1

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def max_seqlen_q(self) -> int:
        return int(np.max(np.diff(self.cu_q))) if self.batch else 0

    def with_causal(self, causal: bool) -> "VarlenCase":
        return VarlenCase(self.name, self.q, self.k, self.v, self.cu_q, self.cu_k, self.scale, causal,
                          self.seed, self.recipe)


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def varlen_case(name, lengths_q, lengths_k, num_heads, head_dim, seed, causal, q_mult=1.0,
                scale=None, rng=None, recipe="", num_kv_heads=None) -> VarlenCase:
    """k and v carry num_kv_heads heads (default: num_heads); grouped-query
    cases use num_kv_heads < num_heads."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    cu_q, cu_k = cu_from_lengths(lengths_q), cu_from_lengths(lengths_k)
    hkv = num_heads if num_kv_heads is None else num_kv_heads
    q = normal_bf16(rng, (int(cu_q[-1]), num_heads, head_dim), q_mult)
    k = normal_bf16(rng, (int(cu_k[-1]), hkv, head_dim))
    v = normal_bf16(rng, (int(cu_k[-1]), hkv, head_dim))
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return VarlenCase(name, q, k, v, cu_q, cu_k, float(scale), bool(causal), seed, recipe)


# --- the five synthetic workloads --------------------------------------------

def tiny(causal: bool, seed: int = 1001) -> VarlenCase:
    """3 packed sequences {1, 17, 64}, 2 heads, head_dim 64, scale 1/8."""
    return varlen_case("tiny", [1, 17, 64], [1, 17, 64], 2, 64, seed, causal,
                       recipe="lengths {1,17,64}; H=2; D=64; N(0,1) bf16")


def mixed(seed: int = 2001, causal: bool = True) -> VarlenCase:
    """16 sequences, lengths uniform in [1, 2048] (q = k), 32 heads, head_dim 128."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(1, 2049, size=16)
    return varlen_case("mixed", lengths, lengths, 32, 128, seed, causal, rng=rng,
                       recipe="16 lengths U[1,2048] (q=k); H=32; D=128; N(0,1) bf16; causal")


def mixed_gqa(seed: int = 2001, causal: bool = True) -> VarlenCase:
    """The mixed workload's lengths (seed 2001) with grouped-query K/V: 32 query
    heads over 8 kv heads, head_dim 128."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(1, 2049, size=16)
    return varlen_case("mixed_gqa", lengths, lengths, 32, 128, seed, causal, rng=rng, num_kv_heads=8,
                       recipe="16 lengths U[1,2048] (q=k); H=32, Hkv=8; D=128; N(0,1) bf16; causal")


def skewed(seed: int = 3001, causal: bool = True) -> VarlenCase:
    """q lengths {8192,1024,128,7}, k lengths {8192,3072,128,519}, 16 heads, head_dim 128."""
    return varlen_case("skewed", [8192, 1024, 128, 7], [8192, 3072, 128, 519], 16, 128, seed, causal,
                       recipe="Lq {8192,1024,128,7}, Lk {8192,3072,128,519}; H=16; D=128; bottom-right causal")


def many_short(head_dim: int, causal: bool, seed: int | None = None) -> VarlenCase:
    """1024 sequences, lengths uniform in [1, 128], 8 heads, q scaled by 4."""
    seed = seed if seed is not None else (4064 if head_dim == 64 else 4256 if head_dim == 256 else 4000 + head_dim)
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(1, 129, size=1024)
    return varlen_case(f"many_short_d{head_dim}", lengths, lengths, 8, head_dim, seed, causal, q_mult=4.0,
                       rng=rng, recipe=f"1024 lengths U[1,128]; H=8; D={head_dim}; q x4; N(0,1) bf16")


@dataclass
class PagedPrefillCase:
    """Forward-pass inputs with paged keys and values (chunked prefill):
    q [Tq,H,D] packed by cu_q; k_pool/v_pool [NB,BS,Hkv,D]; sequence b has
    seqlens_k[b] keys in pool blocks block_table[b, :ceil(Lk/BS)].  ``dense``
    is the same data as a packed VarlenCase (k/v [Tk,Hkv,D] by cu_k)."""
    name: str
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    cu_q: np.ndarray
    seqlens_k: np.ndarray
    block_table: np.ndarray
    scale: float
    causal: bool
    seed: int
    dense: VarlenCase
    recipe: str = ""

    @property
    def batch(self) -> int:
        return len(self.cu_q) - 1

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def num_kv_heads(self) -> int:
        return self.k_pool.shape[2]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def block_size(self) -> int:
        return self.k_pool.shape[1]

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    @property
    def max_seqlen_q(self) -> int:
        return int(np.max(np.diff(self.cu_q))) if self.batch else 0


POOL_FILL = 0x7FC0  # bf16 NaN in pool slots past a sequence's last key


def paged_prefill_case(name, lengths_q, lengths_k, num_heads, head_dim, block_size, seed, causal,
                       num_kv_heads=None, q_mult=1.0, scale=None, max_blocks=None, spare_blocks=0,
                       recipe="") -> PagedPrefillCase:
    """Draws exactly what varlen_case draws (lengths, q, k, v), then a seeded
    permutation of the pool blocks: sequence b's blocks are handed out in
    order from the permutation.  Pool slots past the last key of a sequence,
    and ``spare_blocks`` unused blocks, hold NaN, so a read of them shows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dense = varlen_case(name, lengths_q, lengths_k, num_heads, head_dim, seed, causal, q_mult=q_mult, scale=scale,
                        rng=rng, recipe=recipe, num_kv_heads=num_kv_heads)
    lk = np.asarray(lengths_k, dtype=np.int64)
    nblk = (lk + block_size - 1) // block_size
    NB = int(nblk.sum()) + spare_blocks
    perm = rng.permutation(max(NB, 1)).astype(np.int32)
    if max_blocks is None:
        max_blocks = int(max(1, nblk.max() if len(nblk) else 1))
    hkv = dense.num_kv_heads
    k_pool = np.full((max(NB, 1), block_size, hkv, head_dim), POOL_FILL, dtype=np.uint16)
    v_pool = np.full_like(k_pool, POOL_FILL)
    bt = np.full((len(lk), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
        j = np.arange(int(lk[b]))
        k0 = int(dense.cu_k[b])
        k_pool[bt[b, j // block_size], j % block_size] = dense.k[k0:k0 + len(j)]
        v_pool[bt[b, j // block_size], j % block_size] = dense.v[k0:k0 + len(j)]
    return PagedPrefillCase(name, dense.q, k_pool, v_pool, dense.cu_q, lk.astype(np.int32), bt, dense.scale,
                            bool(causal), seed, dense, recipe)


def chunked_paged(block_size: int = 16, seed: int = 3001, causal: bool = True) -> PagedPrefillCase:
    """The skewed/chunked shape (q lengths {8192,1024,128,7}, k lengths
    {8192,3072,128,519}, 16 heads, head_dim 128, bottom-right causal) with K/V
    in a paged pool of ``block_size``-token blocks."""
    return paged_prefill_case(f"chunked_paged_bs{block_size}", [8192, 1024, 128, 7], [8192, 3072, 128, 519], 16,
                              128, block_size, seed, causal,
                              recipe=f"Lq {{8192,1024,128,7}}, Lk {{8192,3072,128,519}}; H=16; D=128; "
                                     f"K/V in {block_size}-token pool blocks, permuted table; bottom-right causal")


@dataclass
class DecodeCase:
    """Paged GQA decode inputs (bf16 bits + int32 tables)."""
    name: str
    q: np.ndarray             # [S, Hq, D]
    k_pool: np.ndarray        # [NB, BS, Hkv, D]
    v_pool: np.ndarray        # [NB, BS, Hkv, D]
    block_table: np.ndarray   # [S, max_blocks] int32, -1 = unused
    context_lens: np.ndarray  # [S] int32
    scale: float
    seed: int
    recipe: str = ""

    @property
    def num_seqs(self): return self.q.shape[0]
    @property
    def num_q_heads(self): return self.q.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def block_size(self): return self.k_pool.shape[1]
    @property
    def num_kv_heads(self): return self.k_pool.shape[2]
    @property
    def max_blocks(self): return self.block_table.shape[1]


def decode_case(name, context_lens, num_q_heads, num_kv_heads, head_dim, block_size, seed,
                max_blocks=None, rng=None, scale=None, recipe="") -> DecodeCase:
    """Pool of NB = sum ceil(ctx/BS) blocks; the block table is a seeded
    permutation of all pool blocks handed out in sequence order; unused
    entries are -1."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(context_lens, dtype=np.int64)
    nblk = (ctx + block_size - 1) // block_size
    NB = int(nblk.sum())
    if max_blocks is None:
        max_blocks = int(max(1, nblk.max() if len(nblk) else 1))
    k_pool = normal_bf16(rng, (max(NB, 1), block_size, num_kv_heads, head_dim))
    v_pool = normal_bf16(rng, (max(NB, 1), block_size, num_kv_heads, head_dim))
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((len(ctx), max_blocks), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(nblk):
        bt[s, :n] = perm[off:off + n]
        off += n
    q = normal_bf16(rng, (len(ctx), num_q_heads, head_dim))
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeCase(name, q, k_pool, v_pool, bt, ctx.astype(np.int32), float(scale), seed, recipe)


def paged_decode(seed: int = 5001) -> DecodeCase:
    """64 sequences, one query each, 32 q heads / 8 kv heads, head_dim 128,
    16-token blocks, context lengths uniform in [1, 8192]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(1, 8193, size=64)
    return decode_case("paged_decode", ctx, 32, 8, 128, 16, seed, max_blocks=8192 // 16, rng=rng,
                       recipe="64 seqs; ctx U[1,8192]; Hq=32, Hkv=8; D=128; BS=16; permuted block table")


# --- algorithmic work counts (measurement, not the method) -------------------

def causal_pairs(Lq: int, Lk: int) -> int:
    """Number of (query, key) pairs with j <= i + Lk - Lq, 0 <= j < Lk."""
    total = 0
    off = Lk - Lq
    # rows with i + off + 1 in [1, Lk]: visible count min(Lk, i + off + 1)
    for i in range(Lq):
        total += min(Lk, max(0, i + off + 1))
    return total


def varlen_pairs(case: VarlenCase) -> int:
    lq = np.diff(case.cu_q).astype(np.int64)
    lk = np.diff(case.cu_k).astype(np.int64)
    if not case.causal:
        return int(np.sum(lq * lk))
    return int(sum(causal_pairs(int(a), int(b)) for a, b in zip(lq, lk)))


def varlen_flops(case: VarlenCase) -> int:
    """4 * D * H * (visible pairs): the two contractions QK^T and PV."""
    return 4 * case.head_dim * case.num_heads * varlen_pairs(case)


def varlen_bytes(case: VarlenCase) -> int:
    """Compulsory HBM bytes: read q, k, v once; write out and lse; read cu_seqlens."""
    H, Hkv, D = case.num_heads, case.num_kv_heads, case.head_dim
    Tq, Tk = int(case.cu_q[-1]), int(case.cu_k[-1])
    return 2 * D * (2 * H * Tq + 2 * Hkv * Tk) + 4 * Tq * H + 8 * (case.batch + 1)


def decode_bytes(case: DecodeCase) -> int:
    """Compulsory bytes: the visible K and V rows, q, out, the used block-table
    entries and the context lengths."""
    ctx = case.context_lens.astype(np.int64)
    nblk = (ctx + case.block_size - 1) // case.block_size
    kv = int(ctx.sum()) * case.num_kv_heads * case.head_dim * 2 * 2
    qo = 2 * case.num_seqs * case.num_q_heads * case.head_dim * 2
    return kv + qo + 4 * int(nblk.sum()) + 4 * case.num_seqs


def decode_flops(case: DecodeCase) -> int:
    return 4 * case.head_dim * case.num_q_heads * int(case.context_lens.astype(np.int64).sum())
