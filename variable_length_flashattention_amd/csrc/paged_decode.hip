// Paged-KV grouped-query decode attention for gfx950.
//
// Method: "spark_storage/attention_ref.rs" -- the decode state (m, l, o) in
// fp32 (AttnState), its update over the tokens of a list of pool blocks
// (step_tile_ref; the state is carried from one block list to the next), and
// the guarded finalize out = o / l, 0 when l == 0 (finalize_ref).  Here the
// context of each sequence is cut into splits of 256 tokens; one wave folds a
// split into a partial state for one kv head and its group of q heads, and a
// second kernel merges the partial states of a sequence and finalizes.
//
// Split kernel, per 16 tokens:
//   S^T[token][q head] = K . Q^T     (v_mfma_f32_16x16x32_bf16; K straight
//                                     from the pool into the A operand)
//   online softmax per q head (max/sum over 4 registers x 4 lane groups)
//   O^T[d][q head] += V^T . P^T      (v_mfma_f32_16x16x16_bf16; V staged in
//                                     wave-private LDS, read transposed)
// Only tokens t < context_lens[s] are read; the block table is never read at
// or past ceil(ctx / block_size).
#include "rra_device.h"
#include "rra_internal.h"

namespace rra {

constexpr int kSplit = kDecodeSplitTokens;

// Element offset of (token t, kv head kh) of a sequence whose block-table row
// is bt.  block_size = 1 << bs_shift.
__device__ __forceinline__ int64_t paged_token_offset(const int32_t *__restrict__ bt, int t, int bs_shift,
                                                      int num_kv_heads, int head_dim, int kh)
{
    const int64_t blk = bt[t >> bs_shift];
    const int64_t slot = t & ((1 << bs_shift) - 1);
    return ((blk << bs_shift) + slot) * num_kv_heads * head_dim + (int64_t)kh * head_dim;
}

// BIG: block_size >= 16, so each group of 16 tokens sits in one pool block
// and its block id is wave-uniform.
template <int D, bool BIG>
__global__ __launch_bounds__(256) void paged_decode_split_kernel(DecodeArgs a)
{
    constexpr int NKS = D / 32;   // k-steps of the QK^T MMA (32 d each)
    constexpr int NDC = D / 16;   // 16-wide d chunks of the output
    constexpr int NV = D / 32;    // 16-byte V pieces per lane per 16 tokens
    constexpr int VST = D + 16;   // LDS row stride of a staged V token
    __shared__ __attribute__((aligned(16))) uint16_t vbuf[4][2][16 * VST];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
    const int unit = blockIdx.y * 4 + wave;
    if (unit >= a.num_kv_heads * a.n_sub) return;  // no block-level barriers below
    const int kh = unit / a.n_sub, sub = unit % a.n_sub;
    const int ctx = a.context_lens[s];
    const int t_begin = split * kSplit;
    if (t_begin >= ctx) return;
    const int t_end = min(ctx, t_begin + kSplit);
    const int ratio = a.num_q_heads / a.num_kv_heads;
    const int qh0 = kh * ratio + 16 * sub;
    const int nq = min(16, ratio - 16 * sub);
    const int col = lane & 15, grp = lane >> 4;
    const bool q_ok = col < nq;
    const int Hkv = a.num_kv_heads;
    const int bs_shift = a.bs_shift;
    const float sl2 = a.scale_log2;
    const int32_t *bt = a.block_table + (int64_t)s * a.max_blocks;

    // Block-table entries covering this split, one per lane (lane j holds the
    // j-th block from the split's first block; 4 registers cover the 256
    // blocks a split spans at block_size 1).  Only blocks below
    // ceil(ctx / block_size) are read.
    const int blk0 = t_begin >> bs_shift;
    const int blk_end = ((t_end - 1) >> bs_shift) + 1;
    constexpr int NBT = BIG ? 1 : 4;
    int btr[NBT];
#pragma unroll
    for (int r = 0; r < NBT; r++) {
        const int bi = blk0 + lane + 64 * r;
        btr[r] = bi < blk_end ? bt[bi] : 0;
    }
    const int64_t row_elems = (int64_t)Hkv * D;  // elements per pool token row
    // Element offset of token t (t_begin <= t < t_end), kv head kh.
    auto token_offset = [&](int t) -> int64_t {
        const int rel = (t >> bs_shift) - blk0;
        int blk = __shfl(btr[0], rel & 63, 64);
        if (!BIG && rel >= 64) {
            const int b1 = __shfl(btr[NBT > 1 ? 1 : 0], rel & 63, 64), b2 = __shfl(btr[NBT > 2 ? 2 : 0], rel & 63, 64),
                      b3 = __shfl(btr[NBT > 3 ? 3 : 0], rel & 63, 64);
            blk = rel < 128 ? b1 : rel < 192 ? b2 : b3;
        }
        const int64_t slot = t & ((1 << bs_shift) - 1);
        return (((int64_t)blk << bs_shift) + slot) * row_elems + (int64_t)kh * D;
    };
    // BIG: base offset of group t0's block (uniform) plus the slot's row
    auto group_base = [&](int t0) -> int64_t {
        const int blk = __builtin_amdgcn_readlane(btr[0], (t0 >> bs_shift) - blk0);
        return ((int64_t)blk << bs_shift) * row_elems + (int64_t)kh * D;
    };

    // Q^T operand: lane holds Q[qh0 + col][32*ks + 8*grp .. +7]
    bf16x8 qf[NKS];
    {
        const uint16_t *qrow = a.q + ((int64_t)s * a.num_q_heads + qh0 + col) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (q_ok) x = load16(qrow + 32 * ks);
            qf[ks] = as_bf16x8(x);
        }
    }
    f32x4 o[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; dc++) o[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
    // m_ref: the max (per q head, common to all lanes of that column) the
    // accumulators are scaled to.  It is raised only when some score exceeds
    // it by more than 2^8 in probability, so most groups need no cross-lane
    // max.  l_part: this lane's share of the denominator (its 4 tokens per
    // group), summed across the lane groups once at the end.
    float m_ref = -INFINITY, l_part = 0.f;
    const float thresh = 8.f / sl2;  // raw-score headroom above m_ref

    // Loads of one group of 16 tokens: K straight into the MMA A operand
    // (lane: token t0 + col, d = 32*ks + 8*grp..), V rows for the LDS stage
    // (lane: token t0 + c/(D/8), 16-byte piece c%(D/8), c = lane + 64 i).
    // Tokens at or past t_end re-read token t_end-1: their scores are masked
    // and their probabilities are exactly 0, and the loads stay unconditional
    // (a conditional load followed by a merge makes the compiler wait for it
    // on the spot, which would defeat the prefetch).
    auto load_group = [&](int t0, u32x4 *kd, u32x4 *vd) {
        const int64_t gb = BIG ? group_base(t0) : 0;
        const int mask = (1 << bs_shift) - 1;
        const int tc = min(t0 + col, t_end - 1);
        const uint16_t *p = a.k_pool + (BIG ? gb + (int64_t)(tc & mask) * row_elems : token_offset(tc)) + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) kd[ks] = load16(p + 32 * ks);
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int c = lane + 64 * i;
            const int tvc = min(t0 + c / (D / 8), t_end - 1);
            const int64_t off = BIG ? gb + (int64_t)(tvc & mask) * row_elems : token_offset(tvc);
            vd[i] = load16(a.v_pool + off + (c % (D / 8)) * 8);
        }
    };

    // Fold one group of 16 tokens into the running state.
    auto process = [&](int t0, const u32x4 *kr, const u32x4 *vr, uint16_t *vb) {
        // stage this group's V rows in the wave's LDS (two buffers, so the
        // next group's stores never race this group's transposed reads; LDS
        // operations of one wave complete in order)
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int c = lane + 64 * i;
            *reinterpret_cast<u32x4 *>(vb + (c / (D / 8)) * VST + (c % (D / 8)) * 8) = vr[i];
        }
        // S^T = K Q^T (16 tokens x 16 q heads)
        f32x4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ks++)
            sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[ks]), qf[ks], sv, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; r++)
            if (t0 + 4 * grp + r >= t_end) sv[r] = -INFINITY;
        const float lmax = max3f(sv[0], sv[1], max3f(sv[2], sv[3], sv[3]));
        if (__builtin_amdgcn_ballot_w64(lmax > m_ref + thresh || (m_ref == -INFINITY && lmax > -INFINITY))) {
            float mx = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_ref - m_new) * sl2);
            l_part *= alpha;
#pragma unroll
            for (int dc = 0; dc < NDC; dc++) o[dc] *= alpha;
            m_ref = m_new;
        }
        const float mc = (m_ref == -INFINITY ? 0.f : m_ref) * sl2;
        const float p0 = fast_exp2(fmaf(sv[0], sl2, -mc)), p1 = fast_exp2(fmaf(sv[1], sl2, -mc));
        const float p2 = fast_exp2(fmaf(sv[2], sl2, -mc)), p3 = fast_exp2(fmaf(sv[3], sl2, -mc));
        const uint32_t u0 = pack_bf16x2(p0, p1), u1 = pack_bf16x2(p2, p3);
        l_part += (p0 + p1) + (p2 + p3);
        const i16x4 pb = __builtin_bit_cast(i16x4, u32x2{u0, u1});
        const uint16_t *vrow = vb + (4 * grp + ((lane & 15) >> 2)) * VST + 4 * (lane & 3);
#pragma unroll
        for (int dc = 0; dc < NDC; dc++) {
            const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vrow + 16 * dc));
            o[dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[dc], 0, 0, 0);
        }
    };

    // Two register sets alternate (no copies between them), so the loads of
    // the next group are in flight while this one is processed.
    u32x4 ka[NKS], va_[NV], kb[NKS], vb_[NV];
    load_group(t_begin, ka, va_);
    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
        if (t0 + 16 < t_end) load_group(t0 + 16, kb, vb_);
        process(t0, ka, va_, vbuf[wave][0]);
        if (t0 + 16 >= t_end) break;
        if (t0 + 32 < t_end) load_group(t0 + 32, ka, va_);
        process(t0 + 16, kb, vb_, vbuf[wave][1]);
    }
    float l_run = l_part + __shfl_xor(l_part, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);

    if (q_ok) {
        const int64_t idx = ((int64_t)s * a.num_q_heads + qh0 + col) * a.n_splits + split;
        if (grp == 0) {
            a.ws_m[idx] = m_ref;
            a.ws_l[idx] = l_run;
        }
        float *op = a.ws_o + idx * D + 4 * grp;
#pragma unroll
        for (int dc = 0; dc < NDC; dc++) *reinterpret_cast<f32x4 *>(op + 16 * dc) = o[dc];
    }
}

// Merge the partial states of every split of a sequence and finalize:
// M = max m_c, L = sum l_c 2^{(m_c - M) c}, O = sum o_c 2^{(m_c - M) c},
// out = O / L (0 when L == 0, i.e. an empty context).
template <int D>
__global__ __launch_bounds__(256) void paged_decode_combine_kernel(DecodeArgs a)
{
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
    if (pair >= (int64_t)a.num_seqs * a.num_q_heads) return;
    const int s = (int)(pair / a.num_q_heads);
    const int ctx = a.context_lens[s];
    const int ns = ctx > 0 ? (ctx + kSplit - 1) / kSplit : 0;
    const int64_t base = pair * a.n_splits;
    float M = -INFINITY;
    for (int c = lane; c < ns; c += 64) M = fmaxf(M, a.ws_m[base + c]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float m_use = M == -INFINITY ? 0.f : M;
    float L = 0.f, acc[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) acc[i] = 0.f;
    for (int c = 0; c < ns; c++) {
        const float wgt = fast_exp2((a.ws_m[base + c] - m_use) * a.scale_log2);
        L += a.ws_l[base + c] * wgt;
        const float *oc = a.ws_o + (base + c) * D;
#pragma unroll
        for (int i = 0; i < PER; i++) acc[i] += wgt * oc[lane + 64 * i];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t *out = a.out + pair * D;
#pragma unroll
    for (int i = 0; i < PER; i++) out[lane + 64 * i] = (uint16_t)(pack_bf16x2(acc[i] * inv, 0.f) & 0xffffu);
}

// Test hook: the split kernel's address computation, as a plain copy.
__global__ __launch_bounds__(256) void paged_gather_kernel(const uint16_t *pool, const int32_t *block_table,
                                                           const int32_t *context_lens, uint16_t *dense,
                                                           int32_t num_kv_heads, int32_t head_dim, int32_t bs_shift,
                                                           int32_t max_blocks)
{
    const int s = blockIdx.y, t = blockIdx.x;
    if (t >= context_lens[s]) return;
    const int32_t *bt = block_table + (int64_t)s * max_blocks;
    const int chunks = num_kv_heads * head_dim / 8;
    const int64_t T = (int64_t)max_blocks << bs_shift;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        const int kh = c / (head_dim / 8), cc = c % (head_dim / 8);
        const uint16_t *src = pool + paged_token_offset(bt, t, bs_shift, num_kv_heads, head_dim, kh) + cc * 8;
        uint16_t *dst = dense + (((int64_t)s * T + t) * num_kv_heads + kh) * head_dim + cc * 8;
        *reinterpret_cast<u32x4 *>(dst) = load16(src);
    }
}

int64_t decode_n_splits(int32_t max_blocks_per_seq, int32_t block_size)
{
    const int64_t tokens = (int64_t)max_blocks_per_seq * block_size;
    return (tokens + kSplit - 1) / kSplit;
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int64_t n_splits)
{
    const size_t n = (size_t)num_seqs * (size_t)num_q_heads * (size_t)n_splits;
    const size_t ml = (2 * n * sizeof(float) + 255) / 256 * 256;
    return ml + n * (size_t)head_dim * sizeof(float);
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t stream)
{
    const int64_t units = (int64_t)a.num_kv_heads * a.n_sub;
    if (a.n_splits > 0) {
        const dim3 grid((unsigned)((int64_t)a.num_seqs * a.n_splits), (unsigned)((units + 3) / 4)), block(256);
        if (a.bs_shift >= 4) hipLaunchKernelGGL((paged_decode_split_kernel<D, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((paged_decode_split_kernel<D, false>), grid, block, 0, stream, a);
    }
    const int64_t pairs = (int64_t)a.num_seqs * a.num_q_heads;
    hipLaunchKernelGGL(paged_decode_combine_kernel<D>, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_paged_decode(const DecodeArgs &a, int head_dim, hipStream_t stream)
{
    switch (head_dim) {
    case 64: return launch_decode_d<64>(a, stream);
    case 128: return launch_decode_d<128>(a, stream);
    case 256: return launch_decode_d<256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_gather(const uint16_t *pool, const int32_t *block_table, const int32_t *context_lens,
                               uint16_t *dense, int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t bs_shift, int32_t max_blocks, hipStream_t stream)
{
    const int64_t T = (int64_t)max_blocks * block_size;
    if (T == 0 || num_seqs == 0) return hipSuccess;
    hipLaunchKernelGGL(paged_gather_kernel, dim3((unsigned)T, (unsigned)num_seqs), dim3(256), 0, stream, pool,
                       block_table, context_lens, dense, num_kv_heads, head_dim, bs_shift, max_blocks);
    return hipGetLastError();
}

}  // namespace rra
