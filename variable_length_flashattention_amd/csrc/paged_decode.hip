// Paged-KV grouped-query decode attention for gfx950.
//
// Method: "spark_storage/attention_ref.rs" -- the decode state (m, l, o) in
// fp32 (AttnState), its update over the tokens of a list of pool blocks
// (step_tile_ref; the state is carried from one block list to the next), and
// the guarded finalize out = o / l, 0 when l == 0 (finalize_ref).
//
// Schedule: the contexts of all sequences, cut into groups of 16 tokens and
// laid end to end, are split into n_ranges equal ranges of groups.  One wave
// owns one range for one kv head (and its group of up to 16 q heads), so
// every wave streams the same number of K/V bytes however the context
// lengths are distributed.  A range that covers pieces of several sequences
// folds each piece into its own partial state; the piece of sequence s in
// range w is stored in partial slot w + s (two pieces (w, s) and (w', s')
// with w + s == w' + s' cannot both exist, since ranges and sequences are
// both in order).  A combine kernel merges the pieces of each sequence and
// finalizes.  The group offsets of the sequences (an exclusive prefix sum
// of ceil(ctx / 16)) are formed in registers by every wave for up to 256
// sequences; above that a first one-workgroup kernel writes them into the
// workspace.  The stateful interface runs the same kernels with each
// sequence's tokens taken from the tile's block count (cut by a token
// count), and the combine merging into the caller's (m, l, o) instead of
// writing out.
//
// Per 16 tokens a wave computes
//   S^T[token][q head] = K . Q^T     (v_mfma_f32_16x16x32_bf16; K straight
//                                     from the pool into the A operand)
//   the online softmax per q head (the cross-lane max and the rescale of o
//   and l only when a score exceeds the running max, so every probability
//   is at most 1 and a dominant one is exactly 1: its bf16 rounding for the
//   MMA then costs nothing, while l sums the fp32 values),
//   O^T[d][q head] += V^T . P^T      (v_mfma_f32_16x16x16_bf16; V staged in
//                                     wave-private LDS, read transposed).
// Only tokens t < ctx (the sequence's clamped token count) are read; the
// block table is never read at or past ceil(ctx / block_size).
#include "rra_device.h"
#include "rra_internal.h"

namespace rra {

constexpr int kGroup = 16;  // tokens per MMA step

// Context length as the kernels use it: clamped to [0, max_blocks * block_size]
// so that no block-table entry past the row is read.
__device__ __forceinline__ int clamp_ctx(int ctx, int max_blocks, int bs_shift)
{
    return min(max(ctx, 0), max_blocks << bs_shift);
}
// Token count of sequence s (see CtxSource), clamped.
__device__ __forceinline__ int ctx_of(const CtxSource &c, int s)
{
    if (c.context_lens) return clamp_ctx(c.context_lens[s], c.max_blocks, c.bs_shift);
    const int nb = min(max(c.block_counts[s], 0), c.max_blocks);
    const int full = nb << c.bs_shift;
    return c.token_counts ? min(max(c.token_counts[s], 0), full) : full;
}
__host__ __device__ inline CtxSource ctx_source(const DecodeArgs &a)
{
    return CtxSource{a.context_lens, a.block_counts, a.token_counts, a.max_blocks, a.bs_shift};
}

// Group offsets goff[s] = sum_{s' < s} ceil(ctx_s' / 16), s = 0..S, into the
// workspace (one workgroup).
__global__ __launch_bounds__(256) void paged_decode_offsets_kernel(CtxSource src, int32_t num_seqs, int32_t *goff)
{
    __shared__ int wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int base = 0; base < num_seqs; base += 256) {
        const int s = base + tid;
        const int ctx = s < num_seqs ? ctx_of(src, s) : 0;
        const int g = (ctx + kGroup - 1) / kGroup;
        int x = g;  // inclusive scan within the wave
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; w++) before += wsum[w];
        if (s < num_seqs) goff[s] = before + x - g;
        carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (tid == 0) goff[num_seqs] = carry;
}

// Token-group offsets goff(s), s = 0..S, and context lengths as one wave
// sees them.  Up to kRegSeqs sequences the wave computes them itself from
// context_lens into registers (lane j holds goff(64 i + j + 1) and the
// clamped ctx of sequence 64 i + j in register i), so no offsets kernel runs
// and no lookup waits on memory; larger batches read the offsets the offsets
// kernel wrote and search them 64 ways per round trip.  All queries take a
// wave-uniform argument and return a wave-uniform value.
constexpr int kRegSeqs = 256;
struct GroupOffsets {
    int incl[kRegSeqs / 64], ctxr[kRegSeqs / 64];
    const int32_t *mem;
    CtxSource src;
    int S;
    bool in_regs;

    __device__ __forceinline__ void init(const CtxSource &src_, const int32_t *goff_mem, int num_seqs, int lane)
    {
        S = num_seqs;
        mem = goff_mem;
        src = src_;
        in_regs = S <= kRegSeqs;
        if (!in_regs) return;
#pragma unroll
        for (int i = 0; i < kRegSeqs / 64; i++) {
            const int s = 64 * i + lane;
            ctxr[i] = (64 * i < S && s < S) ? ctx_of(src, s) : 0;
        }
        int carry = 0;
#pragma unroll
        for (int i = 0; i < kRegSeqs / 64; i++) {
            const int g = (ctxr[i] + kGroup - 1) / kGroup;
            int x = g;  // inclusive scan within the wave
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            incl[i] = x + carry;
            carry = __builtin_amdgcn_readlane(incl[i], 63);
        }
    }
    // register i's value in lane j (i, j wave-uniform)
    __device__ __forceinline__ static int pick(const int *r, int i, int j)
    {
        const int v = i == 0 ? r[0] : i == 1 ? r[1] : i == 2 ? r[2] : r[3];
        return __builtin_amdgcn_readlane(v, j);
    }
    __device__ __forceinline__ int goff(int s) const
    {
        if (!in_regs) return mem[s];
        return s == 0 ? 0 : pick(incl, (s - 1) >> 6, (s - 1) & 63);
    }
    __device__ __forceinline__ int ctx(int s) const
    {
        return in_regs ? pick(ctxr, s >> 6, s & 63) : ctx_of(src, s);
    }
    // first s in [0, S) with goff(s + 1) > g, for 0 <= g < goff(S)
    __device__ __forceinline__ int seq_of_group(int g, int lane) const
    {
        if (in_regs) {
#pragma unroll
            for (int i = 0; i < kRegSeqs / 64; i++) {
                const uint64_t m = __ballot(64 * i + lane < S && incl[i] > g);
                if (m) return 64 * i + __ffsll((unsigned long long)m) - 1;
            }
            return S - 1;  // not reached
        }
        int lo = 0, hi = S - 1;  // the answer is in [lo, hi]
        while (lo < hi) {
            const int step = (hi - lo + 62) / 63;  // lane 63 samples hi
            const int idx = min(hi, lo + lane * step);
            const uint64_t m = __ballot(mem[idx + 1] > g);  // true at idx = hi
            const int f = __ffsll((unsigned long long)m) - 1;
            const int idx_f = min(hi, lo + f * step);
            lo = f == 0 ? lo : lo + (f - 1) * step + 1;
            hi = idx_f;
        }
        return lo;
    }
};

// BIG: block_size >= 16, so each group of 16 tokens sits in one pool block
// and its block id is wave-uniform.
// GATHER: the test hook's mode.  The kernel walks the same ranges, pieces,
// block-table windows and groups and issues the same K and V loads, then
// stores the loaded registers into dense copies (a.gather_k, a.gather_v
// [S, max_blocks * block_size, Hkv, D]) at the positions the operand layouts
// assign them, instead of folding them into a softmax state.
template <int D, bool BIG, bool GATHER>
__global__ __launch_bounds__(256) void paged_decode_split_kernel(DecodeArgs a)
{
    constexpr int NKS = D / 32;   // k-steps of the QK^T MMA (32 d each)
    constexpr int NDC = D / 16;   // 16-wide d chunks of the output
    constexpr int NV = D / 32;    // 16-byte V pieces per lane per 16 tokens
    constexpr int VST = D + 16;   // LDS row stride of a staged V token
    constexpr int NBT = BIG ? 1 : 4;  // registers of block-table entries per lane
    __shared__ __attribute__((aligned(16))) uint16_t vbuf[4][2][kGroup * VST];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int unit = blockIdx.y * 4 + wave;
    if (unit >= a.num_kv_heads * a.n_sub) return;  // no block-level barriers below
    const int kh = unit / a.n_sub, sub = unit % a.n_sub;
    const int S = a.num_seqs;
    GroupOffsets go;
    go.init(ctx_source(a), a.ws_goff, S, lane);
    const int G = go.goff(S);
    const int P = G / a.n_ranges + (G % a.n_ranges != 0);  // groups per range
    const int64_t g_lo64 = (int64_t)blockIdx.x * P;
    if (g_lo64 >= G) return;
    const int g_lo = (int)g_lo64;
    const int g_hi = (int)min((int64_t)G, g_lo64 + P);

    const int ratio = a.num_q_heads / a.num_kv_heads;
    const int qh0 = kh * ratio + 16 * sub;
    const int nq = min(16, ratio - 16 * sub);
    const int col = lane & 15, grp = lane >> 4;
    const bool q_ok = col < nq;
    const int Hkv = a.num_kv_heads;
    const int bs_shift = a.bs_shift;
    const float sl2 = a.scale_log2;
    const int64_t row_elems = (int64_t)Hkv * D;    // elements per pool token row

    for (int s = go.seq_of_group(g_lo, lane), gs0 = go.goff(s); s < S && gs0 < g_hi; s++) {
        const int gs1 = go.goff(s + 1);
        const int ctx = go.ctx(s);
        const int seg_begin = kGroup * (max(g_lo, gs0) - gs0);
        const int seg_end = min(ctx, kGroup * (min(g_hi, gs1) - gs0));
        gs0 = gs1;  // the next sequence's first group
        if (seg_begin >= seg_end) continue;
        const int32_t *bt = a.block_table + (int64_t)s * a.max_blocks;

        // Q^T operand: lane holds Q[qh0 + col][32*ks + 8*grp .. +7]
        bf16x8 qf[NKS];
        if constexpr (!GATHER) {
            const uint16_t *qrow = a.q + ((int64_t)s * a.num_q_heads + qh0 + (q_ok ? col : 0)) * D + 8 * grp;
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) qf[ks] = as_bf16x8(load16(qrow + 32 * ks));
        }
        f32x4 o[NDC];
#pragma unroll
        for (int dc = 0; dc < NDC; dc++) o[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
        // m_ref: the max (per q head, common to all lanes of that column) the
        // accumulators are scaled to; l_part: this lane's share of the
        // denominator (its 4 tokens per group), summed across lanes at the end.
        float m_ref = -INFINITY, l_part = 0.f;

        // the piece in chunks whose blocks fit the lanes' block-table registers
        for (int c_begin = seg_begin; c_begin < seg_end;) {
            const int blk0 = c_begin >> bs_shift;
            const int t_end = (int)min((int64_t)seg_end, (int64_t)(blk0 + 64 * NBT) << bs_shift);
            const int blk_end = ((t_end - 1) >> bs_shift) + 1;
            int btr[NBT];
#pragma unroll
            for (int r = 0; r < NBT; r++) {
                const int bi = blk0 + lane + 64 * r;
                btr[r] = bi < blk_end ? bt[bi] : 0;
            }
            // Element offset of token t (c_begin <= t < t_end), kv head kh.
            auto token_offset = [&](int t) -> int64_t {
                const int rel = (t >> bs_shift) - blk0;
                int blk = __shfl(btr[0], rel & 63, 64);
                if (!BIG && rel >= 64) {
                    const int b1 = __shfl(btr[NBT > 1 ? 1 : 0], rel & 63, 64),
                              b2 = __shfl(btr[NBT > 2 ? 2 : 0], rel & 63, 64),
                              b3 = __shfl(btr[NBT > 3 ? 3 : 0], rel & 63, 64);
                    blk = rel < 128 ? b1 : rel < 192 ? b2 : b3;
                }
                const int64_t slot = t & ((1 << bs_shift) - 1);
                return (((int64_t)blk << bs_shift) + slot) * row_elems + (int64_t)kh * D;
            };
            // BIG: base offset of group t0's block (uniform)
            auto group_base = [&](int t0) -> int64_t {
                const int blk = __builtin_amdgcn_readlane(btr[0], (t0 >> bs_shift) - blk0);
                return ((int64_t)blk << bs_shift) * row_elems + (int64_t)kh * D;
            };
            // Loads of one group: K straight into the MMA A operand (lane:
            // token t0 + col, d = 32*ks + 8*grp..), V rows for the LDS stage
            // (lane: token t0 + c/(D/8), 16-byte piece c%(D/8), c = lane + 64 i).
            // Tokens at or past t_end re-read token t_end-1: their scores are
            // masked and their probabilities are exactly 0, and the loads stay
            // unconditional (a conditional load merged with a default makes the
            // compiler wait for it on the spot, defeating the prefetch).  Every
            // K/V row is read once per call, so the loads carry the streaming
            // (non-temporal) hint: measured on gfx950, the decode workload runs
            // 12 % faster with it (207 -> 183 us per call).
            auto load_group = [&](int t0, u32x4 *kd, u32x4 *vd) {
                const int64_t gb = BIG ? group_base(t0) : 0;
                const int mask = (1 << bs_shift) - 1;
                const int tc = min(t0 + col, t_end - 1);
                const uint16_t *p =
                    a.k_pool + (BIG ? gb + (int64_t)(tc & mask) * row_elems : token_offset(tc)) + 8 * grp;
#pragma unroll
                for (int ks = 0; ks < NKS; ks++) kd[ks] = load16_stream(p + 32 * ks);
#pragma unroll
                for (int i = 0; i < NV; i++) {
                    const int c = lane + 64 * i;
                    const int tvc = min(t0 + c / (D / 8), t_end - 1);
                    const int64_t off = BIG ? gb + (int64_t)(tvc & mask) * row_elems : token_offset(tvc);
                    vd[i] = load16_stream(a.v_pool + off + (c % (D / 8)) * 8);
                }
            };
            // Fold one group of 16 tokens into the running state.
            auto process = [&](int t0, const u32x4 *kr, const u32x4 *vr, uint16_t *vb) {
                // stage this group's V rows in the wave's LDS (two buffers, so
                // the next group's stores never race this group's transposed
                // reads; LDS operations of one wave complete in order)
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
                if (__builtin_amdgcn_ballot_w64(lmax > m_ref)) {
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

            // GATHER: store a group's loaded registers where the operand
            // layouts place them: K lane (col, grp) holds token t0 + col,
            // d = 32*ks + 8*grp..+7; V piece c = lane + 64 i holds token
            // t0 + c/(D/8), d = 8*(c%(D/8))..+7.  Tokens at or past t_end
            // (re-reads of token t_end-1) are not stored.
            auto scatter = [&](int t0, const u32x4 *kr, const u32x4 *vr) {
                const int64_t T = (int64_t)a.max_blocks << bs_shift;  // dense rows per sequence
                const int tk = t0 + col;
                if (tk < t_end) {
                    uint16_t *dk = a.gather_k + (((int64_t)s * T + tk) * Hkv + kh) * D + 8 * grp;
#pragma unroll
                    for (int ks = 0; ks < NKS; ks++) *reinterpret_cast<u32x4 *>(dk + 32 * ks) = kr[ks];
                }
#pragma unroll
                for (int i = 0; i < NV; i++) {
                    const int c = lane + 64 * i;
                    const int tv = t0 + c / (D / 8);
                    if (tv < t_end)
                        *reinterpret_cast<u32x4 *>(a.gather_v + (((int64_t)s * T + tv) * Hkv + kh) * D +
                                                   8 * (c % (D / 8))) = vr[i];
                }
            };
            auto consume = [&](int t0, const u32x4 *kr, const u32x4 *vr, uint16_t *vb) {
                if constexpr (GATHER) scatter(t0, kr, vr);
                else process(t0, kr, vr, vb);
            };

            // Two register sets alternate (no copies between them), so the
            // loads of the next group are in flight while this one is processed.
            u32x4 ka[NKS], va_[NV], kb[NKS], vb_[NV];
            load_group(c_begin, ka, va_);
            for (int t0 = c_begin; t0 < t_end; t0 += 2 * kGroup) {
                if (t0 + kGroup < t_end) load_group(t0 + kGroup, kb, vb_);
                consume(t0, ka, va_, vbuf[wave][0]);
                if (t0 + kGroup >= t_end) break;
                if (t0 + 2 * kGroup < t_end) load_group(t0 + 2 * kGroup, ka, va_);
                consume(t0 + kGroup, kb, vb_, vbuf[wave][1]);
            }
            c_begin = t_end;
        }

        if constexpr (GATHER) continue;
        // this piece's partial state (unnormalised o, l, and the reference max)
        float l_run = l_part + __shfl_xor(l_part, 16, 64);
        l_run += __shfl_xor(l_run, 32, 64);
        if (q_ok) {
            const int64_t idx = ((int64_t)(blockIdx.x + s) * a.num_q_heads + qh0 + col);
            if (grp == 0) {
                a.ws_m[idx] = m_ref;
                a.ws_l[idx] = l_run;
            }
            float *op = a.ws_o + idx * D + 4 * grp;
#pragma unroll
            for (int dc = 0; dc < NDC; dc++) *reinterpret_cast<f32x4 *>(op + 16 * dc) = o[dc];
        }
    }
}

// Merge the pieces of each sequence and finalize: M = max m_c,
// L = sum l_c 2^{(m_c - M) c}, O = sum o_c 2^{(m_c - M) c}, out = O / L
// (0 when L == 0, i.e. an empty context).  A step of the stateful interface
// merges the caller's state (m, l, o) in as one more piece (its m is in
// scaled units) and stores the merged state instead of out.  One wave per
// (sequence, q head), four per workgroup, each on its own (no LDS, no
// barrier): it finds M and L over all pieces (lane-parallel loads) and sums
// o.  A piece's o is D floats; LP = D/4 lanes read it as 16-byte pieces, so
// one wave load covers 64/LP pieces, each lane weighting its own piece
// (weights are held one piece per lane and fetched with a lane shuffle).
template <int D>
__global__ __launch_bounds__(256) void paged_decode_combine_kernel(DecodeArgs a)
{
    constexpr int LP = D / 4 < 64 ? D / 4 : 64;   // lanes per piece
    constexpr int PPL = 64 / LP;                   // pieces per wave load
    constexpr int NA = D / LP / 4;                 // 16-byte pieces per lane
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= (int64_t)a.num_seqs * a.num_q_heads) return;
    const int s = (int)(pair / a.num_q_heads), qh = (int)(pair % a.num_q_heads);
    GroupOffsets go;
    go.init(ctx_source(a), a.ws_goff, a.num_seqs, lane);
    const int G = go.goff(a.num_seqs);
    const int P = max(1, G / a.n_ranges + (G % a.n_ranges != 0));
    const int gs0 = go.goff(s), gs1 = go.goff(s + 1);
    // ranges w_first..w_last hold the pieces of sequence s (none when empty);
    // the clamp keeps the reads inside the workspace whatever the offsets hold
    const int w_first = min(gs0 / P, a.n_ranges - 1);
    const int npieces = gs1 > gs0 ? min((gs1 - 1) / P, a.n_ranges - 1) - w_first + 1 : 0;
    auto slot = [&](int c) -> int64_t { return (int64_t)(w_first + c + s) * a.num_q_heads + qh; };
    const int sub = lane / LP, dl = lane % LP;  // this lane's piece within a load, and d chunk
    // One round trip for the common case: m and l of pieces 0..63 (one per
    // lane), the o of the first KPRE*PPL pieces, and the caller's state max.
    // Loads past the last piece read the last piece (weight 0).
    constexpr int KPRE = 4;
    const bool stateful = a.st_m != nullptr;
    const float m_prev = stateful ? a.st_m[pair] : -INFINITY;
    float m_c = -INFINITY, l_c = 0.f;
    if (lane < npieces) {
        m_c = a.ws_m[slot(lane)];
        l_c = a.ws_l[slot(lane)];
    }
    f32x4 opre[KPRE][NA];
    if (npieces > 0) {
#pragma unroll
        for (int k = 0; k < KPRE; k++) {
            const int cc = min(k * PPL + sub, npieces - 1);
            const float *oc = a.ws_o + slot(cc) * D + 4 * dl;
#pragma unroll
            for (int i = 0; i < NA; i++) opre[k][i] = *reinterpret_cast<const f32x4 *>(oc + 4 * LP * i);
        }
    }
    float M = m_c;
    for (int c = 64 + lane; c < npieces; c += 64) M = fmaxf(M, a.ws_m[slot(c)]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    // stateful step: the caller's state is one more piece (m in scaled units)
    const float M_s = fmaxf(m_prev, M == -INFINITY ? -INFINITY : M * a.scale);  // merged max, scaled units
    if (stateful && M_s == -INFINITY) return;  // nothing seen yet and nothing new (uniform in the wave)
    const float m_use = stateful ? M_s / a.scale : (M == -INFINITY ? 0.f : M);
    float L = 0.f;
    f32x4 acc[NA];
#pragma unroll
    for (int i = 0; i < NA; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < npieces; c0 += 64) {
        // lane j holds piece c0 + j: its weight 2^{(m_c - M) c} (0 past the end)
        const int c = c0 + lane;
        float wgt = 0.f;
        if (c < npieces) {
            const float mc = c0 == 0 ? m_c : a.ws_m[slot(c)];
            wgt = fast_exp2((mc - m_use) * a.scale_log2);
            L += (c0 == 0 ? l_c : a.ws_l[slot(c)]) * wgt;
        }
        const int n = min(64, npieces - c0);
        // pieces j (+ sub), j = 0, PPL, 2 PPL, ... of the chunk; in the first
        // chunk the first KPRE loads are already in registers
        int j = 0;
        if (c0 == 0) {
#pragma unroll
            for (int k = 0; k < KPRE; k++, j += PPL) {
                const int jj = j + sub;
                const float wj = __shfl(wgt, jj & 63, 64);
#pragma unroll
                for (int i = 0; i < NA; i++) acc[i] += (jj < n ? wj : 0.f) * opre[k][i];
            }
        }
        for (; j < n; j += PPL) {
            const int jj = j + sub;  // this lane's piece, relative to c0
            const float wj = __shfl(wgt, jj & 63, 64);
            const int cc = min(c0 + jj, npieces - 1);  // (weight 0 past the end)
            const float *oc = a.ws_o + slot(cc) * D + 4 * dl;
#pragma unroll
            for (int i = 0; i < NA; i++) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(oc + 4 * LP * i);
                acc[i] += (jj < n ? wj : 0.f) * v;
            }
        }
    }
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
    // lanes l and l + k*LP hold the same d range for different pieces
#pragma unroll
    for (int off = LP; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < NA; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) acc[i][e] += __shfl_xor(acc[i][e], off, 64);
    if (sub == 0) {
        if (stateful) {
            const float wp = m_prev == -INFINITY ? 0.f : fast_exp2((m_prev - M_s) * kLog2e);
            float *so = a.st_o + pair * D + 4 * dl;
#pragma unroll
            for (int i = 0; i < NA; i++) {
                f32x4 *p4 = reinterpret_cast<f32x4 *>(so + 4 * LP * i);
                *p4 = acc[i] + wp * *p4;
            }
            if (dl == 0) {
                a.st_l[pair] = L + wp * a.st_l[pair];
                a.st_m[pair] = M_s;
            }
            return;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t *out = a.out + pair * D + 4 * dl;
#pragma unroll
        for (int i = 0; i < NA; i++) {
            const u32x2 pr = {pack_bf16x2(acc[i][0] * inv, acc[i][1] * inv), pack_bf16x2(acc[i][2] * inv, acc[i][3] * inv)};
            *reinterpret_cast<u32x2 *>(out + 4 * LP * i) = pr;
        }
    }
}

// finalize of the stateful interface: out = o / l, 0 where l == 0.  One
// thread per 4 floats of o; its o and its unit's l are loaded together.
__global__ __launch_bounds__(256) void decode_finalize_kernel(const float *state_l, const float *state_o,
                                                              uint16_t *out, int64_t units, int32_t D)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units * (D / 4)) return;
    const f32x4 o = reinterpret_cast<const f32x4 *>(state_o)[i];
    const float l = state_l[i / (D / 4)];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const u32x2 pr = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    reinterpret_cast<u32x2 *>(out)[i] = pr;
}

// The stateful interface's initial state: m = -inf, l = 0, o = 0.  One
// thread per unit for m and l and per 4 floats of o (16-byte stores; D is a
// multiple of 4 and o 16-byte aligned).
__global__ __launch_bounds__(256) void decode_state_init_kernel(float *state_m, float *state_l, float *state_o,
                                                                int64_t units, int32_t D)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < units) {
        state_m[i] = -INFINITY;
        state_l[i] = 0.f;
    }
    if (i < units * (D / 4)) reinterpret_cast<f32x4 *>(state_o)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

hipError_t launch_decode_finalize(const float *state_l, const float *state_o, uint16_t *out, int64_t units,
                                  int32_t head_dim, hipStream_t stream)
{
    if (units == 0) return hipSuccess;
    const int64_t blocks = (units * (head_dim / 4) + 255) / 256;
    hipLaunchKernelGGL(decode_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, state_l, state_o, out,
                       units, head_dim);
    return hipGetLastError();
}

hipError_t launch_decode_state_init(float *state_m, float *state_l, float *state_o, int64_t units, int32_t head_dim,
                                    hipStream_t stream)
{
    if (units == 0) return hipSuccess;
    const int64_t threads = units * (head_dim / 4) > units ? units * (head_dim / 4) : units;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(decode_state_init_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, state_m, state_l,
                       state_o, units, head_dim);
    return hipGetLastError();
}

// Ranges of token groups: enough waves for one full round on a 256-CU device
// (256 CUs x 4 SIMDs x the split kernel's waves per SIMD: 4, 2 and 1 at
// head_dim 64, 128 and 256), spread over the kv-head units.
int32_t decode_n_ranges(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim)
{
    const int ratio = num_q_heads / num_kv_heads;
    const int units = num_kv_heads * ((ratio + 15) / 16);
    const int waves = 256 * 4 * (head_dim == 64 ? 4 : head_dim == 128 ? 2 : 1);
    return max(1, waves / units);
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim)
{
    const size_t goff = ((size_t)num_seqs + 1) * sizeof(int32_t);
    const size_t slots = (size_t)decode_n_ranges(num_q_heads, num_kv_heads, head_dim) + (size_t)num_seqs;
    const size_t n = slots * (size_t)num_q_heads;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return up(goff) + up(2 * n * sizeof(float)) + n * (size_t)head_dim * sizeof(float);
}

template <int D, bool GATHER>
static void launch_split(const DecodeArgs &a, hipStream_t stream)
{
    if (a.num_seqs > kRegSeqs)
        hipLaunchKernelGGL(paged_decode_offsets_kernel, dim3(1), dim3(256), 0, stream, ctx_source(a), a.num_seqs,
                           a.ws_goff);
    const int64_t units = (int64_t)a.num_kv_heads * a.n_sub;
    const dim3 grid((unsigned)a.n_ranges, (unsigned)((units + 3) / 4)), block(256);
    if (a.bs_shift >= 4) hipLaunchKernelGGL((paged_decode_split_kernel<D, true, GATHER>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((paged_decode_split_kernel<D, false, GATHER>), grid, block, 0, stream, a);
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t stream)
{
    launch_split<D, false>(a, stream);
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

hipError_t launch_paged_gather(const DecodeArgs &a, int head_dim, hipStream_t stream)
{
    switch (head_dim) {
    case 64: launch_split<64, true>(a, stream); break;
    case 128: launch_split<128, true>(a, stream); break;
    case 256: launch_split<256, true>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rra
