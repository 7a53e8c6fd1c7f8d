// Backward pass of the variable-length attention forward for gfx950.
//
// The forward ("Varlen Flash Attention Implementation Plan", Task 1) keeps
// the log-sum-exp of every row so that a backward pass can rebuild the
// probabilities P = exp(scale q.k - lse) without the row max and sum; the
// plan names the backward module but gives no code, so this is the chain
// rule of the forward definition:
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - dsum) with dsum_i = dO_i . O_i,
//   dQ = scale dS K,  dK = scale dS^T Q
// (dsum_i equals sum_j P_ij dP_ij, the softmax Jacobian's row term).
// Grouped-query K/V: the dK and dV of kv head kh sum over its query heads.
//
// Two kernels, no atomics, deterministic:
//   1. varlen_bwd_dq_kernel: one work item per (sequence, 128-query tile,
//      head), the forward's work list; each wave owns 32 query rows (Q and
//      dO in VGPRs), forms dsum of its rows from dO and out, and walks the
//      key tiles, staged into LDS:
//        S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T
//      (the S^T orientation of the forward: a query per lane column).  It
//      also stores dsum and lse * log2(e) head-major for the next kernel.
//   2. varlen_bwd_dkv_kernel: one work item per (sequence, 128-key block,
//      kv head); each wave owns 32 keys (K and V in VGPRs) and walks the
//      32-row query tiles of every query head of the group, staged into LDS:
//        S = Q K^T, P, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS
//      (a key per lane column, so P and dS feed the second pair of MMAs
//      straight from the accumulators, with dO^T and Q^T read transposed).
// Tiles that are read both row-wise (ds_read_b128) and transposed
// (ds_read_b64_tr_b16) use one XOR swizzle of their 16-byte chunks that is
// conflict-free enough for both.
#include <type_traits>

#include "rra_device.h"
#include "rra_internal.h"
#include "tile_map.h"

namespace rra {

template <int D>
struct BwdTile {
    static constexpr int NW = 4;               // waves per workgroup
    static constexpr int ROWB = D * 2;         // bytes per row
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int RPL = NW * 1024 / ROWB;  // rows between one lane's 1 KiB loads
    // chunk swizzle: row-wise reads of 8 consecutive rows and transposed reads
    // of 4 consecutive rows (2 chunks each) both spread over the banks
    __device__ static int swz(int row) { return (2 * (row & 3) | ((row >> 2) & 1)) & (CPR - 1); }
    static_assert(RPL % 8 == 0, "the swizzle must repeat with the load period");
};

// Direct-to-LDS staging of `rows` rows (rows past `nvalid` re-read row
// nvalid-1) of a row-major tensor with row stride `stride` bytes, starting at
// `base`, into a swizzled LDS tile: wave w fills 1 KiB blocks w, w+NW, ...
template <int D, int ROWS>
__device__ __forceinline__ void stage_rows(const uint8_t *base, int64_t stride, int nvalid, uint8_t *lds, int wave,
                                           int lane)
{
    using T = BwdTile<D>;
    constexpr int ROWB = T::ROWB, NW = T::NW, RPL = T::RPL;
    constexpr int WL = ROWS * ROWB / 1024 / NW;
    static_assert(WL * 1024 * NW == ROWS * ROWB, "tile must split evenly over the waves");
    const int srow0 = (wave * 1024 + lane * 16) / ROWB, pch = (lane * 16 % ROWB) / 16;
    const __amdgpu_buffer_rsrc_t r = raw_buffer(base);
#pragma unroll
    for (int i = 0; i < WL; i++) {
        const int row = min(srow0 + i * RPL, nvalid - 1);
        const uint32_t voff = (uint32_t)(row * stride + 16 * (pch ^ T::swz(srow0 + i * RPL)));
        buffer_to_lds16(r, lds + (i * NW + wave) * 1024, voff, 0);
    }
}

// A operand of v_mfma_f32_32x32x16_bf16 read row-wise: rows row0 + lane%32,
// d = 16*ks + 8*(lane/32) .. +7.
template <int D>
__device__ __forceinline__ bf16x8 read_rows(const uint8_t *tile, int row0, int ks, int lane)
{
    const int row = row0 + (lane & 31);
    const int ch = (2 * ks + (lane >> 5)) ^ BwdTile<D>::swz(row);
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(tile + row * (D * 2) + 16 * ch));
}

// A operand read transposed: A[m = d][k] for d = 32*dc + lane%32 and the 16
// rows of k-step m of the tile in the order the C registers of a 32x32
// accumulator hold them (rows 16m + 4*(lane/32) + 0..3 and 16m + 8 + ...).
template <int D>
__device__ __forceinline__ bf16x8 read_cols(const uint8_t *tile, int m, int dc, int lane)
{
    const int g = lane >> 4, j = lane & 15;
    const int row = 16 * m + 4 * (g >> 1) + (j >> 2);
    const int sw = BwdTile<D>::swz(row);  // rows row and row + 8 share it
    const uint8_t *r0 = tile + row * (D * 2) + 8 * (j & 1);
    const int ch = (4 * dc + 2 * (g & 1) + ((j & 3) >> 1)) ^ sw;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(r0 + 16 * ch));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(r0 + 8 * (D * 2) + 16 * ch));
    return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                            __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
}

// B operand of k-step m from packed bf16 pairs of a 32x32 accumulator.
__device__ __forceinline__ bf16x8 packed_b(const uint32_t (&pk)[8], int m)
{
    return as_bf16x8(u32x4{pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]});
}

// Store a 32x32 fp32 accumulator tile (C layout: row = d = 32*dc + 8*(r/4) +
// 4*(lane/32) + r%4, col = lane%32 = this lane's row of dst) times `mul` as
// bf16 into the lane's output row.
template <int NDC>
__device__ __forceinline__ void store_rows_T(uint16_t *row_ptr, const f32x16 (&acc)[NDC], float mul, int lane)
{
    uint16_t *p = row_ptr + 4 * (lane >> 5);
#pragma unroll
    for (int dc = 0; dc < NDC; dc++)
#pragma unroll
        for (int rb4 = 0; rb4 < 4; rb4++) {
            const u32x2 pr = {pack_bf16x2(acc[dc][4 * rb4] * mul, acc[dc][4 * rb4 + 1] * mul),
                              pack_bf16x2(acc[dc][4 * rb4 + 2] * mul, acc[dc][4 * rb4 + 3] * mul)};
            *reinterpret_cast<u32x2 *>(p + 32 * dc + 8 * rb4) = pr;
        }
}

// ---------------------------------------------------------------------------
// 1. dQ (and dsum, lse2).  Same work list and query layout as the forward
// kernel.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, (D == 256 ? 1 : 2)) void varlen_bwd_dq_kernel(BwdArgs a)
{
    using T = BwdTile<D>;
    constexpr int NW = T::NW, BQ = kBwdQRows, BK = D <= 64 ? 64 : 32, TB = BK * T::ROWB;
    constexpr int NC = BK / 32, NKS = D / 16, NDC = D / 32;
    static_assert(BQ == 32 * NW, "one 32-row block per wave");
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TB];
    __shared__ int sched[kSchedInts];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.num_heads, Hkv = a.num_kv_heads;
    const float sl2 = a.scale_log2;
    float *ws_lse2 = a.ws, *ws_dsum = a.ws + (int64_t)H * a.total_q;
    const WorkTables wt = build_work_tables(a.cu_q, a.cu_k, a.batch + 1, a.batch, BQ, 0, a.levels_q, sched, kSchedInts);

    for (int64_t k = 0;; k++) {
        const int64_t w = serpentine_item(k, blockIdx.x, gridDim.x);
        if (w >= a.n_items_q) break;
        int b, qt, h;
        if (!decode_work_item(wt, a.cu_q, H, w, lane, b, qt, h)) break;
        __syncthreads();  // LDS of the previous item no longer in use
        b = __builtin_amdgcn_readfirstlane(b);
        qt = __builtin_amdgcn_readfirstlane(qt);
        h = __builtin_amdgcn_readfirstlane(h);
        const int *cuq = wt.cached ? wt.cuq : a.cu_q, *cuk = wt.cached ? wt.cuk : a.cu_k;
        const int q0 = __builtin_amdgcn_readfirstlane(cuq[b]), k0 = __builtin_amdgcn_readfirstlane(cuk[b]);
        const int Lq = __builtin_amdgcn_readfirstlane(cuq[b + 1]) - q0;
        const int Lk = __builtin_amdgcn_readfirstlane(cuk[b + 1]) - k0;
        const int diag = Lk - Lq;
        const int i0 = qt * BQ, nrows = min(BQ, Lq - i0);
        int kend = Lk;
        if (CAUSAL) kend = max(0, min(Lk, i0 + nrows + diag));
        const int nkt = (kend + BK - 1) / BK;
        const int iw = i0 + 32 * wave;           // this wave's first row
        const int my_i = iw + (lane & 31);
        const bool row_ok = my_i < Lq;
        int kend_w = Lk;
        if (CAUSAL) kend_w = max(0, min(Lk, min(iw + 31, Lq - 1) + 1 + diag));
        if (32 * wave >= nrows) kend_w = 0;
        const int nkt_w = (kend_w + BK - 1) / BK;

        const int kh = h / a.gqa_ratio;
        const int64_t kstride = (int64_t)Hkv * T::ROWB;
        const uint8_t *kseq = reinterpret_cast<const uint8_t *>(a.k + ((int64_t)k0 * Hkv + kh) * D);
        const uint8_t *vseq = reinterpret_cast<const uint8_t *>(a.v + ((int64_t)k0 * Hkv + kh) * D);
        auto stage = [&](int kt, uint8_t *kb, uint8_t *vb) __attribute__((always_inline)) {
            stage_rows<D, BK>(kseq + kt * BK * kstride, kstride, Lk - kt * BK, kb, wave, lane);
            stage_rows<D, BK>(vseq + kt * BK * kstride, kstride, Lk - kt * BK, vb, wave, lane);
        };
        if (nkt > 0) stage(0, k_lds0, v_lds0);

        // Q^T and dO^T operands: lane holds row my_i (clamped), d = 16*ks + 8*(lane/32) ..
        bf16x8 qf[NKS], gf[NKS];
        const int qr = min(my_i, Lq - 1);
        {
            const int64_t off = ((int64_t)(q0 + qr) * H + h) * D + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) {
                qf[ks] = as_bf16x8(load16(a.q + off + 16 * ks));
                gf[ks] = as_bf16x8(load16(a.dout + off + 16 * ks));
            }
        }
        // dsum = dO . out of the row (each half-wave holds half of d), and
        // lse2 = lse * log2(e) (+inf for a row without visible keys, so that
        // every probability of the row is 0); stored for the dk/dv kernel
        float dsum, lse2;
        {
            const int64_t row = (int64_t)(q0 + qr) * H + h;
            const uint16_t *orow = a.out + row * D + 8 * (lane >> 5);
            float part = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) {
                const u32x4 o4 = load16(orow + 16 * ks), g4 = __builtin_bit_cast(u32x4, gf[ks]);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    part += bf16lo_to_f32(o4[e]) * bf16lo_to_f32(g4[e]) + bf16hi_to_f32(o4[e]) * bf16hi_to_f32(g4[e]);
            }
            dsum = sum_across_halves(part);
            const float l = a.lse[row];
            lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
            if (row_ok && lane < 32) {
                ws_lse2[(int64_t)h * a.total_q + q0 + my_i] = lse2;
                ws_dsum[(int64_t)h * a.total_q + q0 + my_i] = dsum;
            }
        }
        f32x16 acc[NDC];
#pragma unroll
        for (int dc = 0; dc < NDC; dc++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[dc][r] = 0.f;

        auto tile = [&](int kt, const uint8_t *Kb, const uint8_t *Vb, uint8_t *kn, uint8_t *vn) {
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // tile kt visible; every wave is done with tile kt-1
            if (kt + 1 < nkt) stage(kt + 1, kn, vn);
            if (kt >= nkt_w) return;
            const int kbase = kt * BK;
            // S^T = K Q^T and dP^T = V dO^T
            f32x16 s[NC], dp[NC];
#pragma unroll
            for (int c = 0; c < NC; c++)
#pragma unroll
                for (int r = 0; r < 16; r++) s[c][r] = dp[c][r] = 0.f;
#pragma unroll
            for (int c = 0; c < NC; c++)
#pragma unroll
                for (int ks = 0; ks < NKS; ks++) {
                    s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows<D>(Kb, 32 * c, ks, lane), qf[ks], s[c], 0, 0, 0);
                    dp[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows<D>(Vb, 32 * c, ks, lane), gf[ks], dp[c], 0, 0, 0);
                }
            // P^T and dS^T (masked pairs give exactly 0); the mask is applied
            // only on the tiles that need it (a wave-uniform branch between
            // two versions of the loop)
            const bool need_mask = (kbase + BK > Lk) || (CAUSAL && kbase + BK - 1 > iw + diag);
            const int last = CAUSAL ? min(Lk - 1, my_i + diag) : Lk - 1;
            uint32_t pk[NC][8];
            auto probs = [&](auto masked) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
                for (int c = 0; c < NC; c++)
#pragma unroll
                    for (int r2 = 0; r2 < 8; r2++) {
                        float d2[2];
#pragma unroll
                        for (int e = 0; e < 2; e++) {
                            const int r = 2 * r2 + e;
                            const float p = fast_exp2(s[c][r] * sl2 - lse2);
                            d2[e] = p * (dp[c][r] - dsum);
                            if (MASKED) {
                                const int key = kbase + 32 * c + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                                if (key > last) d2[e] = 0.f;
                            }
                        }
                        pk[c][r2] = pack_bf16x2(d2[0], d2[1]);
                    }
            };
            if (need_mask) probs(std::true_type{});
            else probs(std::false_type{});
            // dQ^T += K^T dS^T, 16 keys per MMA
#pragma unroll
            for (int m = 0; m < BK / 16; m++)
#pragma unroll
                for (int dc = 0; dc < NDC; dc++)
                    acc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_cols<D>(Kb, m, dc, lane),
                                                                    packed_b(pk[m >> 1], m & 1), acc[dc], 0, 0, 0);
        };
        for (int kt = 0; kt < nkt; kt += 2) {
            tile(kt, k_lds0, v_lds0, k_lds1, v_lds1);
            if (kt + 1 < nkt) tile(kt + 1, k_lds1, v_lds1, k_lds0, v_lds0);
        }
        if (row_ok) store_rows_T<NDC>(a.dq + ((int64_t)(q0 + my_i) * H + h) * D, acc, a.scale, lane);
    }
}

// ---------------------------------------------------------------------------
// 3. dK and dV.  Work list over 128-key blocks (the keys are the tiled
// dimension; level r of a sequence is its (r+1)-th block from the end, which
// under causal masking sees the most query tiles at the highest level).  At
// head_dim 256 the dK/dV accumulators of a wave would not fit next to its K
// and V, so an item there owns one half of the d range (S and dP are
// computed by both halves' items).
template <int D>
constexpr int bwd_dkv_split() { return D == 256 ? 2 : 1; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void varlen_bwd_dkv_kernel(BwdArgs a)
{
    using T = BwdTile<D>;
    constexpr int NW = T::NW, BKB = kBwdKRows, BQB = 32, TB = BQB * T::ROWB;
    constexpr int NSPLIT = bwd_dkv_split<D>();
    constexpr int NKS = D / 16, NDC = D / 32 / NSPLIT;  // accumulated 32-wide d chunks
    static_assert(BKB == 32 * NW, "32 keys per wave");
    __shared__ __attribute__((aligned(1024))) uint8_t q_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t g_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t q_lds1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t g_lds1[TB];
    __shared__ __attribute__((aligned(256))) float st_lds0[64];  // lse2 of the 32 rows, then dsum
    __shared__ __attribute__((aligned(256))) float st_lds1[64];
    __shared__ int sched[kSchedInts];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.num_heads, Hkv = a.num_kv_heads, R = a.gqa_ratio;
    const float sl2 = a.scale_log2;
    // (the key offsets are the tiled list here, the query offsets the other)
    const WorkTables wt = build_work_tables(a.cu_k, a.cu_q, a.batch + 1, a.batch, BKB, 0, a.levels_k, sched, kSchedInts);
    const __amdgpu_buffer_rsrc_t ws_r = raw_buffer(a.ws);

    for (int64_t k = 0;; k++) {
        const int64_t w = serpentine_item(k, blockIdx.x, gridDim.x);
        if (w >= a.n_items_k) break;
        int b, lvl, hs;
        if (!decode_work_item(wt, a.cu_k, Hkv * NSPLIT, w, lane, b, lvl, hs)) break;
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(b);
        lvl = __builtin_amdgcn_readfirstlane(lvl);
        hs = __builtin_amdgcn_readfirstlane(hs);
        const int kh = hs / NSPLIT, dc0 = (hs % NSPLIT) * NDC;  // kv head, first accumulated d chunk
        const int *cuk = wt.cached ? wt.cuq : a.cu_k, *cuq = wt.cached ? wt.cuk : a.cu_q;
        const int k0 = __builtin_amdgcn_readfirstlane(cuk[b]), q0 = __builtin_amdgcn_readfirstlane(cuq[b]);
        const int Lk = __builtin_amdgcn_readfirstlane(cuk[b + 1]) - k0;
        const int Lq = __builtin_amdgcn_readfirstlane(cuq[b + 1]) - q0;
        const int diag = Lk - Lq;
        const int nkb = (Lk + BKB - 1) / BKB;
        const int kbase = (nkb - 1 - lvl) * BKB;
        const int kw0 = kbase + 32 * wave;  // this wave's first key
        const int my_key = kw0 + (lane & 31);
        int qt0 = 0;
        if (CAUSAL) qt0 = max(0, kbase - diag) / BQB;
        const int nqt = (Lq + BQB - 1) / BQB;
        const int nq = max(0, nqt - qt0);
        const int ntiles = R * nq;

        // K and V of this wave's keys as B operands (key = lane%32; rows past
        // the sequence re-read its last key; their columns are masked)
        bf16x8 kf[NKS], vf[NKS];
        {
            const int kr = min(my_key, Lk - 1);
            const int64_t off = ((int64_t)(k0 + kr) * Hkv + kh) * D + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) {
                kf[ks] = as_bf16x8(load16(a.k + off + 16 * ks));
                vf[ks] = as_bf16x8(load16(a.v + off + 16 * ks));
            }
        }
        f32x16 dk[NDC], dv[NDC];
#pragma unroll
        for (int dc = 0; dc < NDC; dc++)
#pragma unroll
            for (int r = 0; r < 16; r++) dk[dc][r] = dv[dc][r] = 0.f;

        const int64_t qstride = (int64_t)H * T::ROWB;
        auto stage = [&](int t, uint8_t *qb, uint8_t *gb, float *sb) __attribute__((always_inline)) {
            const int h = kh * R + t / nq, qbase = (qt0 + t % nq) * BQB;
            const int64_t off = ((int64_t)(q0 + qbase) * H + h) * T::ROWB;
            stage_rows<D, BQB>(reinterpret_cast<const uint8_t *>(a.q) + off, qstride, Lq - qbase, qb, wave, lane);
            stage_rows<D, BQB>(reinterpret_cast<const uint8_t *>(a.dout) + off, qstride, Lq - qbase, gb, wave, lane);
            if (wave == 0) {
                // lanes 0-31: lse2 of rows qbase + lane; lanes 32-63: dsum (rows clamped)
                const int row = min(qbase + (lane & 31), Lq - 1);
                const int64_t idx = (lane >> 5) * (int64_t)H * a.total_q + (int64_t)h * a.total_q + q0 + row;
                buffer_to_lds4(ws_r, sb, (uint32_t)(idx * 4), 0);
            }
        };
        if (ntiles > 0) stage(0, q_lds0, g_lds0, st_lds0);

        auto tile = [&](int t, const uint8_t *Qb, const uint8_t *Gb, const float *Sb, uint8_t *qn, uint8_t *gn,
                        float *sn) {
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // tile t visible; every wave is done with tile t-1
            if (t + 1 < ntiles) stage(t + 1, qn, gn, sn);
            const int qbase = (qt0 + t % nq) * BQB;
            // some pair of this wave's keys and the tile's rows visible?
            const int qlast = min(qbase + BQB - 1, Lq - 1);
            if (kw0 >= Lk || (CAUSAL && kw0 > qlast + diag)) return;
            // S = Q K^T, then dP = dO V^T (rows = queries, cols = keys); the
            // row operands are read RA MMAs ahead, and the scheduling
            // barriers keep the two chains apart (interleaved, they keep
            // both accumulators and all their operands live at once)
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; r++) s[r] = dp[r] = 0.f;
            {
                constexpr int NM = 2 * NKS, RA = 2;
                auto rd = [&](int m) __attribute__((always_inline)) -> bf16x8 {
                    return read_rows<D>(m < NKS ? Qb : Gb, 0, m % NKS, lane);
                };
                bf16x8 op[RA];
#pragma unroll
                for (int m = 0; m < RA; m++) op[m] = rd(m);
#pragma unroll
                for (int m = 0; m < NM; m++) {
                    const bf16x8 x = op[m % RA];
                    if (m + RA < NM) op[m % RA] = rd(m + RA);
                    if (m < NKS) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, kf[m], s, 0, 0, 0);
                    else dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, vf[m - NKS], dp, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // P and dS (masked pairs give exactly 0); the mask is applied only
            // on the tiles that need it (a wave-uniform branch between two
            // versions of the loop)
            const bool need_mask = (qbase + BQB > Lq) || (kw0 + 32 > Lk) || (CAUSAL && kw0 + 31 > qbase + diag);
            uint32_t pp[8], pd[8];
            auto probs = [&](auto masked) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    // rows 8j + 4*(lane/32) + 0..3 of the tile
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(Sb + 8 * j + 4 * (lane >> 5));
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(Sb + 32 + 8 * j + 4 * (lane >> 5));
                    float pv[4], dv4[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int r = 4 * j + e;
                        const float p = fast_exp2(s[r] * sl2 - l4[e]);
                        pv[e] = p;
                        dv4[e] = p * (dp[r] - d4[e]);
                        if (MASKED) {
                            const int qi = qbase + 8 * j + 4 * (lane >> 5) + e;
                            const bool vis = qi < Lq && my_key < Lk && (!CAUSAL || my_key <= qi + diag);
                            if (!vis) pv[e] = dv4[e] = 0.f;
                        }
                    }
                    pp[2 * j] = pack_bf16x2(pv[0], pv[1]);
                    pp[2 * j + 1] = pack_bf16x2(pv[2], pv[3]);
                    pd[2 * j] = pack_bf16x2(dv4[0], dv4[1]);
                    pd[2 * j + 1] = pack_bf16x2(dv4[2], dv4[3]);
                }
            };
            if (need_mask) probs(std::true_type{});
            else probs(std::false_type{});
            // dV^T += dO^T P and dK^T += Q^T dS, 16 query rows per MMA
            {
                // MMA n: m = n / (2 NDC), dc = n / 2 % NDC, dV (even n) or dK (odd n)
                constexpr int NM = 4 * NDC, RA = 2;
                auto rd = [&](int n) __attribute__((always_inline)) -> bf16x8 {
                    return read_cols<D>(n & 1 ? Qb : Gb, n / (2 * NDC), dc0 + n / 2 % NDC, lane);
                };
                bf16x8 op[RA];
#pragma unroll
                for (int n = 0; n < RA; n++) op[n] = rd(n);
#pragma unroll
                for (int n = 0; n < NM; n++) {
                    const bf16x8 x = op[n % RA];
                    if (n + RA < NM) op[n % RA] = rd(n + RA);
                    const int m = n / (2 * NDC), dc = n / 2 % NDC;
                    if (n & 1) dk[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, packed_b(pd, m), dk[dc], 0, 0, 0);
                    else dv[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, packed_b(pp, m), dv[dc], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        for (int t = 0; t < ntiles; t += 2) {
            tile(t, q_lds0, g_lds0, st_lds0, q_lds1, g_lds1, st_lds1);
            if (t + 1 < ntiles) tile(t + 1, q_lds1, g_lds1, st_lds1, q_lds0, g_lds0, st_lds0);
        }
        if (my_key < Lk) {
            const int64_t row = ((int64_t)(k0 + my_key) * Hkv + kh) * D + 32 * dc0;
            store_rows_T<NDC>(a.dk + row, dk, a.scale, lane);
            store_rows_T<NDC>(a.dv + row, dv, 1.f, lane);
        }
    }
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs &a, bool causal, int num_cus, hipStream_t stream)
{
    BwdArgs ak = a;
    ak.n_items_k *= bwd_dkv_split<D>();  // items per (block, kv head) d range
    const int64_t slots_q = (int64_t)num_cus * (D == 256 ? 1 : 2), slots_k = (int64_t)num_cus * (D == 64 ? 2 : 1);
    const dim3 gq((unsigned)(a.n_items_q < slots_q ? a.n_items_q : slots_q));
    const dim3 gk((unsigned)(ak.n_items_k < slots_k ? ak.n_items_k : slots_k));
    if (a.n_items_q > 0) {
        if (causal) hipLaunchKernelGGL((varlen_bwd_dq_kernel<D, true>), gq, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((varlen_bwd_dq_kernel<D, false>), gq, dim3(256), 0, stream, a);
    }
    if (ak.n_items_k > 0) {
        if (causal) hipLaunchKernelGGL((varlen_bwd_dkv_kernel<D, true>), gk, dim3(256), 0, stream, ak);
        else hipLaunchKernelGGL((varlen_bwd_dkv_kernel<D, false>), gk, dim3(256), 0, stream, ak);
    }
    return hipGetLastError();
}

hipError_t launch_varlen_bwd(const BwdArgs &a, bool causal, int num_cus, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_bwd_d<64>(a, causal, num_cus, stream);
    case 128: return launch_bwd_d<128>(a, causal, num_cus, stream);
    case 256: return launch_bwd_d<256>(a, causal, num_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rra
