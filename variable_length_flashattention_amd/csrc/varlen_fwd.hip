// Variable-length (packed, cu_seqlens) attention forward for gfx950.
//
// Method: "Varlen Flash Attention Implementation Plan", Task 1 (the online
// softmax over key tiles: running row max m and denominator l in fp32,
// rescaling of the accumulator, out = acc / l, lse = m + ln l).  The work
// decomposition, tile shapes and data movement here are this library's own.
//
// One workgroup of NW waves owns a work item (sequence b, query tile qt,
// head h) of BQ = 32*NW query rows; each wave owns a 32-row block of the tile.
// Key tiles of BK keys are staged global->LDS with direct-to-LDS loads,
// NBUF-deep so that loads run ahead of the compute.  Per key tile each wave
//   S^T[key][query] = K . Q^T          (v_mfma_f32_32x32x16_bf16, Q in VGPRs)
//   masks the tail and the causal diagonal (bottom-right: j <= i + Lk - Lq),
//   updates m and l (exp2 with log2(e) folded into the scale; l sums the fp32
//   probabilities, the MMA takes them rounded to bf16),
//   O^T[d][query] += V^T . P^T         (V^T read with ds_read_b64_tr_b16).
// The S^T orientation puts one query per lane column, so row statistics are
// lane-local plus one permlane32 swap, and P^T feeds the second MMA straight
// from the accumulator registers.  Key tiles past the last visible key of a
// causal tile are never loaded.
#include "rra_device.h"
#include "rra_internal.h"
#include "tile_map.h"

namespace rra {

template <int D, int NW>
struct VarlenTile {
    static constexpr int BQ = 32 * NW;
    static constexpr int BK = D <= 128 ? 64 : 32;
    static constexpr int ROWB = D * 2;                 // bytes per K/V row
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int TILE_BYTES = BK * ROWB;       // one K (or V) tile
    static constexpr int WAVE_LOADS = TILE_BYTES / 1024 / NW;  // 1 KiB direct-to-LDS loads per wave per tensor
    static_assert(WAVE_LOADS * 1024 * NW == TILE_BYTES, "tile must split evenly over the waves");
    // K/V buffers: two tiles, so that two workgroups fit in one CU's LDS
    // (deeper pipelines at one workgroup per CU measured slower)
    static constexpr int NBUF = 2;
    static constexpr int LDS_BYTES = NBUF * 2 * TILE_BYTES;
    static constexpr int LDS_INTS = LDS_BYTES / 4;
    // XOR swizzles of the 16-byte chunks of a row (LDS has 32 banks of 4 B):
    // K is read as 16-byte row pieces of 32 consecutive rows (ds_read_b128),
    // V as 4 rows x 32 bytes per 16 lanes (ds_read_b64_tr_b16).
    __device__ static int swz_k(int row) { return row & (CPR < 16 ? CPR - 1 : 15); }
    __device__ static int swz_v(int row) { return 2 * (row & 3); }
    __device__ static int row_block(int w) { return w; }
    static constexpr int THREADS = 64 * NW;
    static constexpr int MIN_BLOCKS = D <= 128 ? 2 : 1;
};

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__((VarlenTile<D, NW>::THREADS), (VarlenTile<D, NW>::MIN_BLOCKS)) void varlen_fwd_kernel(VarlenArgs a)
{
    using T = VarlenTile<D, NW>;
    constexpr int BQ = T::BQ, BK = T::BK, ROWB = T::ROWB, TB = T::TILE_BYTES, NBUF = T::NBUF;
    constexpr int NC = BK / 32;          // 32-key accumulator tiles per key tile
    constexpr int NKS = D / 16;          // k-steps of the QK^T MMA
    constexpr int NDC = D / 32;          // 32-wide d chunks of the output
    // K and V tiles, two buffers each, as distinct LDS objects: the compiler
    // then knows a read of one buffer does not depend on direct-to-LDS loads
    // still in flight into the other, and does not wait for them.
    static_assert(NBUF == 2, "the tile loop below alternates two buffers");
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TB];
    __shared__ int sched[kSchedInts];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.num_heads;
    const float sl2 = a.scale_log2;
    const int rb = T::row_block(wave);
    const WorkTables wt = build_work_tables(a.cu_q, a.cu_k, a.batch, BQ, a.levels, sched, kSchedInts);

    // persistent workgroups: items are dealt out in serpentine order
    for (int64_t k = 0;; k++) {
        const int64_t w = serpentine_item(k, blockIdx.x, gridDim.x);
        if (w >= a.n_items) break;
        int b, qt, h;
        if (!decode_work_item(wt, a.cu_q, H, w, lane, b, qt, h)) break;  // the same in every wave
        __syncthreads();  // LDS buffers of the previous item no longer in use

        const int *cuq = wt.cached ? wt.cuq : a.cu_q, *cuk = wt.cached ? wt.cuk : a.cu_k;
        const int q0 = cuq[b], k0 = cuk[b];
        const int Lq = cuq[b + 1] - q0, Lk = cuk[b + 1] - k0;
        const int diag = Lk - Lq;  // causal: key j visible to query i iff j <= i + diag
        const int i0 = qt * BQ;
        const int nrows = min(BQ, Lq - i0);
        const int iw = i0 + 32 * rb;           // first row of this wave
        const int my_i = iw + (lane & 31);
        const bool row_ok = my_i < Lq;
        int kend = Lk, kend_w = Lk;
        if (CAUSAL) {
            kend = max(0, min(Lk, i0 + nrows + diag));
            kend_w = max(0, min(Lk, min(iw + 31, Lq - 1) + 1 + diag));
        }
        if (32 * rb >= nrows) kend_w = 0;
        const int nkt = (kend + BK - 1) / BK;
        const int nkt_w = (kend_w + BK - 1) / BK;

        // Direct-to-LDS staging of key tile kt into buffer kt % NBUF.  Wave w
        // fills 1 KiB blocks w, w+NW, ... of each tensor; lane l of a block
        // writes the 16 bytes at block*1024 + 16*l, i.e. row r, physical
        // chunk p, which holds logical chunk p ^ swz(r).  Rows past the
        // sequence end re-read its last row (their scores are masked and
        // their probabilities are exactly 0).
        auto stage = [&](int kt, uint8_t *kb, uint8_t *vb) {
#pragma unroll
            for (int i = 0; i < T::WAVE_LOADS; i++) {
                const int blk = i * NW + wave;
                const int byte = blk * 1024 + lane * 16;
                const int row = byte / ROWB, pch = (byte % ROWB) / 16;
                const int tok = k0 + min(kt * BK + row, Lk - 1);
                const int64_t off = ((int64_t)tok * H + h) * D;
                // (the sources go through named locals: with the address
                // expression inline as the builtin's argument, the host pass
                // silently dropped the kernel's launch stub)
                const uint16_t *ksrc = a.k + off + 8 * (pch ^ T::swz_k(row));
                const uint16_t *vsrc = a.v + off + 8 * (pch ^ T::swz_v(row));
                __builtin_amdgcn_global_load_lds(ksrc, (__attribute__((address_space(3))) void *)(kb + blk * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vsrc, (__attribute__((address_space(3))) void *)(vb + blk * 1024), 16, 0, 0);
            }
        };

        // Q^T operand: lane holds Q[my_i][16*ks + 8*(lane/32) .. +7]
        bf16x8 qf[NKS];
        {
            const uint16_t *qrow = a.q + ((int64_t)(q0 + my_i) * H + h) * D + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (row_ok) x = load16(qrow + 16 * ks);
                qf[ks] = as_bf16x8(x);
            }
        }
        f32x16 o[NDC];
#pragma unroll
        for (int dc = 0; dc < NDC; dc++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[dc][r] = 0.f;
        // m_ref: the max the accumulators are currently scaled to; it is only
        // raised when a row max exceeds it by more than 2^8 in probability
        // (probabilities stay <= 256, far inside fp32/bf16 range), which
        // skips most rescales of O.
        float m_ref = -INFINITY, l_run = 0.f;

        if (nkt > 0) stage(0, k_lds0, v_lds0);
        // one key tile; tile kt lives in buffer kt & 1
        auto tile = [&](int kt, const uint8_t *Kb, const uint8_t *Vb, uint8_t *kn, uint8_t *vn) {
            const int kbase = kt * BK;
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of tile kt
            __syncthreads();  // tile kt visible; every wave is done with tile kt-1
            if (kt + 1 < nkt) stage(kt + 1, kn, vn);
            if (kt >= nkt_w) return;

            // S^T = K Q^T
            f32x16 s[NC];
#pragma unroll
            for (int c = 0; c < NC; c++) {
#pragma unroll
                for (int r = 0; r < 16; r++) s[c][r] = 0.f;
                const int row = 32 * c + (lane & 31);
                const uint8_t *kp = Kb + row * ROWB;
                const int sw = T::swz_k(row);
#pragma unroll
                for (int ks = 0; ks < NKS; ks++) {
                    const int ch = (2 * ks + (lane >> 5)) ^ sw;
                    const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4 *>(kp + 16 * ch));
                    s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[c], 0, 0, 0);
                }
            }
            // tail and causal masks (only tiles that need them)
            const bool need_mask = (kbase + BK > Lk) || (CAUSAL && kbase + BK - 1 > iw + diag);
            if (need_mask) {
                const int last = CAUSAL ? min(Lk - 1, my_i + diag) : Lk - 1;
#pragma unroll
                for (int c = 0; c < NC; c++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int key = kbase + 32 * c + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        if (key > last) s[c][r] = -INFINITY;
                    }
            }
            // online softmax (row = this lane's query; lanes l and l^32 share it)
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < NC; c++)
#pragma unroll
                for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[c][r], s[c][r + 1]);
            mx = max_across_halves(mx);
            const bool raise = mx > m_ref && (m_ref == -INFINITY || (mx - m_ref) * sl2 > 8.f);
            if (__builtin_amdgcn_ballot_w64(raise)) {
                const float m_new = fmaxf(m_ref, mx);
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_ref - m_new) * sl2);
                l_run *= alpha;
#pragma unroll
                for (int dc = 0; dc < NDC; dc++)
#pragma unroll
                    for (int r = 0; r < 16; r++) o[dc][r] *= alpha;
                m_ref = m_new;
            }
            const float mc = (m_ref == -INFINITY ? 0.f : m_ref) * sl2;
            uint32_t pk[NC][8];
            float rs = 0.f;
#pragma unroll
            for (int c = 0; c < NC; c++)
#pragma unroll
                for (int r2 = 0; r2 < 8; r2++) {
                    const float p0 = fast_exp2(fmaf(s[c][2 * r2], sl2, -mc));
                    const float p1 = fast_exp2(fmaf(s[c][2 * r2 + 1], sl2, -mc));
                    pk[c][r2] = pack_bf16x2(p0, p1);
                    rs += p0 + p1;
                }
            l_run += sum_across_halves(rs);

            // O^T += V^T P^T, 16 keys per MMA
            const int g = lane >> 4, j = lane & 15;
#pragma unroll
            for (int m = 0; m < BK / 16; m++) {
                const u32x4 pb = {pk[m >> 1][4 * (m & 1) + 0], pk[m >> 1][4 * (m & 1) + 1],
                                  pk[m >> 1][4 * (m & 1) + 2], pk[m >> 1][4 * (m & 1) + 3]};
                const int row = 16 * m + 4 * (g >> 1) + (j >> 2);
                const int sw = T::swz_v(row);  // rows row and row+8 share it
                const uint8_t *v0 = Vb + row * ROWB + 8 * (j & 1);
#pragma unroll
                for (int dc = 0; dc < NDC; dc++) {
                    const int ch = (4 * dc + 2 * (g & 1) + ((j & 3) >> 1)) ^ sw;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v0 + 16 * ch));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v0 + 8 * ROWB + 16 * ch));
                    const u32x4 vv = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                      __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
                    o[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), as_bf16x8(pb), o[dc], 0, 0, 0);
                }
            }
        };
        for (int kt = 0; kt < nkt; kt += 2) {
            tile(kt, k_lds0, v_lds0, k_lds1, v_lds1);
            if (kt + 1 < nkt) tile(kt + 1, k_lds1, v_lds1, k_lds0, v_lds0);
        }

        // epilogue: out = O / l (0 when no key is visible), lse = scale*m + ln l (-inf then)
        if (row_ok) {
            const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
            uint16_t *orow = a.out + ((int64_t)(q0 + my_i) * H + h) * D + 4 * (lane >> 5);
#pragma unroll
            for (int dc = 0; dc < NDC; dc++)
#pragma unroll
                for (int rb4 = 0; rb4 < 4; rb4++) {
                    const u32x2 pr = {pack_bf16x2(o[dc][4 * rb4] * inv_l, o[dc][4 * rb4 + 1] * inv_l),
                                      pack_bf16x2(o[dc][4 * rb4 + 2] * inv_l, o[dc][4 * rb4 + 3] * inv_l)};
                    *reinterpret_cast<u32x2 *>(orow + 32 * dc + 8 * rb4) = pr;
                }
            if (lane < 32)
                a.lse[(int64_t)(q0 + my_i) * H + h] = l_run > 0.f ? a.scale * m_ref + logf(l_run) : -INFINITY;
        }
    }
}

// Test hook: the same work tables and decoder, one wave per workgroup.
__global__ __launch_bounds__(64) void varlen_tile_map_kernel(const int32_t *cu_q, const int32_t *cu_k, int32_t batch,
                                                             int32_t num_heads, int32_t block_q, int32_t levels,
                                                             int64_t n_items, int32_t *items)
{
    __shared__ int sched[kSchedInts];
    const int lane = threadIdx.x;
    const WorkTables wt = build_work_tables(cu_q, cu_k, batch, block_q, levels, sched, kSchedInts);
    for (int64_t w = blockIdx.x; w < n_items; w += gridDim.x) {
        int b = -1, qt = -1, h = -1;
        const bool ok = decode_work_item(wt, cu_q, num_heads, w, lane, b, qt, h);
        if (lane == 0) {
            items[3 * w + 0] = ok ? b : -1;
            items[3 * w + 1] = ok ? qt : -1;
            items[3 * w + 2] = ok ? h : -1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template <int D, int NW>
static hipError_t launch_d(const VarlenArgs &a, bool causal, int num_cus, hipStream_t stream)
{
    // persistent grid: as many workgroups as fit on the device at once
    const int64_t slots = (int64_t)num_cus * VarlenTile<D, NW>::MIN_BLOCKS;
    const dim3 grid((unsigned)(a.n_items < slots ? a.n_items : slots)), block(64 * NW);
    if (causal) hipLaunchKernelGGL((varlen_fwd_kernel<D, true, NW>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((varlen_fwd_kernel<D, false, NW>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_varlen_fwd(const VarlenArgs &a, int head_dim, bool causal, int num_cus, hipStream_t stream)
{
    if (a.block_q != 32 * 4) return hipErrorInvalidValue;
    switch (head_dim) {
    case 64: return launch_d<64, 4>(a, causal, num_cus, stream);
    case 128: return launch_d<128, 4>(a, causal, num_cus, stream);
    case 256: return launch_d<256, 4>(a, causal, num_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_varlen_tile_map(const int32_t *cu_q, const int32_t *cu_k, int32_t batch, int32_t num_heads,
                                  int32_t block_q, int32_t levels, int64_t n_items, int32_t *items_out,
                                  hipStream_t stream)
{
    const unsigned grid = (unsigned)(n_items < 1024 ? n_items : 1024);
    hipLaunchKernelGGL(varlen_tile_map_kernel, dim3(grid), dim3(64), 0, stream, cu_q, cu_k, batch, num_heads, block_q,
                       levels, n_items, items_out);
    return hipGetLastError();
}

}  // namespace rra
