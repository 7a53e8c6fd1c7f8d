// Variable-length (packed, cu_seqlens) attention forward for gfx950.
//
// Method: "Varlen Flash Attention Implementation Plan", Task 1 (the online
// softmax over key tiles: running row max m and denominator l in fp32,
// rescaling of the accumulator, out = acc / l, lse = m + ln l).  Grouped-query
// attention reads kv head h / (H / Hkv) for query head h, the grouping of
// step_tile_ref in "spark_storage/attention_ref.rs"; heads are innermost in
// the work list, so the query heads of one kv head run side by side and share
// its K/V in L2.  The work decomposition, tile shapes and data movement here
// are this library's own.
//
// One workgroup of NW waves owns a work item (sequence b, query tile qt,
// head h) of BQ = 32*NW query rows; each wave owns a 32-row block of the tile.
// Key tiles of BK keys are staged global->LDS with direct-to-LDS loads,
// double-buffered so that loads run ahead of the compute.  Per key tile each wave
//   S^T[key][query] = K . Q^T          (v_mfma_f32_32x32x16_bf16, Q in VGPRs)
//   masks the tail and the causal diagonal (bottom-right: j <= i + Lk - Lq),
//   updates m and l (exp2 with log2(e) folded into the scale; the MMA takes
//   the probabilities rounded to bf16, and the row sums are kept twice: of
//   the fp32 probabilities for lse, and of the bf16 values the MMA takes for
//   the normalisation of out, so that out is an exact convex combination of
//   the rows of V with the weights the MMA used),
//   O^T[d][query] += V^T . P^T         (V^T read with ds_read_b64_tr_b16).
// The S^T orientation puts one query per lane column, so row statistics are
// lane-local plus one permlane32 swap, and P^T feeds the second MMA straight
// from the accumulator registers.  Key tiles past the last visible key of a
// causal tile are never loaded.
//
// Paged keys and values (chunked prefill; PAGED): k and v are pools of
// BS-token blocks and key j of sequence b is slot j % BS of block
// block_table[b, j / BS], the addressing of step_tile_ref.  Each 1 KiB
// direct-to-LDS load covers 1024 / (2D) consecutive keys, which lie in one
// block when BS >= 8, so a load keeps one scalar buffer descriptor, based at
// its first key's pool row; the table entries of a key tile are fetched
// one per lane a tile ahead and picked with readlane.
#include "rra_device.h"
#include "rra_internal.h"
#include "tile_map.h"

namespace rra {

template <int D>
struct VarlenTile {
    static constexpr int NW = 4;                       // waves per workgroup
    static constexpr int BQ = 32 * NW;                 // query rows per work item (32 per wave)
    static constexpr int BK = varlen_block_k(D);
    static constexpr int NBUF = 2;                     // K/V tile buffers (one in flight, one in use)
    static constexpr int ROWB = D * 2;                 // bytes per K/V row
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int TILE_BYTES = BK * ROWB;       // one K (or V) tile
    static constexpr int WAVE_LOADS = TILE_BYTES / 1024 / NW;  // 1 KiB direct-to-LDS loads per wave per tensor
    static_assert(WAVE_LOADS * 1024 * NW == TILE_BYTES, "tile must split evenly over the waves");
    // XOR swizzles of the 16-byte chunks of a row (LDS has 32 banks of 4 B):
    // K is read as 16-byte row pieces of 32 consecutive rows (ds_read_b128),
    // V as 4 rows x 32 bytes per 16 lanes (ds_read_b64_tr_b16).
    __device__ static int swz_k(int row) { return row & (CPR < 16 ? CPR - 1 : 15); }
    __device__ static int swz_v(int row) { return 2 * (row & 3); }
    static constexpr int THREADS = 64 * NW;
    // workgroups per CU: three at head_dim 64, two at 128 (256 VGPRs each),
    // one at 256
    static constexpr int MIN_BLOCKS = D == 64 ? 3 : D == 128 ? 2 : 1;
};

// SORTED: the work list orders the sequences of a level by length (the
// work-list tables sort them at the kernel's start).
template <int D, bool CAUSAL, bool PAGED, bool SORTED>
__global__ __launch_bounds__((VarlenTile<D>::THREADS), (VarlenTile<D>::MIN_BLOCKS)) void varlen_fwd_kernel(VarlenArgs a)
{
    using T = VarlenTile<D>;
    constexpr int NW = T::NW, BQ = T::BQ, BK = T::BK, ROWB = T::ROWB, TB = T::TILE_BYTES;
    constexpr int NC = BK / 32;          // 32-key accumulator tiles per key tile
    constexpr int NKS = D / 16;          // k-steps of the QK^T MMA
    constexpr int NDC = D / 32;          // 32-wide d chunks of the output
    // Two K/V buffers: each tile waits for every load issued before it (its
    // own tile, and in paged mode the table fetch for the next) at its top.
    static_assert(T::NBUF == 2, "the staging assumes two buffers");
    // K and V tiles, two buffers each, as distinct LDS objects: the compiler
    // then knows a read of one buffer does not depend on direct-to-LDS loads
    // still in flight into another, and does not wait for them.
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TB];

    __shared__ int sched[kSchedInts];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.num_heads;
    const float sl2 = a.scale_log2;
    const int32_t *kcount = PAGED ? a.seqlens_k : a.cu_k;  // per-sequence key counts, or key offsets
    const WorkTables wt = build_work_tables(a.cu_q, kcount, PAGED ? a.batch : a.batch + 1, a.batch, BQ,
                                            SORTED ? BK : 0, a.levels, sched, kSchedInts);

    // Output stores.  The accumulators hold O^T, 4 consecutive d of one query
    // per register quad, so stores straight from them would write 8-byte
    // pieces of 32 rows per instruction.  Instead each wave writes its rows
    // (bf16) to a private LDS slot and reads them back so that consecutive
    // lanes hold consecutive 16-byte pieces of a row: every store then writes
    // whole 128-d row segments.  NST store instructions go out per item (lanes
    // with nothing to store get an offset past the buffer's range, and the
    // hardware drops those writes).
    // At head_dim <= 128 the slots are in the K/V buffer the item's last tile
    // did not use, and the rows are stored at once.  At head_dim 256 they do
    // not fit there; the slots are an array of their own, and the stores are
    // held back until the next item's first loads are issued: the load/store
    // counter retires in order, so stores issued before those loads would
    // have to be written out before the next item's first key tile could
    // start, and with a constant NST the wait there can leave exactly the NST
    // youngest operations in flight.  (Holding back at head_dim <= 128 needs
    // the slots in the second buffer, and with an even number of tiles a
    // barrier before writing them: measured slower on gfx950 than storing at
    // once, while at head_dim 256 holding back is 5 % faster.)
    constexpr int CW = D < 128 ? D : 128;  // d columns per row segment
    constexpr int RB = D * 2;              // slot bytes per row
    constexpr int CHR = CW / 8;            // 16-byte chunks per row segment
    constexpr int SLOT = 32 * RB;
    constexpr int RPI = 64 / CHR;          // rows per read (and store) instruction
    constexpr int NPASS = D / CW, NRD = 32 / RPI;
    constexpr int NST = NPASS * NRD + 1;   // store instructions per item: out rows, then lse
    constexpr bool DEFER = 2 * SLOT > TB;  // own slots, stores held back to the next item
    __shared__ __attribute__((aligned(1024))) uint8_t o_lds[DEFER ? NW * SLOT : 16];
    constexpr uint32_t kDrop = 0x80000000u;  // a buffer offset past the range: the write is dropped
    float pend_lse_v = 0.f;
    uint16_t *pend_out = a.out;
    float *pend_lse = a.lse;
    int pend_n = 0;  // rows of the block to store (0: nothing)
    // chunk c of a slot row r sits at physical chunk c ^ (r & 7): the 8-byte
    // writes (32 rows, one chunk) and the 16-byte reads (RPI rows) are then
    // spread evenly over the banks
    auto flush_from = [&](const uint8_t *slot) __attribute__((always_inline)) {
        int lid = lane;
        __asm__ volatile("" : "+v"(lid));
        const __amdgpu_buffer_rsrc_t ob = raw_buffer(pend_out), lb = raw_buffer(pend_lse);
        const uint32_t rstride = (uint32_t)H * D * 2;
        // all slot reads first, then the stores (one LDS round trip, not one per store)
        u32x4 val[NPASS][NRD];
#pragma unroll
        for (int p = 0; p < NPASS; p++)
#pragma unroll
            for (int i = 0; i < NRD; i++) {
                const int r = i * RPI + lid / CHR, c = p * CHR + lid % CHR;
                val[p][i] = *reinterpret_cast<const u32x4 *>(slot + r * RB + 16 * (c ^ (r & 7)));
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NPASS; p++)
#pragma unroll
            for (int i = 0; i < NRD; i++) {
                const int r = i * RPI + lid / CHR, c = p * CHR + lid % CHR;
                const uint32_t off = r < pend_n ? r * rstride + 16 * c : kDrop;
                __builtin_amdgcn_raw_buffer_store_b128(val[p][i], ob, off, 0, 0);
            }
        const uint32_t loff = (lid < 32 && lid < pend_n) ? (uint32_t)(lid * H * 4) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pend_lse_v), lb, loff, 0, 0);
    };

    // persistent workgroups: items are dealt out in serpentine order
    for (int64_t k = 0;; k++) {
        const int64_t w = serpentine_item(k, blockIdx.x, gridDim.x);
        if (w >= a.n_items) break;
        int b, qt, h;
        if (!decode_work_item(wt, a.cu_q, H, w, lane, b, qt, h)) break;  // the same in every wave
        __syncthreads();  // LDS buffers of the previous item no longer in use

        // (the item's indices are the same in every lane; saying so keeps the
        // per-item arithmetic and the buffer descriptors scalar)
        b = __builtin_amdgcn_readfirstlane(b);
        qt = __builtin_amdgcn_readfirstlane(qt);
        h = __builtin_amdgcn_readfirstlane(h);
        const int *cuq = wt.cached ? wt.cuq : a.cu_q, *cuk = wt.cached ? wt.cuk : kcount;
        const int q0 = __builtin_amdgcn_readfirstlane(cuq[b]);
        const int Lq = __builtin_amdgcn_readfirstlane(cuq[b + 1]) - q0;
        int k0, Lk;
        if constexpr (PAGED) {
            k0 = 0;
            Lk = min(max(__builtin_amdgcn_readfirstlane(cuk[b]), 0), a.max_blocks << a.bs_shift);
        } else {
            k0 = __builtin_amdgcn_readfirstlane(cuk[b]);
            Lk = __builtin_amdgcn_readfirstlane(cuk[b + 1]) - k0;
        }
        const int diag = Lk - Lq;  // causal: key j visible to query i iff j <= i + diag
        const int i0 = qt * BQ;
        const int nrows = min(BQ, Lq - i0);
        int kend = Lk;
        if (CAUSAL) kend = max(0, min(Lk, i0 + nrows + diag));
        const int nkt = (kend + BK - 1) / BK;

        // This wave owns rows i0 + 32*wave + lane%32 and needs key tiles 0..nkt_w-1.
        const int iw = i0 + 32 * wave;
        const int my_i = iw + (lane & 31);
        int kend_w = Lk;
        if (CAUSAL) kend_w = max(0, min(Lk, min(iw + 31, Lq - 1) + 1 + diag));
        if (32 * wave >= nrows) kend_w = 0;
        const int nkt_w = (kend_w + BK - 1) / BK;

        // Direct-to-LDS staging of key tile kt with buffer loads: the tile's
        // first row is the buffer base (64-bit, scalar), each load adds a
        // uniform row offset (scalar) to a per-lane offset (vector) that does
        // not change from tile to tile, so a tile costs no vector address
        // arithmetic.  Wave w fills 1 KiB blocks w, w+NW, ... of each tensor;
        // lane l of a block writes the 16 bytes at block*1024 + 16*l, i.e. row
        // r, physical chunk p, which holds logical chunk p ^ swz(r).  In the
        // sequence's last tile, rows past its end re-read its last row (their
        // scores are masked and their probabilities are exactly 0).
        constexpr int WL = T::WAVE_LOADS;
        constexpr int RPL = NW * 1024 / ROWB;        // rows between a lane's loads
        constexpr int NKO = RPL % 16 == 0 ? 1 : 16 / RPL;  // distinct K swizzles over the loads
        static_assert(RPL % 4 == 0 && (RPL % 16 == 0 || 16 % RPL == 0), "swizzle period");
        const int srow0 = (wave * 1024 + lane * 16) / ROWB, pch = (lane * 16 % ROWB) / 16;
        const int row_bytes = a.num_kv_heads * D * 2;  // bytes from one K/V token to the next
        uint32_t lane_k[NKO];
#pragma unroll
        for (int j = 0; j < NKO; j++)
            lane_k[j] = (uint32_t)(srow0 * row_bytes + 16 * (pch ^ T::swz_k(srow0 + j * RPL)));
        const uint32_t lane_v = (uint32_t)(srow0 * row_bytes + 16 * (pch ^ T::swz_v(srow0)));
        const int kh = h / a.gqa_ratio;  // the kv head of query head h
        const uint8_t *kseq = reinterpret_cast<const uint8_t *>(a.k + ((int64_t)k0 * a.num_kv_heads + kh) * D);
        const uint8_t *vseq = reinterpret_cast<const uint8_t *>(a.v + ((int64_t)k0 * a.num_kv_heads + kh) * D);
        // paged: a load's keys are rows lrow of a 1 KiB piece that starts at
        // tile row (i*NW + wave) * RPB; the per-lane offsets hold lrow and
        // the swizzled chunk, the descriptor the piece's first pool row
        constexpr int RPB = 1024 / ROWB;
        const int lrow = lane * 16 / ROWB;
        uint32_t plane_k[NKO];
#pragma unroll
        for (int j = 0; j < NKO; j++)
            plane_k[j] = (uint32_t)(lrow * row_bytes + 16 * (pch ^ T::swz_k(srow0 + j * RPL)));
        const uint32_t plane_v = (uint32_t)(lrow * row_bytes + 16 * (pch ^ T::swz_v(srow0)));
        // paged, blocks of at least KPW keys: wave w stages the tile's pieces
        // w*WL .. w*WL+WL-1 instead, i.e. keys KPW*w .. KPW*w+KPW-1, which lie in
        // one pool block: one table entry and one descriptor per tile, and per
        // piece a per-lane offset holding the key's row past the wave's first
        // key and the swizzled chunk
        constexpr int KPW = WL * RPB;
        const bool one_block = PAGED && (1 << a.bs_shift) >= KPW;
        uint32_t wk[PAGED ? WL : 1], wv[PAGED ? WL : 1];
        if constexpr (PAGED) {
#pragma unroll
            for (int i = 0; i < WL; i++) {
                const int lr = i * RPB + lrow, trow = wave * KPW + lr;
                wk[i] = (uint32_t)(lr * row_bytes + 16 * (pch ^ T::swz_k(trow)));
                wv[i] = (uint32_t)(lr * row_bytes + 16 * (pch ^ T::swz_v(trow)));
            }
        }
        const int32_t *table = PAGED ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
        const int last_blk = PAGED ? (Lk - 1) >> a.bs_shift : 0;
        // lane j holds the table entry of block (tile's first block + j),
        // clamped to the sequence's last block
        auto fetch_table = [&](int kt) __attribute__((always_inline)) -> int {
            return table[min(((kt * BK) >> a.bs_shift) + lane, last_blk)];
        };
        int tab = 0;
        if (PAGED && Lk > 0) tab = fetch_table(0);
        auto stage_paged = [&](int kt, uint8_t *kb, uint8_t *vb) __attribute__((always_inline)) {
            const int kbase = kt * BK;
            const int blk0 = kbase >> a.bs_shift;
            const int cur = tab;
            if (kt + 1 < nkt) tab = fetch_table(kt + 1);  // the next tile's, a tile ahead
            if (one_block) {
                const int r0 = min(kbase + wave * KPW, Lk - 1);  // the wave's first key (the last key past the end)
                const int ent = __builtin_amdgcn_readlane(cur, (r0 >> a.bs_shift) - blk0);
                const int64_t prow = ((int64_t)ent << a.bs_shift) + (r0 & ((1 << a.bs_shift) - 1));
                const int64_t off = (prow * a.num_kv_heads + kh) * ROWB;
                const __amdgpu_buffer_rsrc_t kr = raw_buffer(reinterpret_cast<const uint8_t *>(a.k) + off);
                const __amdgpu_buffer_rsrc_t vr = raw_buffer(reinterpret_cast<const uint8_t *>(a.v) + off);
                const int lim = Lk - 1 - r0;  // keys past r0 + lim re-read key r0 + lim
#pragma unroll
                for (int i = 0; i < WL; i++) {
                    const int lr = i * RPB + lrow;
                    const uint32_t back = lr > lim ? (uint32_t)((lr - lim) * row_bytes) : 0u;
                    buffer_to_lds16(kr, kb + (wave * WL + i) * 1024, wk[i] - back, 0);
                    buffer_to_lds16(vr, vb + (wave * WL + i) * 1024, wv[i] - back, 0);
                }
                return;
            }
#pragma unroll
            for (int i = 0; i < WL; i++) {
                const int piece = i * NW + wave;
                const int r = min(kbase + piece * RPB, Lk - 1);  // first key read (the last key past the end)
                const int ent = __builtin_amdgcn_readlane(cur, (r >> a.bs_shift) - blk0);
                const int64_t prow = ((int64_t)ent << a.bs_shift) + (r & ((1 << a.bs_shift) - 1));
                const int64_t off = (prow * a.num_kv_heads + kh) * ROWB;
                const __amdgpu_buffer_rsrc_t kr = raw_buffer(reinterpret_cast<const uint8_t *>(a.k) + off);
                const __amdgpu_buffer_rsrc_t vr = raw_buffer(reinterpret_cast<const uint8_t *>(a.v) + off);
                const int lim = Lk - 1 - r;  // keys of this piece past lim re-read key r + lim
                const uint32_t back = lrow > lim ? (uint32_t)((lrow - lim) * row_bytes) : 0u;
                const int blk = piece;
                buffer_to_lds16(kr, kb + blk * 1024, plane_k[i % NKO] - back, 0);
                buffer_to_lds16(vr, vb + blk * 1024, plane_v - back, 0);
            }
        };
        auto stage_packed = [&](int kt, uint8_t *kb, uint8_t *vb) __attribute__((always_inline)) {
            const int64_t toff = (int64_t)kt * BK * row_bytes;
            const __amdgpu_buffer_rsrc_t kr = raw_buffer(kseq + toff), vr = raw_buffer(vseq + toff);
            if ((kt + 1) * BK <= Lk) {
#pragma unroll
                for (int i = 0; i < WL; i++) {
                    const int blk = i * NW + wave;
                    buffer_to_lds16(kr, kb + blk * 1024, lane_k[i % NKO], i * RPL * row_bytes);
                    buffer_to_lds16(vr, vb + blk * 1024, lane_v, i * RPL * row_bytes);
                }
            } else {
                const int last_row = Lk - 1 - kt * BK;
#pragma unroll
                for (int i = 0; i < WL; i++) {
                    const int blk = i * NW + wave;
                    const int row = srow0 + i * RPL;
                    const uint32_t back = (uint32_t)((row - min(row, last_row)) * row_bytes);
                    buffer_to_lds16(kr, kb + blk * 1024, lane_k[i % NKO] - back, i * RPL * row_bytes);
                    buffer_to_lds16(vr, vb + blk * 1024, lane_v - back, i * RPL * row_bytes);
                }
            }
        };
        auto stage = [&](int kt, uint8_t *kb, uint8_t *vb) {
            if constexpr (PAGED) stage_paged(kt, kb, vb);
            else stage_packed(kt, kb, vb);
        };
        if (nkt > 0) stage(0, k_lds0, v_lds0);

        // Q^T operand: lane holds Q[my_i][16*ks + 8*(lane/32) .. +7]
        // (rows past the sequence end read its last row; their results are
        // never stored, and an unconditional load is not waited on at once)
        bf16x8 qf[NKS];
        {
            const int qr = min(my_i, Lq - 1);
            const uint16_t *qrow = a.q + ((int64_t)(q0 + qr) * H + h) * D + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) qf[ks] = as_bf16x8(load16(qrow + 16 * ks));
        }
        if constexpr (DEFER) {
            // the previous item's stores, behind this item's first loads
            __builtin_amdgcn_sched_barrier(0);
            flush_from(o_lds + wave * SLOT);
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x16 o[NDC];
#pragma unroll
        for (int dc = 0; dc < NDC; dc++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[dc][r] = 0.f;
        // m_ref: the max the accumulators are currently scaled to; it is only
        // raised when a tile's probabilities against it grow too large (a
        // lane's share of a row sum above 2^15), which skips most row-max
        // reductions and rescales of O.  l_run sums the fp32 probabilities
        // (for lse), l_mma the bf16 values the PV MMA takes (for out).
        float m_ref = -INFINITY, l_run = 0.f, l_mma = 0.f;

        // one key tile; tile kt lives in buffer kt % 2, and tile kt+1 is
        // staged into the buffer tile kt-1 used
        auto tile = [&](int kt, const uint8_t *Kb, const uint8_t *Vb, uint8_t *kn, uint8_t *vn) {
            const int kbase = kt * BK;
            // this wave's loads of tile kt are done (at the first tile, the
            // previous item's NST stores, issued last, may stay in flight)
            // (the builtin, unlike inline asm, is known to the compiler's own
            // wait placement, which then counts the first loads as done)
            if (DEFER && kt == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NST));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __syncthreads();  // tile kt visible; every wave is done with tile kt-1
            if (kt + 1 < nkt) stage(kt + 1, kn, vn);
            if (kt >= nkt_w) return;  // the wave's rows see no key of this tile

            // S^T = K Q^T
            f32x16 s[NC];
#pragma unroll
            for (int c = 0; c < NC; c++)
#pragma unroll
                for (int r = 0; r < 16; r++) s[c][r] = 0.f;
            // K fragments are read KD MMAs ahead of use; the scheduling
            // barriers keep the compiler from sinking the reads next to
            // their MMAs (it does that under register pressure, and each
            // MMA then waits out a full LDS latency).  In items of at most
            // 2048 visible keys the wave runs this phase at raised priority,
            // so that a SIMD shared with a wave in its softmax keeps issuing
            // these MMAs first; longer items run faster without it (measured
            // on gfx950: 16 x U[1,2048] causal 6 % faster with the raise,
            // 8192-key items 5 % faster without).
            if (nkt * BK <= 2048) __builtin_amdgcn_s_setprio(1);
            {
                constexpr int NM = NC * NKS, KD = 3;
                auto kread = [&](int m) -> bf16x8 {
                    const int c = m / NKS, ks = m % NKS;
                    const int row = 32 * c + (lane & 31);
                    const int ch = (2 * ks + (lane >> 5)) ^ T::swz_k(row);
                    return as_bf16x8(*reinterpret_cast<const u32x4 *>(Kb + row * ROWB + 16 * ch));
                };
                bf16x8 kf[KD];
#pragma unroll
                for (int m = 0; m < KD; m++) kf[m] = kread(m);
#pragma unroll
                for (int m = 0; m < NM; m++) {
                    const bf16x8 ka = kf[m % KD];
                    if (m + KD < NM) kf[m % KD] = kread(m + KD);
                    const int c = m / NKS, ks = m % NKS;
                    s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[c], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            uint32_t pk[NC][8];
            {
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
                // online softmax (row = this lane's query; lanes l and l^32 share it).
                // Probabilities are formed against the reference max m_ref without
                // looking at this tile's row max; the tile falls back to the
                // exact max (and rescales O and l) when a row has no reference
                // yet or this lane's share of the row sum exceeds 2^15 (every
                // probability then stays <= 2^15, far inside fp32/bf16 range).
                // l_run sums the fp32 probabilities (summing their bf16
                // roundings would cost lse up to ~2^-9 on rows with few keys);
                // l_mma sums the bf16 values, so that out = O / l_mma weighs
                // each V row by exactly what the MMA used (with the fp32 sum a
                // dominant weight above 1 would be off by its rounding, up to
                // 2^-9 |v|).
                // At head_dim >= 128 the scores go in chunks of 8 (8 independent
                // FMAs, then 8 independent exponentials) and the sums run in
                // 4 + 2 partial accumulators, so that a wave alone on its
                // SIMD's VALU is not held up by one long dependency chain; at
                // head_dim 64, where three workgroups share a CU's registers,
                // a pair at a time.
                float rb = 0.f;
                auto probs = [&](float mc) __attribute__((always_inline)) -> float {
                    if constexpr (D >= 128) {
                        float rs4[4], rb2[2] = {0.f, 0.f};
#pragma unroll
                        for (int q = 0; q < 2 * NC; q++) {
                            const int c = q >> 1, base = 8 * (q & 1);
                            float t[8];
#pragma unroll
                            for (int i = 0; i < 8; i++) t[i] = fmaf(s[c][base + i], sl2, -mc);
#pragma unroll
                            for (int i = 0; i < 8; i++) t[i] = fast_exp2(t[i]);
#pragma unroll
                            for (int i = 0; i < 4; i++) {
                                const uint32_t pair = pack_bf16x2(t[2 * i], t[2 * i + 1]);
                                pk[c][base / 2 + i] = pair;
                                rs4[i] = q == 0 ? t[2 * i] + t[2 * i + 1] : rs4[i] + (t[2 * i] + t[2 * i + 1]);
                                rb2[i & 1] = add_bf16x2(pair, rb2[i & 1]);
                            }
                        }
                        rb = rb2[0] + rb2[1];
                        return (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);
                    } else {
                        float rs = 0.f;
                        rb = 0.f;
#pragma unroll
                        for (int c = 0; c < NC; c++)
#pragma unroll
                            for (int r2 = 0; r2 < 8; r2++) {
                                const float p0 = fast_exp2(fmaf(s[c][2 * r2], sl2, -mc));
                                const float p1 = fast_exp2(fmaf(s[c][2 * r2 + 1], sl2, -mc));
                                pk[c][r2] = pack_bf16x2(p0, p1);
                                rs += p0 + p1;
                                rb = add_bf16x2(pk[c][r2], rb);
                            }
                        return rs;
                    }
                };
                float rs = 0.f;
                bool slow = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
                if (!slow) {
                    rs = probs(m_ref * sl2);
                    slow = __builtin_amdgcn_ballot_w64(!(rs <= 32768.f)) != 0;  // (also catches inf)
                }
                if (slow) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int c = 0; c < NC; c++)
#pragma unroll
                        for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[c][r], s[c][r + 1]);
                    mx = max_across_halves(mx);
                    const float m_new = fmaxf(m_ref, mx);
                    const float alpha =
                        (m_ref == -INFINITY || m_new == m_ref) ? 1.f : fast_exp2((m_ref - m_new) * sl2);
                    l_run *= alpha;
                    l_mma *= alpha;
#pragma unroll
                    for (int dc = 0; dc < NDC; dc++)
#pragma unroll
                        for (int r = 0; r < 16; r++) o[dc][r] *= alpha;
                    m_ref = m_new;
                    rs = probs((m_new == -INFINITY ? 0.f : m_new) * sl2);
                }
                l_run += sum_across_halves(rs);
                l_mma += sum_across_halves(rb);
            }

            // O^T += V^T P^T, 16 keys per MMA; V^T fragments (two transposed
            // reads each) read VD MMAs ahead of use
            const int g = lane >> 4, j = lane & 15;
            {
                constexpr int NM = (BK / 16) * NDC, VD = 3;
                auto vread = [&](int mm) -> u32x4 {
                    const int m = mm / NDC, dc = mm % NDC;
                    const int row = 16 * m + 4 * (g >> 1) + (j >> 2);
                    const int sw = T::swz_v(row);  // rows row and row+8 share it
                    const uint8_t *v0 = Vb + row * ROWB + 8 * (j & 1);
                    const int ch = (4 * dc + 2 * (g & 1) + ((j & 3) >> 1)) ^ sw;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v0 + 16 * ch));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v0 + 8 * ROWB + 16 * ch));
                    return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                 __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
                };
                u32x4 vf[VD];
#pragma unroll
                for (int mm = 0; mm < VD; mm++) vf[mm] = vread(mm);
#pragma unroll
                for (int mm = 0; mm < NM; mm++) {
                    const u32x4 vv = vf[mm % VD];
                    if (mm + VD < NM) vf[mm % VD] = vread(mm + VD);
                    const int m = mm / NDC, dc = mm % NDC;
                    const u32x4 pb = {pk[m >> 1][4 * (m & 1) + 0], pk[m >> 1][4 * (m & 1) + 1],
                                      pk[m >> 1][4 * (m & 1) + 2], pk[m >> 1][4 * (m & 1) + 3]};
                    o[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), as_bf16x8(pb), o[dc], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        if constexpr (DEFER) {
            // The first tile is peeled off the loop: the compiler waits for
            // every load and store in flight before a loop that uses registers
            // loaded ahead of it (the Q fragments), and that wait then comes
            // after the first tile, where the loads of the second are due
            // anyway, instead of holding the first tile up until the previous
            // item's stores are written.
            if (nkt > 0) {
                tile(0, k_lds0, v_lds0, k_lds1, v_lds1);
                for (int kt = 1; kt < nkt; kt += 2) {
                    tile(kt, k_lds1, v_lds1, k_lds0, v_lds0);
                    if (kt + 1 < nkt) tile(kt + 1, k_lds0, v_lds0, k_lds1, v_lds1);
                }
            }
        } else {
            for (int kt = 0; kt < nkt; kt += 2) {
                tile(kt, k_lds0, v_lds0, k_lds1, v_lds1);
                if (kt + 1 < nkt) tile(kt + 1, k_lds1, v_lds1, k_lds0, v_lds0);
            }
        }

        // epilogue: out = O / l_mma (0 when no key is visible), lse = scale*m + ln l_run (-inf then),
        // as bf16 rows in the wave's slot; chunk c of a slot row r sits at
        // physical chunk c ^ (r & 7), so that the 8-byte writes (32 rows, one
        // chunk) and the 16-byte reads (RPI rows) spread evenly over the banks
        auto to_slot = [&](uint8_t *slot) __attribute__((always_inline)) {
            int lid = lane;
            __asm__ volatile("" : "+v"(lid));
            const int wrow = lid & 31, half = lid >> 5;
            const float inv_l = l_run > 0.f ? 1.f / l_mma : 0.f;
#pragma unroll
            for (int dc = 0; dc < NDC; dc++)
#pragma unroll
                for (int rb4 = 0; rb4 < 4; rb4++) {
                    const u32x2 pr = {pack_bf16x2(o[dc][4 * rb4] * inv_l, o[dc][4 * rb4 + 1] * inv_l),
                                      pack_bf16x2(o[dc][4 * rb4 + 2] * inv_l, o[dc][4 * rb4 + 3] * inv_l)};
                    const int ch = (4 * dc + rb4) ^ (wrow & 7);
                    *reinterpret_cast<u32x2 *>(slot + wrow * RB + 16 * ch + 8 * half) = pr;
                }
        };
        pend_lse_v = l_run > 0.f ? a.scale * m_ref + logf(l_run) : -INFINITY;
        pend_out = a.out + ((int64_t)(q0 + iw) * H + h) * D;
        pend_lse = a.lse + (int64_t)(q0 + iw) * H + h;
        pend_n = max(0, min(32, nrows - 32 * wave));
        if constexpr (DEFER) {
            to_slot(o_lds + wave * SLOT);
        } else {
            // the K/V buffer the last tile, nkt - 1, did not use: no load is in
            // flight into it, and the next item stages into it only after the
            // barrier at the item's start
            uint8_t *kfree = (nkt & 1) ? k_lds1 : k_lds0, *vfree = (nkt & 1) ? v_lds1 : v_lds0;
            uint8_t *slot = ((wave & 2) ? vfree : kfree) + (wave & 1) * SLOT;
            to_slot(slot);
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's rows are in the slot
            flush_from(slot);
        }
    }
    if constexpr (DEFER) flush_from(o_lds + wave * SLOT);  // the last item's stores
}

// Test hook: the same work tables and decoder, one wave per workgroup.
__global__ __launch_bounds__(64) void varlen_tile_map_kernel(const int32_t *cu_q, const int32_t *cu_k, int32_t batch,
                                                             int32_t num_heads, int32_t block_q, int32_t grain,
                                                             int32_t levels, int64_t n_items, int32_t *items)
{
    __shared__ int sched[kSchedInts];
    const int lane = threadIdx.x;
    const WorkTables wt = build_work_tables(cu_q, cu_k, batch + 1, batch, block_q, grain, levels, sched, kSchedInts);
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

template <int D, bool CAUSAL, bool PAGED>
static void launch_fwd(bool sorted, dim3 grid, dim3 block, hipStream_t stream, const VarlenArgs &a)
{
    if (sorted) hipLaunchKernelGGL((varlen_fwd_kernel<D, CAUSAL, PAGED, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((varlen_fwd_kernel<D, CAUSAL, PAGED, false>), grid, block, 0, stream, a);
}

template <int D>
static hipError_t launch_d(const VarlenArgs &a, bool causal, int num_cus, hipStream_t stream)
{
    using T = VarlenTile<D>;
    if (a.block_q != T::BQ) return hipErrorInvalidValue;
    // paged keys: one 1 KiB load's keys must lie in one block
    if (a.block_table && (1 << a.bs_shift) * T::ROWB < 1024) return hipErrorInvalidValue;
    // persistent grid: as many workgroups as fit on the device at once
    const int64_t slots = (int64_t)num_cus * T::MIN_BLOCKS;
    const dim3 grid((unsigned)(a.n_items < slots ? a.n_items : slots)), block(T::THREADS);
    const bool sorted = varlen_sort_grain(D, a.batch, a.levels) > 0;
    if (a.block_table) {
        if (causal) launch_fwd<D, true, true>(sorted, grid, block, stream, a);
        else launch_fwd<D, false, true>(sorted, grid, block, stream, a);
    } else {
        if (causal) launch_fwd<D, true, false>(sorted, grid, block, stream, a);
        else launch_fwd<D, false, false>(sorted, grid, block, stream, a);
    }
    return hipGetLastError();
}

int32_t varlen_sort_grain(int32_t head_dim, int32_t batch, int32_t levels)
{
    const int g = varlen_block_k(head_dim);
    const bool sort = batch >= kSortMinBatch &&
                      work_tables_sorted(batch, levels, varlen_block_q(head_dim, 0), g, kSchedInts);
    return sort ? g : 0;
}

hipError_t launch_varlen_fwd(const VarlenArgs &a, int head_dim, bool causal, int num_cus, hipStream_t stream)
{
    switch (head_dim) {
    case 64: return launch_d<64>(a, causal, num_cus, stream);
    case 128: return launch_d<128>(a, causal, num_cus, stream);
    case 256: return launch_d<256>(a, causal, num_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_varlen_tile_map(const int32_t *cu_q, const int32_t *cu_k, int32_t batch, int32_t num_heads,
                                  int32_t block_q, int32_t grain, int32_t levels, int64_t n_items, int32_t *items_out,
                                  hipStream_t stream)
{
    const unsigned grid = (unsigned)(n_items < 1024 ? n_items : 1024);
    hipLaunchKernelGGL(varlen_tile_map_kernel, dim3(grid), dim3(64), 0, stream, cu_q, cu_k, batch, num_heads, block_q,
                       grain, levels, n_items, items_out);
    return hipGetLastError();
}

}  // namespace rra
