// Padded <-> packed copies of per-token rows for gfx950.
//
// "Varlen Flash Attention Implementation Plan", Goal: a batch of sequences
// of different lengths runs packed, one after another with cu_seqlens
// offsets, instead of padded to the longest.  These two copies bring a
// padded batch [batch, max_seqlen, row] into that packed layout [total, row]
// and back: row t of sequence b sits at b*max_seqlen + t when padded and at
// cu_seqlens[b] + t when packed.  A row is any fixed number of bytes (the
// heads x head_dim bf16 values of q/k/v/out, or the heads fp32 values of lse).
//
// The copies are HBM-bound.  Each workgroup moves about 16 KiB: a run of
// consecutive rows of one sequence, as 16-byte (or 4-byte) pieces with
// consecutive lanes on consecutive addresses on both sides.
#include <type_traits>

#include "rra_device.h"
#include "rra_internal.h"

namespace rra {

template <int VEC, bool TO_PACKED>
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                        const int32_t *__restrict__ cu, int32_t max_seqlen,
                                                        int64_t row_bytes, int32_t rows_per_wg, int32_t wg_per_seq)
{
    using piece_t = std::conditional_t<VEC == 16, u32x4, uint32_t>;
    const int b = blockIdx.x / wg_per_seq, chunk = blockIdx.x % wg_per_seq;
    const int L = min(max(cu[b + 1] - cu[b], 0), max_seqlen);
    const int t0 = chunk * rows_per_wg;
    const int t1 = min(t0 + rows_per_wg, max_seqlen);
    // unpack writes every padded row of the chunk (zeros past L); pack only
    // the rows that exist
    const int t_end = TO_PACKED ? min(t1, L) : t1;
    if (t0 >= t_end) return;
    // pieces per row, and pieces in this workgroup's rows (at most 16 KiB / VEC
    // when several rows, one row's worth otherwise; both fit 32 bits)
    const int per_row = (int)(row_bytes / VEC);
    const int n = (t_end - t0) * per_row;
    const int64_t packed0 = (int64_t)cu[b] + t0, padded0 = (int64_t)b * max_seqlen + t0;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const int r = e / per_row, c = e % per_row;
        const int64_t pk = (packed0 + r) * row_bytes + (int64_t)c * VEC;
        const int64_t pd = (padded0 + r) * row_bytes + (int64_t)c * VEC;
        if constexpr (TO_PACKED) {
            *reinterpret_cast<piece_t *>(dst + pk) = *reinterpret_cast<const piece_t *>(src + pd);
        } else {
            piece_t x = {};
            if (t0 + r < L) x = *reinterpret_cast<const piece_t *>(src + pk);
            *reinterpret_cast<piece_t *>(dst + pd) = x;
        }
    }
}

int64_t pack_rows_per_wg(int64_t row_bytes) { return row_bytes >= 16384 ? 1 : 16384 / row_bytes; }

hipError_t launch_pack_rows(const void *src, void *dst, const int32_t *cu, int32_t batch, int32_t max_seqlen,
                            int64_t row_bytes, bool to_packed, bool vec16, hipStream_t stream)
{
    const int64_t rows = pack_rows_per_wg(row_bytes);
    const int64_t wg_per_seq = (max_seqlen + rows - 1) / rows;
    const dim3 grid((unsigned)(wg_per_seq * batch)), block(256);
    const uint8_t *s = static_cast<const uint8_t *>(src);
    uint8_t *d = static_cast<uint8_t *>(dst);
    const int32_t r = (int32_t)rows, w = (int32_t)wg_per_seq;
    if (vec16) {
        if (to_packed) hipLaunchKernelGGL((pack_rows_kernel<16, true>), grid, block, 0, stream, s, d, cu, max_seqlen, row_bytes, r, w);
        else hipLaunchKernelGGL((pack_rows_kernel<16, false>), grid, block, 0, stream, s, d, cu, max_seqlen, row_bytes, r, w);
    } else {
        if (to_packed) hipLaunchKernelGGL((pack_rows_kernel<4, true>), grid, block, 0, stream, s, d, cu, max_seqlen, row_bytes, r, w);
        else hipLaunchKernelGGL((pack_rows_kernel<4, false>), grid, block, 0, stream, s, d, cu, max_seqlen, row_bytes, r, w);
    }
    return hipGetLastError();
}

}  // namespace rra
