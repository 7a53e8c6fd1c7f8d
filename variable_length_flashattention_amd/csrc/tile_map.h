// Work list of the varlen forward pass, decoded inside the kernel.
//
// Sequence b has n_b = ceil(Lq_b / BQ) query tiles.  Tiles are ordered level
// by level: level r holds query tile r of every sequence with n_b > r, in
// ascending b, and levels run from the highest r down to 0.  With a causal
// mask and Lq == Lk, the tile at level r sees r+1 key tiles, so this order
// hands out the most expensive tiles first (longest-processing-time first
// under the hardware's in-order workgroup dispatch).  Each tile is split into
// num_heads items, head innermost: item w -> tile position w / H, head w % H.
// When H is a multiple of 8 every item of head h lands on the same XCD
// (workgroups are dealt round-robin over the 8 XCDs), so all query tiles of a
// (sequence, head) share one L2.
#pragma once
#include "rra_device.h"

namespace rra {

__device__ __forceinline__ int seq_tiles(const int32_t *__restrict__ cu, int b, int bq)
{
    const int L = cu[b + 1] - cu[b];
    return L > 0 ? (L + bq - 1) / bq : 0;
}

// Executed by all 64 lanes of one wave (wave-uniform control flow).  lds_nt
// caches n_b when batch <= lds_cap (it may alias other LDS the caller is not
// using yet).  On return every lane holds the same result.
__device__ __forceinline__ bool decode_work_item(const int32_t *__restrict__ cu_q, int batch, int num_heads, int bq,
                                                 int64_t w, int *lds_nt, int lds_cap, int lane, int &b_out,
                                                 int &qt_out, int &h_out)
{
    const bool cached = batch <= lds_cap;
    int64_t total = 0;
    int levels = 0;
    for (int b = lane; b < batch; b += 64) {
        const int n = seq_tiles(cu_q, b, bq);
        if (cached) lds_nt[b] = n;
        total += n;
        levels = max(levels, n);
    }
    total = wave_sum_i64(total);
    levels = wave_max_i32(levels);
    // make this wave's LDS writes visible to its own later reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int64_t tau = w / num_heads;
    h_out = (int)(w % num_heads);
    if (tau >= total) return false;

    // G(x) = sum_b max(0, n_b - x): tiles at levels >= x.
    auto tiles_from = [&](int x) -> int64_t {
        int64_t s = 0;
        for (int b = lane; b < batch; b += 64) {
            const int n = cached ? lds_nt[b] : seq_tiles(cu_q, b, bq);
            s += max(0, n - x);
        }
        return wave_sum_i64(s);
    };
    // smallest x in [1, levels] with G(x) <= tau; the item's level is x - 1
    int lo = 1, hi = levels;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tiles_from(mid) <= tau) hi = mid;
        else lo = mid + 1;
    }
    const int r = lo - 1;
    int64_t j = tau - tiles_from(lo);  // rank within level r
    for (int base = 0; base < batch; base += 64) {
        const int b = base + lane;
        const bool pred = b < batch && (cached ? lds_nt[b] : seq_tiles(cu_q, b, bq)) > r;
        const uint64_t mask = __ballot(pred);
        const int cnt = __popcll(mask);
        if (j < cnt) {
            const uint64_t below = lane == 0 ? 0ull : (mask & (~0ull >> (64 - lane)));
            const uint64_t hit = __ballot(pred && (int64_t)__popcll(below) == j);
            b_out = base + __ffsll((unsigned long long)hit) - 1;
            qt_out = r;
            return true;
        }
        j -= cnt;
    }
    return false;  // not reached when cu_seqlens is non-decreasing
}

}  // namespace rra
