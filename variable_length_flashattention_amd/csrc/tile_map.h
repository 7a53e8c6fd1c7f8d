// Work list of the varlen forward pass, decoded inside the kernel.
//
// Sequence b has n_b = ceil(Lq_b / BQ) query tiles.  Tiles are ordered level
// by level: level r holds query tile r of every sequence with n_b > r, and
// levels run from the highest r down to 0.  With a causal mask and Lq == Lk,
// the tile at level r sees r+1 key tiles, so this order lists the most
// expensive tiles first.  Inside a level the sequences come in descending
// order of the sort key ceil(Lq_b / g) (ties: ascending b), for a cost grain
// g that divides BQ (the kernel's key tile): with a causal mask and
// Lq == Lk, the full tiles of level r all see the same keys, and a
// sequence's last tile sees ceil(Lq_b / g) key tiles, so the list also runs
// from costly to cheap inside a level.  The persistent workgroups are dealt
// the list in serpentine order, which balances them when it is sorted: with
// a thousand sequences of one or two key tiles, in ascending b the costs
// within a level are in random order.  When the sort does not apply (no
// grain given, more than 64 distinct keys, or too little LDS for the
// permutation) sequences come in ascending b.  Each tile is split into
// num_heads items, head innermost: item w -> tile position w / H, head w % H.
//
// With G(x) = sum_b max(0, n_b - x) (the number of tiles at levels >= x), the
// item's level r is the one with G(r+1) <= w/H < G(r), and its sequence is the
// (w/H - G(r+1))-th of the sequences with n_b > r, in the order above.  The
// sort key is non-decreasing in n_b (n_b = ceil(key / (BQ / g))), so those
// sequences are the first C(r) = #{b : n_b > r} entries of the sorted list.
#pragma once
#include "rra_device.h"

namespace rra {

__device__ __forceinline__ int seq_tiles(const int32_t *__restrict__ cu, int b, int bq)
{
    const int L = cu[b + 1] - cu[b];
    return L > 0 ? (L + bq - 1) / bq : 0;
}

// Tables one workgroup builds once in LDS and then decodes any number of
// items from: copies of cu_seqlens_q and of the key counts (nk ints: the
// batch + 1 entries of cu_seqlens_k, or the batch entries of per-sequence
// key counts), C(y) and G(x) for x, y = 0..levels, and (sorted tables) the
// permutation of the sequences in sort-key order.
// They are used when 2*(batch+1) + 2*(levels+1) ints fit the LDS space
// given; otherwise items are decoded from global memory
// (decode_work_item_global), with sequences in ascending b.  The sort needs
// batch + 1 + kSortScratchInts more ints and at most 64 distinct keys
// (levels * BQ / g <= 64).
constexpr int kSortScratchInts = 256;  // per-wave key counts, up to 4 waves
// The forward pass sorts only batches of at least this many sequences: with
// fewer, a level holds too few tiles for their order to change the balance,
// and the kernel built without the sort runs (its code is otherwise the same).
constexpr int kSortMinBatch = 64;

struct WorkTables {
    int *cuq, *cuk, *G, *perm;  // LDS
    int batch, levels, bq;
    bool cached, sorted;
};

// Whether tables over `batch` sequences with `levels` levels, tile height bq
// and cost grain `grain` (0: no sort) are sorted, for an LDS space of lds_ints.
__host__ __device__ __forceinline__ bool work_tables_sorted(int batch, int levels, int bq, int grain, int lds_ints)
{
    if (grain <= 0 || bq % grain != 0 || batch <= 0) return false;
    const int64_t keys = (int64_t)levels * (bq / grain);
    const int64_t need = 3 * (int64_t)(batch + 1) + 2 * (int64_t)(levels + 1) + kSortScratchInts;
    return keys >= 1 && keys <= 64 && need <= lds_ints;
}

// Sort key of sequence b: ceil(Lq_b / grain), clamped to kmax (0 for an
// empty sequence).
__device__ __forceinline__ int seq_sort_key(const int32_t *__restrict__ cu, int b, int grain, int kmax)
{
    const int L = cu[b + 1] - cu[b];
    return L > 0 ? min((L + grain - 1) / grain, kmax) : 0;
}

// All threads of the workgroup call this (blockDim.x a multiple of 64, at most
// 256); it ends with a barrier.  levels is an upper bound on max_b n_b
// (ceil(max_seqlen_q / bq)); grain is the cost grain g of the sort (0: no
// sort), a divisor of bq.
__device__ __forceinline__ WorkTables build_work_tables(const int32_t *__restrict__ cu_q,
                                                        const int32_t *__restrict__ cu_k, int nk, int batch, int bq,
                                                        int grain, int levels, int *lds, int lds_ints)
{
    WorkTables t;
    t.batch = batch;
    t.bq = bq;
    t.levels = levels;
    const bool cached = 2 * (batch + 1) + 2 * (levels + 1) <= lds_ints;
    const bool sorted = cached && work_tables_sorted(batch, levels, bq, grain, lds_ints);
    t.cached = cached;
    t.sorted = sorted;
    int *cuq = lds, *cuk = lds + (batch + 1);
    int *cnt = cuk + (batch + 1);      // C(y) = #{b : n_b > y}, y = 0..levels
    int *G = cnt + (levels + 1);
    int *perm = G + (levels + 1);      // batch entries (sorted tables)
    int *kcnt = perm + batch;          // per-wave key counts (sorted tables)
    t.cuq = cuq;
    t.cuk = cuk;
    t.G = G;
    t.perm = perm;
    if (!cached) return t;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nt >> 6;
    // the sort: wave v owns chunks [c0, c1) of 64 sequences; keys k = 1..kmax
    // are counted in lane k - 1
    const int kmax = sorted ? levels * (bq / grain) : 0;
    const int nch = (batch + 63) / 64, cpw = (nch + nwaves - 1) / nwaves;
    const int c0 = min(nch, wave * cpw), c1 = min(nch, c0 + cpw);
    for (int i = tid; i <= batch; i += nt) {
        cuq[i] = cu_q[i];
        if (i < nk) cuk[i] = cu_k[i];
    }
    for (int y = tid; y <= levels; y += nt) cnt[y] = 0;
    __syncthreads();
    // histogram of n_b (cnt[n] += 1), then suffix sums turn it into C(y)
    for (int b = tid; b < batch; b += nt) {
        const int n = seq_tiles(cuq, b, bq);
        if (n > 0) atomicAdd(&cnt[min(n, levels)], 1);
    }
    if (sorted) {
        // each wave counts the keys of its chunks, one ballot per distinct key
        int kc = 0;
        for (int c = c0; c < c1; c++) {
            const int b = 64 * c + lane;
            const int key = b < batch ? seq_sort_key(cuq, b, grain, kmax) : 0;
            uint64_t left = __ballot(key > 0);
            while (left) {
                const int k = __builtin_amdgcn_readlane(key, __builtin_ctzll(left));
                const uint64_t m = __ballot(key == k);
                if (lane == k - 1) kc += __popcll(m);
                left &= ~m;
            }
        }
        kcnt[64 * wave + lane] = kc;
    }
    __syncthreads();
    if (tid < 64) {
        // C(y) = sum_{n > y} hist[n]; G(x) = sum_{y >= x} C(y); one wave, serial over
        // chunks of 64 levels from the top
        int carry_c = 0, carry_g = 0;
        for (int top = levels; top >= 0; top -= 64) {
            const int y = top - tid;
            const int hist = y >= 0 ? cnt[y] : 0;
            // inclusive suffix sum of hist over y' >= y within the chunk
            int s = hist;
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(s, off, 64);
                if (tid >= off) s += o;
            }
            const int c_incl = s + carry_c;          // sum_{n >= y} hist[n]
            const int c_y = c_incl - hist;           // C(y): n > y
            int g = c_y;
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(g, off, 64);
                if (tid >= off) g += o;
            }
            const int g_y = g + carry_g;             // sum_{y' >= y} C(y')
            carry_c = __shfl(c_incl, 63, 64);
            carry_g = __shfl(g_y, 63, 64);
            if (y >= 0) {
                cnt[y] = c_y;
                G[y] = g_y;
            }
        }
    }
    if (sorted) {
        // key k's sequences start after all sequences with larger keys and,
        // inside key k, after those of lower waves; a wave then places its
        // chunks in ascending b, one ballot per distinct key
        int tot = 0, before = 0;
        for (int v = 0; v < nwaves; v++) {
            const int x = kcnt[64 * v + lane];
            tot += x;
            if (v < wave) before += x;
        }
        int above = tot;  // sum over lanes >= this lane
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_down(above, off, 64);
            if (lane + off < 64) above += o;
        }
        int run = above - tot + before;
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        for (int c = c0; c < c1; c++) {
            const int b = 64 * c + lane;
            const int key = b < batch ? seq_sort_key(cuq, b, grain, kmax) : 0;
            uint64_t left = __ballot(key > 0);
            while (left) {
                const int k = __builtin_amdgcn_readlane(key, __builtin_ctzll(left));
                const uint64_t m = __ballot(key == k);
                const int base = __builtin_amdgcn_readlane(run, k - 1);
                if (key == k) perm[base + __popcll(m & below)] = b;
                if (lane == k - 1) run += __popcll(m);
                left &= ~m;
            }
        }
    }
    __syncthreads();
    return t;
}

// Decode item w from the LDS tables.  Every lane of a wave gets the same
// result; any wave may call it independently.  Returns false past the end.
__device__ __forceinline__ bool decode_work_item_cached(const WorkTables &t, int num_heads, int64_t w, int lane,
                                                        int &b_out, int &qt_out, int &h_out)
{
    const int64_t tau = w / num_heads;
    h_out = (int)(w % num_heads);
    const int *G = t.G;
    if (tau >= G[0]) return false;
    // smallest x in [1, levels] with G(x) <= tau; the item's level is x - 1
    int lo = 1, hi = t.levels;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (G[mid] <= tau) hi = mid;
        else lo = mid + 1;
    }
    const int r = lo - 1;
    int64_t j = tau - G[lo];  // rank within level r
    if (t.sorted) {
        // level r's sequences are the first C(r) entries of the permutation
        b_out = t.perm[j];
        qt_out = r;
        return true;
    }
    for (int base = 0; base < t.batch; base += 64) {
        const int b = base + lane;
        const bool pred = b < t.batch && seq_tiles(t.cuq, b, t.bq) > r;
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

// The same decode straight from global memory (used when the tables do not
// fit in LDS).  Executed by all 64 lanes of one wave.
__device__ __forceinline__ bool decode_work_item_global(const int32_t *__restrict__ cu_q, int batch, int num_heads,
                                                        int bq, int64_t w, int lane, int &b_out, int &qt_out,
                                                        int &h_out)
{
    int64_t total = 0;
    int levels = 0;
    for (int b = lane; b < batch; b += 64) {
        const int n = seq_tiles(cu_q, b, bq);
        total += n;
        levels = max(levels, n);
    }
    total = wave_sum_i64(total);
    levels = wave_max_i32(levels);
    const int64_t tau = w / num_heads;
    h_out = (int)(w % num_heads);
    if (tau >= total) return false;
    auto tiles_from = [&](int x) -> int64_t {
        int64_t s = 0;
        for (int b = lane; b < batch; b += 64) s += max(0, seq_tiles(cu_q, b, bq) - x);
        return wave_sum_i64(s);
    };
    int lo = 1, hi = levels;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tiles_from(mid) <= tau) hi = mid;
        else lo = mid + 1;
    }
    const int r = lo - 1;
    int64_t j = tau - tiles_from(lo);
    for (int base = 0; base < batch; base += 64) {
        const int b = base + lane;
        const bool pred = b < batch && seq_tiles(cu_q, b, bq) > r;
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
    return false;
}

__device__ __forceinline__ bool decode_work_item(const WorkTables &t, const int32_t *__restrict__ cu_q,
                                                 int num_heads, int64_t w, int lane, int &b, int &qt, int &h)
{
    return t.cached ? decode_work_item_cached(t, num_heads, w, lane, b, qt, h)
                    : decode_work_item_global(cu_q, t.batch, num_heads, t.bq, w, lane, b, qt, h);
}

// Item handed to persistent workgroup g (of G) in its k-th round: rounds walk
// the list in blocks of G items, alternately forwards and backwards, so the
// costlier-first list is dealt out evenly.
__device__ __forceinline__ int64_t serpentine_item(int64_t k, int g, int G)
{
    return k * G + ((k & 1) ? (G - 1 - g) : g);
}

}  // namespace rra
