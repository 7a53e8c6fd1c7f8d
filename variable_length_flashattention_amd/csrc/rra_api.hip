// C ABI of librra (declared in include/rra.h): host-side validation and
// kernel launch.  Validation happens before any HIP call; rejected calls
// launch nothing.
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <mutex>

#include "../../include/rra.h"
#include "rra_internal.h"

using namespace rra;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

bool supported_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? RRA_OK : RRA_ERR_HIP; }

// s with 2^s == x, or -1 if x is not a power of two in [1, 2^30]
int32_t log2_exact(int32_t x)
{
    int32_t s = 0;
    while (s < 30 && (1 << s) < x) s++;
    return (1 << s) == x ? s : -1;
}

// Compute units of the current device (queried once per device).
int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Scratch of rra_paged_decode_attn_noalloc: the decode workspace (token-group
// offsets and fp32 partial states) of one call, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy of the array
// until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels get the address scratch_ptr() looked up.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

// This device's copy of `scratch` (looked up once per device, with the
// device current).  nullptr on a HIP error.
void *scratch_ptr()
{
    static std::mutex mu;
    static void *ptrs[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

// Debug check of the sequence offsets, run when the environment holds
// RRA_VALIDATE=1 (the preconditions of "Varlen Flash Attention
// Implementation Plan", Task 1, are otherwise the caller's to keep):
// cu_q[0] == 0, every Lq in [0, max_q] and cu_q[batch] <= total_q (when
// total_q >= 0); the keys likewise as offsets (every Lk >= 0, and <= max_k
// when max_k >= 0), or, for paged keys, as per-sequence lengths in
// [0, k_cap].  One workgroup writes its verdict (0 or 1) to a static device
// word, which the host reads back, so the check synchronises the stream.
__device__ int32_t cu_check_bad;

__global__ __launch_bounds__(256) void cu_check_kernel(const int32_t *cu_q, const int32_t *k, int32_t batch,
                                                       int32_t max_q, int64_t total_q, int32_t max_k,
                                                       int32_t k_lens, int32_t k_cap)
{
    int bad = 0;
    if (threadIdx.x == 0) {
        bad |= cu_q[0] != 0 || (!k_lens && k[0] != 0);
        bad |= total_q >= 0 && (int64_t)cu_q[batch] > total_q;
    }
    for (int b = threadIdx.x; b < batch; b += blockDim.x) {
        const int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b];
        bad |= lq < 0 || lq > max_q;
        const int64_t lk = k_lens ? (int64_t)k[b] : (int64_t)k[b + 1] - k[b];
        bad |= lk < 0 || (k_lens ? lk > k_cap : (max_k >= 0 && lk > max_k));
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) cu_check_bad = bad;
}

bool validate_requested()
{
    const char *e = std::getenv("RRA_VALIDATE");
    return e && e[0] == '1' && e[1] == '\0';
}

int32_t check_offsets(const int32_t *cu_q, const int32_t *k, int32_t batch, int32_t max_q, int64_t total_q,
                      int32_t max_k, bool k_lens, int32_t k_cap, void *stream)
{
    if (!validate_requested()) return RRA_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(cu_check_kernel, dim3(1), dim3(256), 0, st, cu_q, k, batch, max_q, total_q, max_k,
                       (int32_t)k_lens, k_cap);
    if (hipGetLastError() != hipSuccess) return RRA_ERR_HIP;
    int32_t bad = 1;
    if (hipMemcpyFromSymbolAsync(&bad, HIP_SYMBOL(cu_check_bad), sizeof bad, 0, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return RRA_ERR_HIP;
    return bad ? RRA_ERR_INVALID_ARG : RRA_OK;
}

}  // namespace

extern "C" {

const char *rra_status_string(int32_t status)
{
    switch (status) {
    case RRA_OK: return "RRA_OK";
    case RRA_ERR_INVALID_ARG: return "RRA_ERR_INVALID_ARG";
    case RRA_ERR_UNSUPPORTED: return "RRA_ERR_UNSUPPORTED";
    case RRA_ERR_WORKSPACE: return "RRA_ERR_WORKSPACE";
    case RRA_ERR_HIP: return "RRA_ERR_HIP";
    case RRA_ERR_SCRATCH: return "RRA_ERR_SCRATCH";
    default: return "RRA_UNKNOWN_STATUS";
    }
}

int32_t rra_varlen_block_q(int32_t head_dim, int32_t max_seqlen_q)
{
    return supported_head_dim(head_dim) && max_seqlen_q >= 0 ? varlen_block_q(head_dim, max_seqlen_q) : 0;
}

int32_t rra_varlen_attn_fwd_gqa(const void *q, const void *k, const void *v, void *out, float *lse,
                                const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t max_seqlen_q,
                                int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                float softmax_scale, int32_t causal, void *stream)
{
    if (batch < 0 || num_heads <= 0 || head_dim <= 0 || max_seqlen_q < 0) return RRA_ERR_INVALID_ARG;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return RRA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return RRA_ERR_INVALID_ARG;
    if (!good_scale(softmax_scale)) return RRA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return RRA_ERR_UNSUPPORTED;
    if (batch == 0 || max_seqlen_q == 0) return RRA_OK;  // no query rows exist
    if (!q || !k || !v || !out || !lse || !cu_seqlens_q || !cu_seqlens_k) return RRA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lse) & 3u))
        return RRA_ERR_INVALID_ARG;

    const int32_t vrc = check_offsets(cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, -1, -1, false, 0, stream);
    if (vrc != RRA_OK) return vrc;

    VarlenArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.batch = batch;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.gqa_ratio = num_heads / num_kv_heads;
    a.block_q = varlen_block_q(head_dim, max_seqlen_q);
    const int64_t tiles_per_seq = ((int64_t)max_seqlen_q + a.block_q - 1) / a.block_q;
    a.levels = (int32_t)tiles_per_seq;
    a.n_items = (int64_t)batch * tiles_per_seq * num_heads;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * kLog2e;
    a.block_table = nullptr;
    a.seqlens_k = nullptr;
    a.bs_shift = 0;
    a.max_blocks = 0;
    return hip_status(launch_varlen_fwd(a, head_dim, causal == 1, device_cus(), static_cast<hipStream_t>(stream)));
}

int32_t rra_varlen_attn_fwd_paged(const void *q, const void *k_pool, const void *v_pool, void *out, float *lse,
                                  const int32_t *cu_seqlens_q, const int32_t *seqlens_k,
                                  const int32_t *block_table, int32_t max_seqlen_q, int32_t batch,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, float softmax_scale, int32_t causal, void *stream)
{
    if (batch < 0 || num_heads <= 0 || head_dim <= 0 || max_seqlen_q < 0) return RRA_ERR_INVALID_ARG;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return RRA_ERR_INVALID_ARG;
    if (block_size <= 0 || max_blocks_per_seq < 0) return RRA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return RRA_ERR_INVALID_ARG;
    if (!good_scale(softmax_scale)) return RRA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return RRA_ERR_UNSUPPORTED;
    const int32_t bs_shift = log2_exact(block_size);
    if (bs_shift < 0 || block_size < 8 || block_size > 1024) return RRA_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return RRA_ERR_INVALID_ARG;
    if (batch == 0 || max_seqlen_q == 0) return RRA_OK;  // no query rows exist
    if (!q || !out || !lse || !cu_seqlens_q || !seqlens_k || !block_table || !k_pool || !v_pool)
        return RRA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return RRA_ERR_INVALID_ARG;

    const int32_t vrc = check_offsets(cu_seqlens_q, seqlens_k, batch, max_seqlen_q, -1, -1, true,
                                      max_blocks_per_seq * block_size, stream);
    if (vrc != RRA_OK) return vrc;

    VarlenArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k_pool);
    a.v = static_cast<const uint16_t *>(v_pool);
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.cu_q = cu_seqlens_q;
    a.cu_k = nullptr;
    a.batch = batch;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.gqa_ratio = num_heads / num_kv_heads;
    a.block_q = varlen_block_q(head_dim, max_seqlen_q);
    const int64_t tiles_per_seq = ((int64_t)max_seqlen_q + a.block_q - 1) / a.block_q;
    a.levels = (int32_t)tiles_per_seq;
    a.n_items = (int64_t)batch * tiles_per_seq * num_heads;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * kLog2e;
    a.block_table = block_table;
    a.seqlens_k = seqlens_k;
    a.bs_shift = bs_shift;
    a.max_blocks = max_blocks_per_seq;
    return hip_status(launch_varlen_fwd(a, head_dim, causal == 1, device_cus(), static_cast<hipStream_t>(stream)));
}

int32_t rra_varlen_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                            const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t max_seqlen_q,
                            int32_t batch, int32_t num_heads, int32_t head_dim, float softmax_scale,
                            int32_t causal, void *stream)
{
    return rra_varlen_attn_fwd_gqa(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, batch, num_heads,
                                   num_heads, head_dim, softmax_scale, causal, stream);
}

size_t rra_varlen_attn_bwd_workspace_bytes(int32_t total_q, int32_t num_heads)
{
    if (total_q < 0 || num_heads <= 0) return 0;
    return 2 * (size_t)total_q * (size_t)num_heads * sizeof(float);
}

int32_t rra_varlen_attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
                            const void *dout, void *dq, void *dk, void *dv, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, float softmax_scale, int32_t causal, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    if (batch < 0 || num_heads <= 0 || head_dim <= 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
        return RRA_ERR_INVALID_ARG;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return RRA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return RRA_ERR_INVALID_ARG;
    if (!good_scale(softmax_scale)) return RRA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return RRA_ERR_UNSUPPORTED;
    // workspace byte offsets are 32-bit inside the kernels
    if ((int64_t)total_q * num_heads > ((int64_t)1 << 28)) return RRA_ERR_INVALID_ARG;
    if (batch == 0 || (max_seqlen_q == 0 && max_seqlen_k == 0)) return RRA_OK;
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
        return RRA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || (reinterpret_cast<uintptr_t>(lse) & 3u))
        return RRA_ERR_INVALID_ARG;
    const size_t need = rra_varlen_attn_bwd_workspace_bytes(total_q, num_heads);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return RRA_ERR_WORKSPACE;

    const int32_t vrc =
        check_offsets(cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, total_q, max_seqlen_k, false, 0, stream);
    if (vrc != RRA_OK) return vrc;

    BwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.out = static_cast<const uint16_t *>(out);
    a.dout = static_cast<const uint16_t *>(dout);
    a.lse = lse;
    a.dq = static_cast<uint16_t *>(dq);
    a.dk = static_cast<uint16_t *>(dk);
    a.dv = static_cast<uint16_t *>(dv);
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.ws = static_cast<float *>(workspace);
    a.batch = batch;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.gqa_ratio = num_heads / num_kv_heads;
    a.head_dim = head_dim;
    a.total_q = total_q;
    a.levels_q = (int32_t)(((int64_t)max_seqlen_q + kBwdQRows - 1) / kBwdQRows);
    a.levels_k = (int32_t)(((int64_t)max_seqlen_k + kBwdKRows - 1) / kBwdKRows);
    a.n_items_q = (int64_t)batch * a.levels_q * num_heads;
    a.n_items_k = (int64_t)batch * a.levels_k * num_kv_heads;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * kLog2e;
    return hip_status(launch_varlen_bwd(a, causal == 1, device_cus(), static_cast<hipStream_t>(stream)));
}

static int32_t pack_call(const void *src, void *dst, const int32_t *cu_seqlens, int32_t batch, int32_t max_seqlen,
                         int64_t row_bytes, bool to_packed, void *stream)
{
    if (batch < 0 || max_seqlen < 0 || row_bytes <= 0 || row_bytes % 4 != 0) return RRA_ERR_INVALID_ARG;
    if (batch == 0 || max_seqlen == 0) return RRA_OK;
    if (!src || !dst || !cu_seqlens) return RRA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 3u) || (reinterpret_cast<uintptr_t>(dst) & 3u)) return RRA_ERR_INVALID_ARG;
    // one workgroup per run of rows of one sequence; a row's pieces are
    // counted in 32 bits
    const int64_t rows = pack_rows_per_wg(row_bytes);
    const int64_t wgs = (int64_t)batch * ((max_seqlen + rows - 1) / rows);
    if (wgs > INT32_MAX || row_bytes / 4 > INT32_MAX) return RRA_ERR_INVALID_ARG;
    const int32_t vrc = check_offsets(cu_seqlens, cu_seqlens, batch, max_seqlen, -1, -1, false, 0, stream);
    if (vrc != RRA_OK) return vrc;
    const bool vec16 = row_bytes % 16 == 0 && aligned16(src) && aligned16(dst);
    return hip_status(launch_pack_rows(src, dst, cu_seqlens, batch, max_seqlen, row_bytes, to_packed, vec16,
                                       static_cast<hipStream_t>(stream)));
}

int32_t rra_pack_rows(const void *padded, void *packed, const int32_t *cu_seqlens, int32_t batch,
                      int32_t max_seqlen, int64_t row_bytes, void *stream)
{
    return pack_call(padded, packed, cu_seqlens, batch, max_seqlen, row_bytes, true, stream);
}

int32_t rra_unpack_rows(const void *packed, void *padded, const int32_t *cu_seqlens, int32_t batch,
                        int32_t max_seqlen, int64_t row_bytes, void *stream)
{
    return pack_call(packed, padded, cu_seqlens, batch, max_seqlen, row_bytes, false, stream);
}

int32_t rra_debug_varlen_tile_map(const int32_t *cu_seqlens_q, int32_t batch, int32_t num_heads,
                                  int32_t max_seqlen_q, int32_t head_dim, int32_t *items_out, int64_t capacity,
                                  int64_t *item_count, void *stream)
{
    if (batch < 0 || num_heads <= 0 || max_seqlen_q < 0 || !item_count) return RRA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return head_dim <= 0 ? RRA_ERR_INVALID_ARG : RRA_ERR_UNSUPPORTED;
    const int32_t bq = varlen_block_q(head_dim, max_seqlen_q);
    const int64_t tiles_per_seq = ((int64_t)max_seqlen_q + bq - 1) / bq;
    const int64_t n = (int64_t)batch * tiles_per_seq * num_heads;
    *item_count = n;
    if (n == 0) return RRA_OK;
    if (!cu_seqlens_q || !items_out || capacity < n) return RRA_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_varlen_tile_map(cu_seqlens_q, cu_seqlens_q, batch, num_heads, bq,
                                          varlen_sort_grain(head_dim, batch, (int32_t)tiles_per_seq),
                                          (int32_t)tiles_per_seq, n, items_out, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return hip_status(e);
}

size_t rra_paged_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
    if (!supported_head_dim(head_dim)) return 0;
    return decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim);
}

// Checks and DecodeArgs set-up shared by the one-shot decode and the
// stateful step: everything except the context source and the destination.
// (gather: the test hook, which reads no q and takes no scale.)
static int32_t decode_setup(DecodeArgs &a, const void *q, const void *k_pool, const void *v_pool,
                            const int32_t *block_table, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks,
                            float softmax_scale, void *workspace, size_t workspace_bytes, bool gather = false)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks < 0)
        return RRA_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0) return RRA_ERR_INVALID_ARG;
    if (!good_scale(softmax_scale)) return RRA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return RRA_ERR_UNSUPPORTED;
    const int32_t bs_shift = log2_exact(block_size);
    if (bs_shift < 0 || block_size > 1024) return RRA_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks * block_size > INT32_MAX) return RRA_ERR_INVALID_ARG;
    if ((int64_t)num_seqs * num_q_heads > INT32_MAX) return RRA_ERR_INVALID_ARG;  // one combine workgroup each
    if (num_seqs == 0) return RRA_OK;
    if ((!gather && !q) || !k_pool || !v_pool || !block_table) return RRA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return RRA_ERR_INVALID_ARG;
    const size_t need = decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return RRA_ERR_WORKSPACE;

    a = DecodeArgs{};
    a.q = static_cast<const uint16_t *>(q);
    a.k_pool = static_cast<const uint16_t *>(k_pool);
    a.v_pool = static_cast<const uint16_t *>(v_pool);
    a.block_table = block_table;
    // workspace: goff [num_seqs + 1] int32 | m, l [slots * num_q_heads] fp32 |
    // o [slots * num_q_heads * head_dim] fp32, slots = n_ranges + num_seqs,
    // each part starting on a 256-byte boundary
    const int32_t n_ranges = decode_n_ranges(num_q_heads, num_kv_heads, head_dim);
    const size_t n = ((size_t)n_ranges + (size_t)num_seqs) * num_q_heads;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    char *ws = static_cast<char *>(workspace);
    a.ws_goff = reinterpret_cast<int32_t *>(ws);
    ws += up(((size_t)num_seqs + 1) * sizeof(int32_t));
    a.ws_m = reinterpret_cast<float *>(ws);
    a.ws_l = a.ws_m + n;
    a.ws_o = reinterpret_cast<float *>(ws + up(2 * n * sizeof(float)));
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.bs_shift = bs_shift;
    a.max_blocks = max_blocks;
    a.n_ranges = n_ranges;
    const int32_t ratio = num_q_heads / num_kv_heads;
    a.n_sub = (ratio + 15) / 16;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * kLog2e;
    return RRA_OK;
}

int32_t rra_paged_decode_attn(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                              const int32_t *context_lens, void *out, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t max_blocks_per_seq, float softmax_scale, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    DecodeArgs a;
    const int32_t rc = decode_setup(a, q, k_pool, v_pool, block_table, num_seqs, num_q_heads, num_kv_heads,
                                    head_dim, block_size, max_blocks_per_seq, softmax_scale, workspace,
                                    workspace_bytes);
    if (rc != RRA_OK || num_seqs == 0) return rc;
    if (!context_lens || !out || !aligned16(out)) return RRA_ERR_INVALID_ARG;
    a.context_lens = context_lens;
    a.out = static_cast<uint16_t *>(out);
    return hip_status(launch_paged_decode(a, head_dim, static_cast<hipStream_t>(stream)));
}

size_t rra_paged_decode_scratch_bytes(void) { return kDecodeScratchBytes; }

int32_t rra_paged_decode_attn_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                      const int32_t *block_table, const int32_t *context_lens, void *out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq, float softmax_scale,
                                      void *stream)
{
    // Validate first, with a stand-in address for the scratch (decode_setup
    // only checks its alignment): a rejected call makes no HIP call.
    DecodeArgs a;
    void *const stand_in = reinterpret_cast<void *>((uintptr_t)256);
    int32_t rc = decode_setup(a, q, k_pool, v_pool, block_table, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              block_size, max_blocks_per_seq, softmax_scale, stand_in, kDecodeScratchBytes);
    if (rc == RRA_ERR_WORKSPACE) return RRA_ERR_SCRATCH;  // the partial states need more than the scratch holds
    if (rc != RRA_OK || num_seqs == 0) return rc;
    if (!context_lens || !out || !aligned16(out)) return RRA_ERR_INVALID_ARG;
    void *ws = scratch_ptr();
    if (!ws) return RRA_ERR_HIP;
    rc = decode_setup(a, q, k_pool, v_pool, block_table, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq, softmax_scale, ws, kDecodeScratchBytes);
    if (rc != RRA_OK) return rc;
    a.context_lens = context_lens;
    a.out = static_cast<uint16_t *>(out);
    return hip_status(launch_paged_decode(a, head_dim, static_cast<hipStream_t>(stream)));
}

int32_t rra_paged_decode_step(float *state_m, float *state_l, float *state_o, const void *q, const void *k_pool,
                              const void *v_pool, const int32_t *tile_blocks, const int32_t *tile_block_counts,
                              const int32_t *tile_token_counts, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t tile_capacity,
                              float softmax_scale, void *workspace, size_t workspace_bytes, void *stream)
{
    DecodeArgs a;
    const int32_t rc = decode_setup(a, q, k_pool, v_pool, tile_blocks, num_seqs, num_q_heads, num_kv_heads,
                                    head_dim, block_size, tile_capacity, softmax_scale, workspace,
                                    workspace_bytes);
    if (rc != RRA_OK || num_seqs == 0) return rc;
    if (!tile_block_counts || !state_m || !state_l || !state_o || !aligned16(state_o)) return RRA_ERR_INVALID_ARG;
    a.block_counts = tile_block_counts;
    a.token_counts = tile_token_counts;
    a.st_m = state_m;
    a.st_l = state_l;
    a.st_o = state_o;
    return hip_status(launch_paged_decode(a, head_dim, static_cast<hipStream_t>(stream)));
}

int32_t rra_paged_decode_finalize(const float *state_l, const float *state_o, void *out, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t head_dim, void *stream)
{
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0) return RRA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return RRA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return RRA_OK;
    if (!state_l || !state_o || !out || !aligned16(state_o) || !aligned16(out)) return RRA_ERR_INVALID_ARG;
    return hip_status(launch_decode_finalize(state_l, state_o, static_cast<uint16_t *>(out),
                                             (int64_t)num_seqs * num_q_heads, head_dim,
                                             static_cast<hipStream_t>(stream)));
}

int32_t rra_paged_decode_state_init(float *state_m, float *state_l, float *state_o, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t head_dim, void *stream)
{
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0) return RRA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return RRA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return RRA_OK;
    if (!state_m || !state_l || !state_o || !aligned16(state_o)) return RRA_ERR_INVALID_ARG;
    return hip_status(launch_decode_state_init(state_m, state_l, state_o, (int64_t)num_seqs * num_q_heads,
                                               head_dim, static_cast<hipStream_t>(stream)));
}

int32_t rra_debug_paged_gather(const void *k_pool, const void *v_pool, const int32_t *block_table,
                               const int32_t *context_lens, void *k_dense, void *v_dense, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, void *workspace, size_t workspace_bytes, void *stream)
{
    DecodeArgs a;
    const int32_t rc = decode_setup(a, nullptr, k_pool, v_pool, block_table, num_seqs, num_q_heads, num_kv_heads,
                                    head_dim, block_size, max_blocks_per_seq, 1.f, workspace, workspace_bytes, true);
    if (rc != RRA_OK || num_seqs == 0) return rc;
    if (!context_lens || !k_dense || !v_dense || !aligned16(k_dense) || !aligned16(v_dense))
        return RRA_ERR_INVALID_ARG;
    a.context_lens = context_lens;
    a.gather_k = static_cast<uint16_t *>(k_dense);
    a.gather_v = static_cast<uint16_t *>(v_dense);
    return hip_status(launch_paged_gather(a, head_dim, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
