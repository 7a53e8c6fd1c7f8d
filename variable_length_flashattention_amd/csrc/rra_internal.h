// Host-side launchers shared between the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rra {

constexpr float kLog2e = 1.4426950408889634f;

// Query rows per work item of the forward kernel: 4 waves x 32 rows.  (Two
// 32-row blocks per wave halve the LDS operand reads per FLOP but need more
// than 256 VGPR+AGPR per wave; that variant spilled and ran 2x slower.)
inline int varlen_block_q(int head_dim, int max_seqlen_q)
{
    (void)head_dim;
    (void)max_seqlen_q;
    return 128;
}
// Keys per key tile of the forward kernel (64, or 32 at head_dim 256): also
// the cost grain by which its work list orders the sequences of a level.
constexpr int varlen_block_k(int head_dim) { return head_dim <= 128 ? 64 : 32; }
// LDS ints a forward workgroup sets aside for its work-list tables (enough
// for about 1700 sequences; more fall back to decoding from global memory).
constexpr int kSchedInts = 3584;

struct VarlenArgs {
    const uint16_t *q, *k, *v;
    uint16_t *out;
    float *lse;
    const int32_t *cu_q, *cu_k;
    int32_t batch, num_heads;
    int32_t num_kv_heads;  // k and v heads; query head h reads kv head h / gqa_ratio
    int32_t gqa_ratio;     // num_heads / num_kv_heads
    int32_t block_q;     // query rows per work item (varlen_block_q)
    int32_t levels;      // ceil(max_seqlen_q / block_q): upper bound on tiles per sequence
    int64_t n_items;     // batch * levels * num_heads: upper bound on real items
    float scale;         // softmax scale
    float scale_log2;    // softmax scale * log2(e)
    // paged keys and values (block_table != nullptr): k, v are pools
    // [NB, BS, Hkv, D]; sequence b has seqlens_k[b] keys (clamped to
    // [0, max_blocks * BS]) in blocks block_table[b * max_blocks + j]
    const int32_t *block_table, *seqlens_k;
    int32_t bs_shift, max_blocks;
};

// Backward pass of the packed forward pass.  Workspace: lse2 and dsum,
// fp32 [num_heads][total_q] each (head-major, so a head's consecutive query
// rows are contiguous): lse2 = lse * log2(e) (+inf where lse = -inf), dsum =
// rowsum(dout * out).
struct BwdArgs {
    const uint16_t *q, *k, *v, *out, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    const int32_t *cu_q, *cu_k;
    float *ws;           // lse2 [H][total_q] then dsum [H][total_q]
    int32_t batch, num_heads, num_kv_heads, gqa_ratio, head_dim;
    int32_t total_q;
    int32_t levels_q, levels_k;   // ceil(max_seqlen / tile) for the two work lists
    int64_t n_items_q, n_items_k; // batch * levels * heads (dq items over q heads, dk/dv items over kv heads)
    float scale, scale_log2;
};
constexpr int kBwdQRows = 128;  // query rows per dq work item
constexpr int kBwdKRows = 128;  // keys per dk/dv work item
hipError_t launch_varlen_bwd(const BwdArgs &a, bool causal, int num_cus, hipStream_t stream);

hipError_t launch_varlen_fwd(const VarlenArgs &a, int head_dim, bool causal, int num_cus, hipStream_t stream);
// The cost grain by which the forward kernel orders the sequences of a level
// for this batch (0: ascending b), and so the grain its tile map uses.
int32_t varlen_sort_grain(int32_t head_dim, int32_t batch, int32_t levels);
hipError_t launch_varlen_tile_map(const int32_t *cu_q, const int32_t *cu_k, int32_t batch, int32_t num_heads,
                                  int32_t block_q, int32_t grain, int32_t levels, int64_t n_items, int32_t *items_out,
                                  hipStream_t stream);

// Where a sequence's token count comes from: context_lens[s] when given;
// otherwise (a step of the stateful interface) block_counts[s] whole blocks,
// cut at token_counts[s] when that is given.  Clamped to
// [0, max_blocks * block_size] either way.
struct CtxSource {
    const int32_t *context_lens, *block_counts, *token_counts;
    int32_t max_blocks, bs_shift;
};

struct DecodeArgs {
    const uint16_t *q, *k_pool, *v_pool;
    const int32_t *block_table, *context_lens;
    const int32_t *block_counts, *token_counts;  // stateful step (context_lens null)
    float *st_m, *st_l, *st_o;  // stateful step: the caller's state, merged in place
    uint16_t *out;
    uint16_t *gather_k, *gather_v;  // test hook only: dense copies of the loaded K and V rows
    int32_t *ws_goff;    // [num_seqs + 1] token-group offsets of the sequences
    float *ws_m, *ws_l, *ws_o;  // [n_ranges + num_seqs] x num_q_heads partial states
    int32_t num_seqs, num_q_heads, num_kv_heads;
    int32_t block_size, bs_shift, max_blocks;
    int32_t n_ranges;    // equal ranges of token groups, one wave each per kv head
    int32_t n_sub;       // q-head subgroups of 16 per kv head
    float scale;         // softmax scale
    float scale_log2;    // softmax scale * log2(e)
};

int32_t decode_n_ranges(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);
hipError_t launch_paged_decode(const DecodeArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_decode_finalize(const float *state_l, const float *state_o, uint16_t *out, int64_t units,
                                  int32_t head_dim, hipStream_t stream);
hipError_t launch_decode_state_init(float *state_m, float *state_l, float *state_o, int64_t units, int32_t head_dim,
                                    hipStream_t stream);
// The decode split kernel in its gather mode (test hook): a.gather_k and
// a.gather_v receive the K and V rows its loads fetch.
hipError_t launch_paged_gather(const DecodeArgs &a, int head_dim, hipStream_t stream);

// Padded <-> packed row copies (pack_rows.hip).  Rows of one workgroup:
// about 16 KiB worth.
int64_t pack_rows_per_wg(int64_t row_bytes);
hipError_t launch_pack_rows(const void *src, void *dst, const int32_t *cu, int32_t batch, int32_t max_seqlen,
                            int64_t row_bytes, bool to_packed, bool vec16, hipStream_t stream);

}  // namespace rra
