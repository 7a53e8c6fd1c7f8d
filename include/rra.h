/*
 * rra.h -- C ABI of librra.so: variable-length (packed-sequence) attention
 * forward pass and paged-KV grouped-query decode attention for AMD MI355X
 * (gfx950).
 *
 * Conventions for every entry point
 *   - Tensors are passed as plain device pointers; bf16 tensors as void*.
 *     All tensors are dense, row-major, and must not alias one another.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the call returns without synchronising.
 *   - Arguments are validated on the host before any HIP call; a rejected
 *     call launches nothing and returns a status below.  Launch failures
 *     reported by the HIP runtime return RRA_ERR_HIP.  No C++ exception
 *     crosses this boundary.
 *   - The library allocates no device memory: the caller owns every buffer
 *     (outputs and workspaces included).  Two static device arrays live in
 *     the library itself: the allocation-free decode's scratch and the
 *     one-word verdict of the debug check below.
 *   - The contents of device-side index arrays (cu_seqlens, block tables,
 *     context lengths) are preconditions, as stated per entry point; they are
 *     not read on the host.
 *   - Debug check: with RRA_VALIDATE=1 in the environment, the forward
 *     (packed, GQA, paged), backward and pack/unpack calls first check their
 *     sequence offsets on the device ([PLAN] Task 1 leaves these
 *     preconditions to the caller) and, launching nothing else, return
 *     RRA_ERR_INVALID_ARG when cu_seqlens[0] != 0, a sequence length is
 *     negative or above max_seqlen_q (max_seqlen_k for the backward's keys,
 *     max_seqlen for pack/unpack), the backward's cu_seqlens_q[batch] exceeds
 *     total_q, or a paged key length lies outside
 *     [0, max_blocks_per_seq * block_size].  The check is one small kernel
 *     and a synchronisation of `stream` per call; without the variable
 *     nothing is checked and nothing synchronises.
 *
 * Sources are cited by page title and section:
 *   [PLAN]   "Varlen Flash Attention Implementation Plan" (rustytorch)
 *   [DECODE] "spark_storage/attention_ref.rs"
 */
#ifndef RRA_H
#define RRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define RRA_OK                 0
#define RRA_ERR_INVALID_ARG    1  /* bad size, null pointer with work to do, bad scale, ... */
#define RRA_ERR_UNSUPPORTED    2  /* valid but not implemented (e.g. head_dim not 64/128/256) */
#define RRA_ERR_WORKSPACE      3  /* decode workspace missing or too small */
#define RRA_ERR_HIP            4  /* the HIP runtime reported an error at launch */
#define RRA_ERR_SCRATCH        5  /* the sizes need more than the library's static decode scratch */

/* Human-readable name of a status code (static string, never NULL). */
const char *rra_status_string(int32_t status);

/*
 * Variable-length attention forward ([PLAN] Task 1, kernel signature and
 * preconditions; Task 2, forward wrapper arguments).
 *
 * For every sequence b, head h and local query i of that sequence:
 *   out[cu_q[b]+i, h, :] = softmax_j(softmax_scale * q_i . k_j  over visible j) . V
 *   lse[cu_q[b]+i, h]    = log-sum-exp of the same scaled scores (natural log)
 * with fp32 accumulation and bf16 rounding of the output.  Key j of sequence b
 * (0 <= j < Lk_b) is visible to query i (0 <= i < Lq_b) when causal == 0, or
 * when j <= i + Lk_b - Lq_b (bottom-right aligned causal mask; for Lq == Lk this
 * is the usual "no key after the query" rule).  A query with no visible key
 * gets out = 0 and lse = -inf.
 *
 *   q, out        bf16 [total_q, num_heads, head_dim]; element (t,h,d) at (t*H+h)*D+d
 *   k, v          bf16 [total_k, num_heads, head_dim]
 *   lse           fp32 [total_q, num_heads]; element (t,h) at t*H+h
 *   cu_seqlens_q  int32 [batch+1] device array: 0 = cu[0] <= cu[1] <= ... ,
 *   cu_seqlens_k  sequence b owns tokens [cu[b], cu[b+1]); cu[batch] = total
 *   max_seqlen_q  >= every query length cu_q[b+1]-cu_q[b] (sizes the launch)
 *   batch         number of sequences (0 = nothing to do, returns RRA_OK)
 *   num_heads     > 0
 *   head_dim      64, 128 or 256 (others: RRA_ERR_UNSUPPORTED)
 *   softmax_scale finite and > 0
 *   causal        0 or 1
 * Rows of out/lse for tokens outside every query sequence are not written.
 */
int32_t rra_varlen_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                            const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                            int32_t max_seqlen_q, int32_t batch, int32_t num_heads,
                            int32_t head_dim, float softmax_scale, int32_t causal, void *stream);

/*
 * Grouped-query variant: k and v are [total_k, num_kv_heads, head_dim] bf16
 * and query head h reads kv head h / (num_heads / num_kv_heads) (contiguous
 * groups, the grouping of [DECODE] step_tile_ref; num_kv_heads == 1 is
 * multi-query attention).  num_kv_heads must be > 0 and divide num_heads
 * (else RRA_ERR_INVALID_ARG).  Everything else is as rra_varlen_attn_fwd,
 * which is this call with num_kv_heads == num_heads.
 */
int32_t rra_varlen_attn_fwd_gqa(const void *q, const void *k, const void *v, void *out, float *lse,
                                const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t batch, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                                int32_t causal, void *stream);

/*
 * Paged keys and values (chunked prefill): the forward pass above with each
 * sequence's keys and values read through a block table, with the paged
 * layout of [DECODE] step_tile_ref, e.g. a prompt chunk attending to the
 * context already in a paged KV cache.
 *
 *   q, out         bf16 [total_q, num_heads, head_dim], packed by cu_seqlens_q
 *   lse            fp32 [total_q, num_heads]
 *   k_pool, v_pool bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *   cu_seqlens_q   int32 [batch + 1] device array (as above)
 *   seqlens_k      int32 [batch] device array: keys of sequence b (Lk_b),
 *                  clamped into [0, max_blocks_per_seq * block_size]
 *   block_table    int32 [batch, max_blocks_per_seq] device array: key j of
 *                  sequence b is slot j % block_size of pool block
 *                  block_table[b, j / block_size]; entries at or past
 *                  ceil(Lk_b / block_size) are never read
 *   num_kv_heads   divides num_heads; query head h reads kv head
 *                  h / (num_heads / num_kv_heads)
 *   block_size     power of two in [8, 1024]
 * Other arguments and results as for rra_varlen_attn_fwd; with causal = 1
 * the mask is bottom-right aligned (query i of a sequence sees key j iff
 * j <= i + Lk - Lq), so a chunk of the last Lq positions of a sequence sees
 * its whole cached prefix.
 */
int32_t rra_varlen_attn_fwd_paged(const void *q, const void *k_pool, const void *v_pool, void *out, float *lse,
                                  const int32_t *cu_seqlens_q, const int32_t *seqlens_k,
                                  const int32_t *block_table, int32_t max_seqlen_q, int32_t batch,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, float softmax_scale, int32_t causal, void *stream);

/*
 * Backward pass of rra_varlen_attn_fwd / _gqa: the gradients of a loss L
 * with respect to q, k and v, given dout = dL/dout.  The plan names a
 * backward module and keeps lse for it ([PLAN] Task 1, "Write output and
 * LSE") without defining it further; this is the chain rule of the forward
 * definition: with P_ij = exp(scale q_i.k_j - lse_i) over the visible pairs,
 *   dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (dout_i.v_j - dout_i.out_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i
 * (grouped-query: dk, dv of a kv head sum over its query heads).
 *
 *   q, out, dout, dq  bf16 [total_q, num_heads, head_dim]
 *   k, v, dk, dv      bf16 [total_k, num_kv_heads, head_dim]
 *   lse               fp32 [total_q, num_heads]: the forward's lse (-inf for a
 *                     row without visible keys)
 *   out               the forward's output for the same inputs
 *   total_q           cu_seqlens_q[batch] (sizes the workspace)
 *   max_seqlen_q/_k   bound every query / key length (they size the launch)
 *   workspace         at least rra_varlen_attn_bwd_workspace_bytes(total_q,
 *                     num_heads) bytes, 16-byte aligned, caller-owned; its
 *                     contents on entry do not matter
 * Rows of dq without visible keys are 0; keys no query sees get dk = dv = 0.
 * Other arguments as for the forward pass.  total_q * num_heads must not
 * exceed 2^28.  Two kernels run on `stream` (dq, which also leaves the
 * rows' dout.out and rescaled lse in the workspace, then dk/dv); the result
 * is deterministic (no atomics).
 */
int32_t rra_varlen_attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
                            const void *dout, void *dq, void *dk, void *dv, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, float softmax_scale, int32_t causal, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Workspace bytes rra_varlen_attn_bwd needs: 8 * total_q * num_heads (0 if
 * the sizes are invalid). */
size_t rra_varlen_attn_bwd_workspace_bytes(int32_t total_q, int32_t num_heads);

/* Query rows per work item of rra_varlen_attn_fwd for this head_dim and
 * max_seqlen_q (0 if head_dim is unsupported or max_seqlen_q < 0).  Work
 * items are (sequence, query tile, head). */
int32_t rra_varlen_block_q(int32_t head_dim, int32_t max_seqlen_q);

/*
 * Paged-KV grouped-query decode attention ([DECODE] AttnState, step_tile_ref,
 * finalize_ref): one query token per sequence attends to the first
 * context_lens[s] tokens of its paged K/V.
 *
 *   q, out        bf16 [num_seqs, num_q_heads, head_dim]
 *   k_pool,v_pool bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_table   int32 [num_seqs, max_blocks_per_seq] device array; token t of
 *                 sequence s is slot t % block_size of pool block
 *                 block_table[s, t / block_size]; entries at or past
 *                 ceil(context_lens[s] / block_size) are never read
 *   context_lens  int32 [num_seqs] device array, 0 <= ctx <= max_blocks_per_seq*block_size
 *   num_q_heads   multiple of num_kv_heads; q head qh reads kv head
 *                 qh / (num_q_heads / num_kv_heads) (contiguous groups)
 *   head_dim      64, 128 or 256
 *   block_size    power of two in [1, 1024]
 *   softmax_scale finite and > 0
 *   workspace     device buffer of at least rra_paged_decode_workspace_bytes(...)
 *                 bytes (fp32 partial softmax states), owned by the caller; its
 *                 contents on entry do not matter
 * out = sum_t softmax_t(softmax_scale * q . K_t) V_t over t < context_lens[s],
 * and out = 0 for a sequence with context length 0.  Context lengths
 * outside [0, max_blocks_per_seq*block_size] are clamped into it, and the sum
 * over sequences of ceil(ctx / 16) must stay below 2^31.  Two kernels run on
 * `stream`: the partial states of equal ranges of token groups, then a
 * combine that writes out; above 256 sequences a first kernel writes the
 * sequences' token-group offsets into the workspace.
 */
int32_t rra_paged_decode_attn(const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *block_table, const int32_t *context_lens, void *out,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              float softmax_scale, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Workspace bytes rra_paged_decode_attn needs for these sizes (0 if the sizes
 * are invalid or head_dim is unsupported).  It does not depend on the context
 * lengths or the block size: the contexts are cut into a fixed number of
 * equal ranges, and the workspace holds one partial state per (range,
 * sequence) piece bound plus the sequences' token-group offsets. */
size_t rra_paged_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim);

/*
 * Allocation-free variant of rra_paged_decode_attn, for callers that cannot
 * allocate device memory or hand over a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, layouts and result as rra_paged_decode_attn, without the
 * workspace: the partial softmax states live in a static device array that
 * the library holds on each GPU it runs on, for the life of the process
 * (rra_paged_decode_scratch_bytes() bytes, 32 MiB; the call allocates
 * nothing, and the array's contents on entry do not matter).  Sizes whose
 * workspace (rra_paged_decode_workspace_bytes) exceeds it are rejected with
 * RRA_ERR_SCRATCH before any HIP call; e.g. 32 q heads over 8 kv heads fit
 * up to 1760 sequences at head_dim 128 (887 at 256, 3458 at 64).  All calls
 * on one GPU share the array: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race and give wrong results;
 * calls ordered on one stream are safe.  The first call on a device looks
 * up that device's copy (hipGetSymbolAddress) with the device current.
 */
int32_t rra_paged_decode_attn_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                      const int32_t *block_table, const int32_t *context_lens, void *out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                      float softmax_scale, void *stream);

/* Bytes of the static scratch rra_paged_decode_attn_noalloc uses per GPU. */
size_t rra_paged_decode_scratch_bytes(void);

/*
 * Stateful decode ([DECODE] AttnState, step_tile_ref, finalize_ref): the
 * running softmax state of every (sequence, q head) lives in caller-owned
 * fp32 device buffers, and each step folds one tile of paged K/V into it, so
 * that a context can arrive in pieces (e.g. as its blocks are produced).
 *
 *   state_m       fp32 [num_seqs, num_q_heads]: running max of the scaled
 *                 scores softmax_scale * q . K_t (-inf before any token)
 *   state_l       fp32 [num_seqs, num_q_heads]: sum of exp(score - m)
 *   state_o       fp32 [num_seqs, num_q_heads, head_dim]: sum of
 *                 exp(score - m) V_t; 16-byte aligned
 *
 * rra_paged_decode_state_init sets m = -inf, l = 0, o = 0 (one kernel).
 *
 * rra_paged_decode_step folds, for every sequence s, the tokens of this step's
 * tile into the state, in place:
 *   tile_blocks        int32 [num_seqs, tile_capacity] device array: the pool
 *                      blocks of the tile, in token order
 *   tile_block_counts  int32 [num_seqs] device array: blocks used in the tile
 *                      (clamped into [0, tile_capacity]; 0 leaves s unchanged)
 *   tile_token_counts  int32 [num_seqs] device array or NULL: the tile holds
 *                      the first tile_token_counts[s] tokens of its blocks
 *                      (clamped into [0, blocks * block_size]); NULL means
 *                      every slot of every listed block
 * q, k_pool, v_pool, num_q_heads, num_kv_heads, head_dim, block_size,
 * softmax_scale and the workspace are as for rra_paged_decode_attn (the
 * workspace size is rra_paged_decode_workspace_bytes of the same sizes).  The
 * new tokens' partial states are merged into (m, l, o) with the usual
 * max-shift.  Steps on one state must be ordered (same stream or
 * synchronised); any split of a context into tiles gives the same result up
 * to fp32 rounding.
 *
 * rra_paged_decode_finalize writes out (bf16 [num_seqs, num_q_heads,
 * head_dim], 16-byte aligned) = o / l, and 0 where l == 0 (no token seen).
 */
int32_t rra_paged_decode_state_init(float *state_m, float *state_l, float *state_o, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t head_dim, void *stream);

int32_t rra_paged_decode_step(float *state_m, float *state_l, float *state_o, const void *q,
                              const void *k_pool, const void *v_pool, const int32_t *tile_blocks,
                              const int32_t *tile_block_counts, const int32_t *tile_token_counts,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t tile_capacity,
                              float softmax_scale, void *workspace, size_t workspace_bytes,
                              void *stream);

int32_t rra_paged_decode_finalize(const float *state_l, const float *state_o, void *out, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t head_dim, void *stream);

/*
 * Padded <-> packed row copies ([PLAN] Goal: a batch of sequences of
 * different lengths runs packed back to back, addressed by cu_seqlens,
 * instead of padded to the longest).  They bring a padded batch into the
 * packed layout the calls above take, and their results back out.
 *
 *   padded      [batch, max_seqlen, row]: row t of sequence b at byte
 *               (b * max_seqlen + t) * row_bytes
 *   packed      [total, row]: row t of sequence b at byte
 *               (cu_seqlens[b] + t) * row_bytes
 *   cu_seqlens  int32 [batch + 1] device array, as for rra_varlen_attn_fwd;
 *               every length cu[b+1] - cu[b] must be <= max_seqlen (only the
 *               first max_seqlen rows of a longer sequence are copied)
 *   row_bytes   bytes per token row, a positive multiple of 4 (e.g.
 *               num_heads * head_dim * 2 for bf16 q/k/v/out, num_heads * 4
 *               for fp32 lse); both buffers 4-byte aligned
 * rra_pack_rows:   packed row cu[b] + t = padded row (b, t) for t < L_b;
 *                  other packed rows are left untouched.
 * rra_unpack_rows: padded row (b, t) = packed row cu[b] + t for t < L_b, and
 *                  all zero bytes for L_b <= t < max_seqlen.
 * batch == 0 or max_seqlen == 0 is a successful no-op.  The copies are
 * bit-exact (no arithmetic on the values).
 */
int32_t rra_pack_rows(const void *padded, void *packed, const int32_t *cu_seqlens, int32_t batch,
                      int32_t max_seqlen, int64_t row_bytes, void *stream);

int32_t rra_unpack_rows(const void *packed, void *padded, const int32_t *cu_seqlens, int32_t batch,
                        int32_t max_seqlen, int64_t row_bytes, void *stream);

/*
 * Test hooks (integer work, checked bit-exactly against an independent
 * definition).
 *
 * rra_debug_varlen_tile_map: runs the forward kernel's own work-item decoder
 * for every launched work item and writes items_out[3*w..3*w+2] =
 * (sequence, query tile, head) of item w, or (-1,-1,-1) for launched items
 * beyond the last one.  The order is the one the forward kernel uses for the
 * same batch and head_dim: levels from the highest query tile down, and
 * inside a level the sequences in ascending index, or, for batches of at
 * least 64 sequences whose work tables can hold the permutation and that
 * have at most 64 distinct keys ceil(Lq / key tile), in descending key with
 * ties in ascending index.  *item_count receives the number of launched items
 * (host value).  items_out must hold 3 * capacity int32; capacity must be at
 * least the launched count, which is batch * ceil(max_seqlen_q / block_q) *
 * num_heads with block_q = rra_varlen_block_q(head_dim, max_seqlen_q).
 * Synchronises `stream`.
 */
int32_t rra_debug_varlen_tile_map(const int32_t *cu_seqlens_q, int32_t batch, int32_t num_heads,
                                  int32_t max_seqlen_q, int32_t head_dim, int32_t *items_out,
                                  int64_t capacity, int64_t *item_count, void *stream);

/*
 * rra_debug_paged_gather: runs rra_paged_decode_attn's range-split kernel
 * ([DECODE] step_tile_ref's block-table addressing: token t of sequence s is
 * slot t % block_size of pool block block_table[s, t / block_size]) in a mode
 * that keeps everything up to and including its K and V loads -- the same
 * ranges, pieces, block-table windows, address computation and loads -- and
 * stores the loaded rows into dense copies instead of computing attention:
 *   k_dense[s, t, kh, :] = the row its K-operand loads fetched for token t,
 *   v_dense[s, t, kh, :] = the row its V staging loads fetched for token t,
 * bf16 [num_seqs, max_blocks_per_seq*block_size, num_kv_heads, head_dim], for
 * t < context_lens[s]; other rows are left untouched.  The arguments are
 * those of rra_paged_decode_attn for the same sizes (num_q_heads sets the
 * range split; the workspace is rra_paged_decode_workspace_bytes of them).
 */
int32_t rra_debug_paged_gather(const void *k_pool, const void *v_pool, const int32_t *block_table,
                               const int32_t *context_lens, void *k_dense, void *v_dense, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* RRA_H */
