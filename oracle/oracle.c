/*
 * oracle.c -- plain, slow fp64 CPU reference for variable-length (packed)
 * attention and for paged-KV GQA decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links or calls it, and it shares no code, header or table with the GPU
 * kernels.
 *
 * Sources (web pages; cited by title and section):
 *   [PLAN]   "Varlen Flash Attention Implementation Plan" (rustytorch,
 *            docs/superpowers/plans/2026-06-27-varlen-flash-attention.md)
 *            -- Task 1 (CUDA kernel source) and Task 2 (CPU simulation
 *            varlen_attention_cpu, its tests).
 *   [DECODE] "spark_storage/attention_ref.rs" -- AttnState, step_tile_ref,
 *            finalize_ref.
 *
 * Arithmetic: every bf16 input is widened exactly to double; all sums,
 * exponentials and logarithms are double (libm).  Nothing is blocked, fused
 * or reordered beyond what the definitions below state.
 *
 * Readings of the pages that this file fixes (each one also listed in the
 * design notes):
 *   - causal masking is bottom-right aligned: query i of a sequence with
 *     Lq queries and Lk keys sees key j iff j <= i + Lk - Lq (for Lq == Lk
 *     this is the PLAN kernel's "k_pos > q_pos is masked" rule);
 *   - a query with no visible key gets out = 0 and lse = -inf (the PLAN
 *     kernel writes 0 for out when the denominator is 0; -inf is the exact
 *     log-sum-exp of an empty set);
 *   - lse is natural-log, in the scaled-score domain: lse = m + ln(l)
 *     ([PLAN] Task 1, "Write output and LSE");
 *   - decode only counts the first context_lens[s] tokens of a sequence; a
 *     partially filled last block is cut at the context length.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Simple static work split over POSIX threads.                             */
/* ------------------------------------------------------------------------ */
typedef void (*unit_fn)(void *ctx, int64_t unit, double *scratch);

typedef struct {
    unit_fn fn;
    void *ctx;
    int64_t n_units;
    int64_t first, step;
    size_t scratch_len;
} worker_args;

static void *worker_main(void *p)
{
    worker_args *a = (worker_args *)p;
    double *scratch = (double *)malloc((a->scratch_len ? a->scratch_len : 1) * sizeof(double));
    if (!scratch) return (void *)1;
    for (int64_t u = a->first; u < a->n_units; u += a->step) a->fn(a->ctx, u, scratch);
    free(scratch);
    return NULL;
}

static int run_units(unit_fn fn, void *ctx, int64_t n_units, size_t scratch_len, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    if (n_units < nthreads) nthreads = (int)(n_units > 0 ? n_units : 1);
    pthread_t tid[512];
    worker_args args[512];
    int rc = 0;
    for (int t = 0; t < nthreads; t++) {
        args[t].fn = fn; args[t].ctx = ctx; args[t].n_units = n_units;
        args[t].first = t; args[t].step = nthreads; args[t].scratch_len = scratch_len;
    }
    if (nthreads == 1) return worker_main(&args[0]) == NULL ? 0 : -1;
    int started = 0;
    for (int t = 0; t < nthreads; t++) {
        if (pthread_create(&tid[t], NULL, worker_main, &args[t]) != 0) { rc = -1; break; }
        started++;
    }
    for (int t = 0; t < started; t++) {
        void *ret = NULL;
        pthread_join(tid[t], &ret);
        if (ret != NULL) rc = -1;
    }
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Variable-length attention forward.                                       */
/*                                                                          */
/* Layout ([PLAN] Task 1 preconditions; Task 2 "Layout"): q, out are        */
/* [total_q, H, D], k, v are [total_k, Hkv, D], element (t, h, d) at        */
/* (t*H + h)*D + d.  lse is [total_q, H].  Sequence b owns the half-open    */
/* token ranges [cu_q[b], cu_q[b+1]) and [cu_k[b], cu_k[b+1]).  Query head  */
/* h reads kv head h / (H / Hkv): contiguous groups, the grouping of the    */
/* decode page ([DECODE] step_tile_ref); Hkv == H is plain multi-head       */
/* attention as in [PLAN].                                                  */
/*                                                                          */
/* For query i of sequence b and head h, with A(i) the visible keys:        */
/*   s_j = scale * sum_d q[i,d] k[j,d]                 (j in A(i))          */
/*   M   = max_j s_j,   Z = sum_j exp(s_j - M)                              */
/*   out = sum_j exp(s_j - M) v_j / Z,   lse = M + ln Z                     */
/* computed in the order of the PLAN's CPU simulation: scores for the row,  */
/* then the row max, then the exponential sum, then the weighted V sum.     */
/* ------------------------------------------------------------------------ */
typedef struct {
    const uint16_t *q, *k, *v;
    const int32_t *cu_q, *cu_k;
    int32_t batch, H, D;
    double scale;
    int32_t causal;
    double *out, *lse;
    /* sampled-row mode */
    const int32_t *rows; /* pairs (token, head) */
    int32_t Hkv;         /* kv heads; H % Hkv == 0 */
    /* paged keys and values (block_table != NULL): k, v are pools
     * [NB, BS, Hkv, D]; key j of sequence b is slot j % BS of pool block
     * block_table[b, j / BS]; sequence b has seqlens_k[b] keys */
    const int32_t *block_table, *seqlens_k;
    int32_t BS, max_blocks;
} varlen_ctx;

/* Number of keys of sequence b. */
static int64_t seq_keys(const varlen_ctx *c, int32_t b)
{
    return c->block_table ? (int64_t)c->seqlens_k[b] : (int64_t)c->cu_k[b + 1] - c->cu_k[b];
}

/* Row of kv head kh for key j of sequence b, in k or v (base).  Packed: token
 * cu_k[b] + j of [total_k, Hkv, D].  Paged: the decode page's block-table
 * addressing ([DECODE] step_tile_ref), applied to the keys of a prefill. */
static const uint16_t *key_row(const varlen_ctx *c, const uint16_t *base, int32_t b, int64_t j, int64_t kh)
{
    if (!c->block_table) return base + (((int64_t)c->cu_k[b] + j) * c->Hkv + kh) * c->D;
    const int64_t blk = c->block_table[(int64_t)b * c->max_blocks + j / c->BS];
    return base + ((blk * c->BS + j % c->BS) * c->Hkv + kh) * c->D;
}

/* Is key j visible to query i?  Bottom-right causal alignment. */
static int key_visible(int64_t i, int64_t j, int64_t Lq, int64_t Lk, int causal)
{
    if (j < 0 || j >= Lk) return 0;
    if (!causal) return 1;
    return j <= i + Lk - Lq;
}

/* One output row: sequence b, local query i, head h.  scratch holds Lk doubles. */
static void varlen_row(const varlen_ctx *c, int32_t b, int64_t i, int32_t h,
                       double *scratch, double *out_row, double *lse_out)
{
    const int64_t H = c->H, D = c->D, Hkv = c->Hkv;
    const int64_t kh = h / (H / Hkv);
    const int64_t q0 = c->cu_q[b];
    const int64_t Lq = (int64_t)c->cu_q[b + 1] - q0;
    const int64_t Lk = seq_keys(c, b);
    const uint16_t *qrow = c->q + ((q0 + i) * H + h) * D;

    /* scores of the visible keys, and their maximum */
    double M = -INFINITY;
    int64_t n_visible = 0;
    for (int64_t j = 0; j < Lk; j++) {
        if (!key_visible(i, j, Lq, Lk, c->causal)) { scratch[j] = -INFINITY; continue; }
        const uint16_t *krow = key_row(c, c->k, b, j, kh);
        double dot = 0.0;
        for (int64_t d = 0; d < D; d++) dot += bf16_value(qrow[d]) * bf16_value(krow[d]);
        scratch[j] = c->scale * dot;
        if (scratch[j] > M) M = scratch[j];
        n_visible++;
    }
    if (n_visible == 0) {
        for (int64_t d = 0; d < D; d++) out_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    /* normaliser */
    double Z = 0.0;
    for (int64_t j = 0; j < Lk; j++)
        if (key_visible(i, j, Lq, Lk, c->causal)) Z += exp(scratch[j] - M);
    /* weighted sum of values */
    for (int64_t d = 0; d < D; d++) out_row[d] = 0.0;
    for (int64_t j = 0; j < Lk; j++) {
        if (!key_visible(i, j, Lq, Lk, c->causal)) continue;
        const double w = exp(scratch[j] - M) / Z;
        const uint16_t *vrow = key_row(c, c->v, b, j, kh);
        for (int64_t d = 0; d < D; d++) out_row[d] += w * bf16_value(vrow[d]);
    }
    *lse_out = M + log(Z);
}

/* unit = b*H + h : every query row of one (sequence, head) */
static void varlen_unit(void *p, int64_t unit, double *scratch)
{
    const varlen_ctx *c = (const varlen_ctx *)p;
    const int32_t b = (int32_t)(unit / c->H), h = (int32_t)(unit % c->H);
    const int64_t q0 = c->cu_q[b];
    const int64_t Lq = (int64_t)c->cu_q[b + 1] - q0;
    for (int64_t i = 0; i < Lq; i++) {
        const int64_t t = q0 + i;
        varlen_row(c, b, i, h, scratch, c->out + (t * c->H + h) * c->D, c->lse + t * c->H + h);
    }
}

static int64_t max_len(const int32_t *cu, int32_t batch)
{
    int64_t m = 0;
    for (int32_t b = 0; b < batch; b++) {
        const int64_t L = (int64_t)cu[b + 1] - cu[b];
        if (L > m) m = L;
    }
    return m;
}

/* Returns 0 on success, -1 on bad arguments or allocation failure. */
int oracle_varlen_attn_gqa(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *cu_q, const int32_t *cu_k, int32_t batch,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, double scale,
                           int32_t causal, double *out, double *lse, int32_t nthreads)
{
    if (batch < 0 || num_heads <= 0 || head_dim <= 0) return -1;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return -1;
    for (int32_t b = 0; b < batch; b++)
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return -1;
    varlen_ctx c = {q, k, v, cu_q, cu_k, batch, num_heads, head_dim, scale, causal, out, lse, NULL, num_kv_heads,
                    NULL, NULL, 0, 0};
    return run_units(varlen_unit, &c, (int64_t)batch * num_heads, (size_t)max_len(cu_k, batch), nthreads);
}

int oracle_varlen_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const int32_t *cu_q, const int32_t *cu_k, int32_t batch,
                       int32_t num_heads, int32_t head_dim, double scale, int32_t causal,
                       double *out, double *lse, int32_t nthreads)
{
    return oracle_varlen_attn_gqa(q, k, v, cu_q, cu_k, batch, num_heads, num_heads, head_dim, scale, causal,
                                  out, lse, nthreads);
}

/* Sampled rows: rows[2r] = packed query token, rows[2r+1] = head.  Writes
 * out[r*D .. r*D+D) and lse[r].  The owning sequence of a token is the b
 * with cu_q[b] <= token < cu_q[b+1]. */
static void varlen_sample_unit(void *p, int64_t r, double *scratch)
{
    const varlen_ctx *c = (const varlen_ctx *)p;
    const int32_t t = c->rows[2 * r], h = c->rows[2 * r + 1];
    int32_t b = 0;
    while (!(c->cu_q[b] <= t && t < c->cu_q[b + 1])) b++;
    varlen_row(c, b, (int64_t)t - c->cu_q[b], h, scratch, c->out + r * c->D, c->lse + r);
}

int oracle_varlen_attn_rows_gqa(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *cu_q, const int32_t *cu_k, int32_t batch,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, double scale,
                                int32_t causal, const int32_t *rows, int64_t n_rows,
                                double *out, double *lse, int32_t nthreads)
{
    if (batch <= 0 || num_heads <= 0 || head_dim <= 0) return -1;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return -1;
    for (int64_t r = 0; r < n_rows; r++) {
        if (rows[2 * r] < cu_q[0] || rows[2 * r] >= cu_q[batch]) return -1;
        if (rows[2 * r + 1] < 0 || rows[2 * r + 1] >= num_heads) return -1;
    }
    varlen_ctx c = {q, k, v, cu_q, cu_k, batch, num_heads, head_dim, scale, causal, out, lse, rows, num_kv_heads,
                    NULL, NULL, 0, 0};
    return run_units(varlen_sample_unit, &c, n_rows, (size_t)max_len(cu_k, batch), nthreads);
}

int oracle_varlen_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const int32_t *cu_q, const int32_t *cu_k, int32_t batch,
                            int32_t num_heads, int32_t head_dim, double scale, int32_t causal,
                            const int32_t *rows, int64_t n_rows,
                            double *out, double *lse, int32_t nthreads)
{
    return oracle_varlen_attn_rows_gqa(q, k, v, cu_q, cu_k, batch, num_heads, num_heads, head_dim, scale, causal,
                                       rows, n_rows, out, lse, nthreads);
}

/* Paged keys and values (chunked prefill): the same definition, with the
 * keys and values of sequence b read through its block table as the decode
 * page does ([DECODE] step_tile_ref), seqlens_k[b] of them.  With causal
 * masking and Lk > Lq the queries are the last Lq positions of the sequence
 * (bottom-right alignment above).  rows == NULL: every row; else the listed
 * (packed query token, head) pairs, out/lse indexed by pair. */
static int paged_check(const int32_t *cu_q, const int32_t *seqlens_k, const int32_t *block_table, int32_t batch,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t max_blocks)
{
    if (batch < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks < 0) return -1;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return -1;
    for (int32_t b = 0; b < batch; b++) {
        if (cu_q[b + 1] < cu_q[b]) return -1;
        if (seqlens_k[b] < 0 || (int64_t)seqlens_k[b] > (int64_t)max_blocks * block_size) return -1;
        for (int64_t j = 0; j < ((int64_t)seqlens_k[b] + block_size - 1) / block_size; j++)
            if (block_table[(int64_t)b * max_blocks + j] < 0) return -1;
    }
    return 0;
}

int oracle_varlen_attn_paged(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *cu_q, const int32_t *seqlens_k, const int32_t *block_table,
                             int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks, double scale, int32_t causal,
                             const int32_t *rows, int64_t n_rows, double *out, double *lse, int32_t nthreads)
{
    if (paged_check(cu_q, seqlens_k, block_table, batch, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks))
        return -1;
    int64_t lk_max = 0;
    for (int32_t b = 0; b < batch; b++)
        if (seqlens_k[b] > lk_max) lk_max = seqlens_k[b];
    varlen_ctx c = {q, k_pool, v_pool, cu_q, NULL, batch, num_heads, head_dim, scale, causal, out, lse, rows,
                    num_kv_heads, block_table, seqlens_k, block_size, max_blocks};
    if (!rows) return run_units(varlen_unit, &c, (int64_t)batch * num_heads, (size_t)lk_max, nthreads);
    if (batch <= 0) return -1;
    for (int64_t r = 0; r < n_rows; r++) {
        if (rows[2 * r] < cu_q[0] || rows[2 * r] >= cu_q[batch]) return -1;
        if (rows[2 * r + 1] < 0 || rows[2 * r + 1] >= num_heads) return -1;
    }
    return run_units(varlen_sample_unit, &c, n_rows, (size_t)lk_max, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Backward pass of the packed forward pass (gradients of a scalar loss      */
/* through out = softmax(scale q k^T + mask) v).  The pages name a backward  */
/* module and keep lse for it without giving its arithmetic; this is the    */
/* chain rule of the definition above, nothing more:                        */
/*   P_ij  = exp(s_ij - lse_i)            (the forward's probabilities)     */
/*   dV_j  = sum_i P_ij dO_i                                                */
/*   dP_ij = dO_i . v_j                                                     */
/*   dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')   (softmax Jacobian)        */
/*   dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i          */
/* over the visible pairs (i, j) of one (sequence, query head); with        */
/* grouped-query K/V the kv head's dK and dV sum over its query heads.      */
/* Everything is recomputed in double from the bf16 inputs (out and lse of  */
/* the forward are not inputs here).  A row with no visible key has zero    */
/* gradient; keys that no query sees get dK = dV = 0.                       */
/*                                                                          */
/* Given-out variant: the row term sum_j' P_ij' dP_ij' equals dO_i . out_i  */
/* (out_i = sum_j P_ij v_j), the form a backward pass that takes the        */
/* forward's stored output uses.  When out_given is passed, the row term is */
/* that dot product with the given rows (fp64 [Tq, H, D]) instead; with the */
/* exact out both forms agree to rounding.                                  */
/* ------------------------------------------------------------------------ */
typedef struct {
    const uint16_t *q, *k, *v, *dout;
    const int32_t *cu_q, *cu_k;
    int32_t H, Hkv, D;
    double scale;
    int32_t causal;
    double *dq, *dk, *dv;
    const double *out_given; /* NULL: the exact row term */
} bwd_ctx;

/* unit = b*Hkv + kh: every query head of kv head kh, every row of sequence b
 * (the units write disjoint rows of dq, dk, dv).  scratch: 2*Lk doubles. */
static void bwd_unit(void *p, int64_t unit, double *scratch)
{
    const bwd_ctx *c = (const bwd_ctx *)p;
    const int32_t b = (int32_t)(unit / c->Hkv), kh = (int32_t)(unit % c->Hkv);
    const int64_t H = c->H, Hkv = c->Hkv, D = c->D, R = H / Hkv;
    const int64_t q0 = c->cu_q[b], k0 = c->cu_k[b];
    const int64_t Lq = (int64_t)c->cu_q[b + 1] - q0, Lk = (int64_t)c->cu_k[b + 1] - k0;
    double *prob = scratch, *dprob = scratch + Lk;
    for (int64_t j = 0; j < Lk; j++)
        for (int64_t d = 0; d < D; d++) {
            c->dk[((k0 + j) * Hkv + kh) * D + d] = 0.0;
            c->dv[((k0 + j) * Hkv + kh) * D + d] = 0.0;
        }
    for (int64_t h = kh * R; h < (kh + 1) * R; h++)
        for (int64_t i = 0; i < Lq; i++) {
            const uint16_t *qrow = c->q + ((q0 + i) * H + h) * D;
            const uint16_t *dorow = c->dout + ((q0 + i) * H + h) * D;
            double *dqrow = c->dq + ((q0 + i) * H + h) * D;
            for (int64_t d = 0; d < D; d++) dqrow[d] = 0.0;
            /* probabilities of the row (the forward's softmax) */
            double M = -INFINITY;
            for (int64_t j = 0; j < Lk; j++) {
                prob[j] = -INFINITY;
                if (!key_visible(i, j, Lq, Lk, c->causal)) continue;
                const uint16_t *krow = c->k + ((k0 + j) * Hkv + kh) * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; d++) dot += bf16_value(qrow[d]) * bf16_value(krow[d]);
                prob[j] = c->scale * dot;
                if (prob[j] > M) M = prob[j];
            }
            if (M == -INFINITY) continue; /* no visible key */
            double Z = 0.0;
            for (int64_t j = 0; j < Lk; j++)
                if (prob[j] != -INFINITY) Z += exp(prob[j] - M);
            for (int64_t j = 0; j < Lk; j++) prob[j] = prob[j] == -INFINITY ? 0.0 : exp(prob[j] - M) / Z;
            /* dP and the row's sum_j P_ij dP_ij */
            double rowdot = 0.0;
            for (int64_t j = 0; j < Lk; j++) {
                dprob[j] = 0.0;
                if (!key_visible(i, j, Lq, Lk, c->causal)) continue;
                const uint16_t *vrow = c->v + ((k0 + j) * Hkv + kh) * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; d++) dot += bf16_value(dorow[d]) * bf16_value(vrow[d]);
                dprob[j] = dot;
                rowdot += prob[j] * dot;
            }
            if (c->out_given) {
                const double *orow = c->out_given + ((q0 + i) * H + h) * D;
                rowdot = 0.0;
                for (int64_t d = 0; d < D; d++) rowdot += bf16_value(dorow[d]) * orow[d];
            }
            for (int64_t j = 0; j < Lk; j++) {
                if (!key_visible(i, j, Lq, Lk, c->causal)) continue;
                const double ds = prob[j] * (dprob[j] - rowdot);
                const uint16_t *krow = c->k + ((k0 + j) * Hkv + kh) * D;
                double *dkrow = c->dk + ((k0 + j) * Hkv + kh) * D;
                double *dvrow = c->dv + ((k0 + j) * Hkv + kh) * D;
                for (int64_t d = 0; d < D; d++) {
                    dvrow[d] += prob[j] * bf16_value(dorow[d]);
                    dqrow[d] += c->scale * ds * bf16_value(krow[d]);
                    dkrow[d] += c->scale * ds * bf16_value(qrow[d]);
                }
            }
        }
}

int oracle_varlen_attn_bwd_given_out(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     const uint16_t *dout, const double *out_given, const int32_t *cu_q,
                                     const int32_t *cu_k, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_dim, double scale, int32_t causal, double *dq, double *dk,
                                     double *dv, int32_t nthreads)
{
    if (batch < 0 || num_heads <= 0 || head_dim <= 0) return -1;
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return -1;
    for (int32_t b = 0; b < batch; b++)
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return -1;
    bwd_ctx c = {q, k, v, dout, cu_q, cu_k, num_heads, num_kv_heads, head_dim, scale, causal, dq, dk, dv, out_given};
    return run_units(bwd_unit, &c, (int64_t)batch * num_kv_heads, 2 * (size_t)max_len(cu_k, batch) + 1, nthreads);
}

int oracle_varlen_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                           const int32_t *cu_q, const int32_t *cu_k, int32_t batch, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, double scale, int32_t causal,
                           double *dq, double *dk, double *dv, int32_t nthreads)
{
    return oracle_varlen_attn_bwd_given_out(q, k, v, dout, NULL, cu_q, cu_k, batch, num_heads, num_kv_heads,
                                            head_dim, scale, causal, dq, dk, dv, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Paged-KV GQA decode.                                                     */
/*                                                                          */
/* [DECODE] layout: q, out [S, Hq, D]; k_pool, v_pool [NB, BS, Hkv, D];     */
/* token t of sequence s lives in physical block block_table[s, t / BS] at  */
/* slot t % BS; the q head qh reads kv head qh / (Hq / Hkv).                */
/* ------------------------------------------------------------------------ */
typedef struct {
    const uint16_t *q, *k_pool, *v_pool;
    const int32_t *block_table, *context_lens;
    int32_t S, Hq, Hkv, D, BS, max_blocks;
    double scale;
    int32_t tile_capacity; /* recurrent route only */
    double *out;
} decode_ctx;

static const uint16_t *pool_row(const decode_ctx *c, const uint16_t *pool, int32_t s, int64_t t, int32_t kh)
{
    const int64_t blk = c->block_table[(int64_t)s * c->max_blocks + t / c->BS];
    const int64_t slot = t % c->BS;
    return pool + ((blk * c->BS + slot) * c->Hkv + kh) * c->D;
}

/* Direct definition: out = softmax_t(scale * q.K_t) . V_t over t < ctx. */
static void decode_direct_unit(void *p, int64_t unit, double *scratch)
{
    const decode_ctx *c = (const decode_ctx *)p;
    const int32_t s = (int32_t)(unit / c->Hq), qh = (int32_t)(unit % c->Hq);
    const int32_t kh = qh / (c->Hq / c->Hkv);
    const int64_t ctx = c->context_lens[s], D = c->D;
    const uint16_t *qrow = c->q + ((int64_t)s * c->Hq + qh) * D;
    double *o = c->out + ((int64_t)s * c->Hq + qh) * D;
    for (int64_t d = 0; d < D; d++) o[d] = 0.0;
    if (ctx <= 0) return;
    double M = -INFINITY;
    for (int64_t t = 0; t < ctx; t++) {
        const uint16_t *kr = pool_row(c, c->k_pool, s, t, kh);
        double dot = 0.0;
        for (int64_t d = 0; d < D; d++) dot += bf16_value(qrow[d]) * bf16_value(kr[d]);
        scratch[t] = c->scale * dot;
        if (scratch[t] > M) M = scratch[t];
    }
    double Z = 0.0;
    for (int64_t t = 0; t < ctx; t++) Z += exp(scratch[t] - M);
    for (int64_t t = 0; t < ctx; t++) {
        const double w = exp(scratch[t] - M) / Z;
        const uint16_t *vr = pool_row(c, c->v_pool, s, t, kh);
        for (int64_t d = 0; d < D; d++) o[d] += w * bf16_value(vr[d]);
    }
}

/* Merge a tile's own softmax state (t_max, t_den, t_acc) into a running
 * state (run_max, run_den, run_acc): both are rescaled to the larger of the
 * two maxima (an empty state, max = -inf, gets weight 0). */
static void merge_state(double *run_max, double *run_den, double *run_acc, double t_max, double t_den,
                        const double *t_acc, int64_t D)
{
    const double top = t_max > *run_max ? t_max : *run_max;
    if (top == -INFINITY) return; /* both empty */
    const double w_run = *run_max == -INFINITY ? 0.0 : exp(*run_max - top);
    const double w_tile = t_max == -INFINITY ? 0.0 : exp(t_max - top);
    *run_den = *run_den * w_run + t_den * w_tile;
    for (int64_t d = 0; d < D; d++) run_acc[d] = run_acc[d] * w_run + t_acc[d] * w_tile;
    *run_max = top;
}

/* The softmax state of one tile of tokens, from its definition: scores[i]
 * of the n tokens (already scaled), their maximum, then the sum of
 * exp(score - max) and the same weights applied to the V rows (vrow(i) =
 * pool + voff[i]).  t_acc receives D doubles. */
static void tile_state(const double *scores, const int64_t *voff, const uint16_t *pool, int64_t n, int64_t D,
                       double *t_max, double *t_den, double *t_acc)
{
    double mx = -INFINITY;
    for (int64_t i = 0; i < n; i++)
        if (scores[i] > mx) mx = scores[i];
    *t_max = mx;
    *t_den = 0.0;
    for (int64_t d = 0; d < D; d++) t_acc[d] = 0.0;
    if (mx == -INFINITY) return;
    for (int64_t i = 0; i < n; i++) {
        const double w = exp(scores[i] - mx);
        *t_den += w;
        for (int64_t d = 0; d < D; d++) t_acc[d] += w * bf16_value(pool[voff[i] + d]);
    }
}

/* Score of q row qrow against the pool row at koff (scaled). */
static double pool_score(const uint16_t *qrow, const uint16_t *k_pool, int64_t koff, int64_t D, double scale)
{
    double dot = 0.0;
    for (int64_t d = 0; d < D; d++) dot += bf16_value(qrow[d]) * bf16_value(k_pool[koff + d]);
    return scale * dot;
}

/* The decode page's route (AttnState carried across step_tile_ref calls,
 * then finalize_ref): the context is visited in tiles of tile_capacity
 * blocks in block-table order; each tile's own state is merged into the
 * running state (-inf, 0, 0 at the start), which is all that is kept from
 * one tile to the next; then out = o / l if l > 0 else 0.  scratch holds
 * D + 2 * tile_capacity * BS doubles. */
static void decode_recurrent_unit(void *p, int64_t unit, double *scratch)
{
    const decode_ctx *c = (const decode_ctx *)p;
    const int32_t s = (int32_t)(unit / c->Hq), qh = (int32_t)(unit % c->Hq);
    const int32_t kh = qh / (c->Hq / c->Hkv);
    const int64_t ctx = c->context_lens[s], D = c->D;
    const uint16_t *qrow = c->q + ((int64_t)s * c->Hq + qh) * D;
    double *o_out = c->out + ((int64_t)s * c->Hq + qh) * D;
    const int64_t cap_tok = (int64_t)c->tile_capacity * c->BS;
    double *t_acc = scratch, *scores = scratch + D;
    int64_t *voff = (int64_t *)(scratch + D + cap_tok);

    double run_max = -INFINITY, run_den = 0.0;
    double *run_acc = o_out; /* the running numerator lives in the output row */
    for (int64_t d = 0; d < D; d++) run_acc[d] = 0.0;
    for (int64_t first = 0; first < ctx; first += cap_tok) {
        const int64_t n = ctx - first < cap_tok ? ctx - first : cap_tok;
        for (int64_t i = 0; i < n; i++) {
            const int64_t koff = pool_row(c, c->k_pool, s, first + i, kh) - c->k_pool;
            scores[i] = pool_score(qrow, c->k_pool, koff, D, c->scale);
            voff[i] = pool_row(c, c->v_pool, s, first + i, kh) - c->v_pool;
        }
        double t_max, t_den;
        tile_state(scores, voff, c->v_pool, n, D, &t_max, &t_den, t_acc);
        merge_state(&run_max, &run_den, run_acc, t_max, t_den, t_acc, D);
    }
    const double inv_l = run_den > 0.0 ? 1.0 / run_den : 0.0;
    for (int64_t d = 0; d < D; d++) o_out[d] *= inv_l;
}

static int decode_check(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                        int32_t max_blocks, const int32_t *context_lens)
{
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || max_blocks < 0) return -1;
    if (Hq % Hkv != 0) return -1;
    for (int32_t s = 0; s < S; s++)
        if (context_lens[s] < 0 || context_lens[s] > (int64_t)max_blocks * BS) return -1;
    return 0;
}

static int64_t max_ctx(const int32_t *context_lens, int32_t S)
{
    int64_t m = 1;
    for (int32_t s = 0; s < S; s++) if (context_lens[s] > m) m = context_lens[s];
    return m;
}

int oracle_paged_decode(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                        const int32_t *block_table, const int32_t *context_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        double scale, double *out, int32_t nthreads)
{
    if (decode_check(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, context_lens))
        return -1;
    decode_ctx c = {q, k_pool, v_pool, block_table, context_lens, num_seqs, num_q_heads, num_kv_heads,
                    head_dim, block_size, max_blocks_per_seq, scale, 0, out};
    return run_units(decode_direct_unit, &c, (int64_t)num_seqs * num_q_heads,
                     (size_t)max_ctx(context_lens, num_seqs), nthreads);
}

int oracle_paged_decode_recurrent(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                  const int32_t *block_table, const int32_t *context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                  double scale, int32_t tile_capacity, double *out, int32_t nthreads)
{
    if (decode_check(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, context_lens))
        return -1;
    if (tile_capacity <= 0) return -1;
    decode_ctx c = {q, k_pool, v_pool, block_table, context_lens, num_seqs, num_q_heads, num_kv_heads,
                    head_dim, block_size, max_blocks_per_seq, scale, tile_capacity, out};
    const size_t cap_tok = (size_t)tile_capacity * (size_t)block_size;
    return run_units(decode_recurrent_unit, &c, (int64_t)num_seqs * num_q_heads, (size_t)head_dim + 2 * cap_tok,
                     nthreads);
}

/* The decode page's stateful interface.  The caller owns the state
 * (AttnState): m, l [S, Hq] and o [S, Hq, D], starting at (-inf, 0, 0): the
 * largest scaled score seen, the sum of exp(score - m) and the same weights
 * applied to the V rows.  A step (step_tile_ref) takes, for every sequence
 * s, the tokens of the blocks tile_blocks[s, 0 .. tile_block_counts[s]) in
 * order, every token of each block unless token_counts is given, in which
 * case the tile ends after token_counts[s] tokens (a partly filled last
 * block); the state afterwards is that of the old tokens and the tile's
 * together, formed here as the tile's own state merged into the carried one
 * (tile_state, merge_state).  finalize_ref turns the state into out = o / l
 * (0 where l == 0).  scratch: D + 2 * tile_capacity * BS + 1 doubles. */
typedef struct {
    double *m, *l, *o;
    const uint16_t *q, *k_pool, *v_pool;
    const int32_t *tile_blocks, *tile_block_counts, *token_counts;
    int32_t S, Hq, Hkv, D, BS, tile_capacity;
    double scale;
} step_ctx;

static void decode_step_unit(void *p, int64_t unit, double *scratch)
{
    const step_ctx *c = (const step_ctx *)p;
    const int32_t s = (int32_t)(unit / c->Hq), qh = (int32_t)(unit % c->Hq);
    const int32_t kh = qh / (c->Hq / c->Hkv);
    const int64_t D = c->D;
    const uint16_t *qrow = c->q + ((int64_t)s * c->Hq + qh) * D;
    const int64_t cap_tok = (int64_t)c->tile_capacity * c->BS;
    double *t_acc = scratch, *scores = scratch + D;
    int64_t *voff = (int64_t *)(scratch + D + cap_tok);
    /* the tile's tokens: the first n_tok slots of its listed blocks, in order */
    const int64_t n_tok = c->token_counts ? c->token_counts[s] : (int64_t)c->tile_block_counts[s] * c->BS;
    int64_t n = 0;
    for (int64_t b = 0; b < c->tile_block_counts[s]; b++) {
        const int64_t blk = c->tile_blocks[(int64_t)s * c->tile_capacity + b];
        for (int64_t slot = 0; slot < c->BS; slot++) {
            if (b * c->BS + slot >= n_tok) break;
            const int64_t row = ((blk * c->BS + slot) * c->Hkv + kh) * D;
            scores[n] = pool_score(qrow, c->k_pool, row, D, c->scale);
            voff[n++] = row;
        }
    }
    double t_max, t_den;
    tile_state(scores, voff, c->v_pool, n, D, &t_max, &t_den, t_acc);
    /* the caller's state, carried in from the previous step */
    double carried_max = c->m[unit], carried_den = c->l[unit];
    merge_state(&carried_max, &carried_den, c->o + unit * D, t_max, t_den, t_acc, D);
    c->m[unit] = carried_max;
    c->l[unit] = carried_den;
}

int oracle_paged_decode_step(double *state_m, double *state_l, double *state_o,
                             const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *tile_blocks, const int32_t *tile_block_counts,
                             const int32_t *token_counts, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t tile_capacity,
                             double scale, int32_t nthreads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0) return -1;
    if (num_q_heads % num_kv_heads != 0 || tile_capacity < 0) return -1;
    for (int32_t s = 0; s < num_seqs; s++) {
        if (tile_block_counts[s] < 0 || tile_block_counts[s] > tile_capacity) return -1;
        if (token_counts && (token_counts[s] < 0 || token_counts[s] > (int64_t)tile_block_counts[s] * block_size))
            return -1;
    }
    step_ctx c = {state_m, state_l, state_o, q, k_pool, v_pool, tile_blocks, tile_block_counts, token_counts,
                  num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, tile_capacity, scale};
    const size_t cap_tok = (size_t)tile_capacity * (size_t)block_size;
    return run_units(decode_step_unit, &c, (int64_t)num_seqs * num_q_heads, (size_t)head_dim + 2 * cap_tok + 1,
                     nthreads);
}

int oracle_paged_decode_finalize(const double *state_l, const double *state_o, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t head_dim, double *out)
{
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0) return -1;
    for (int64_t u = 0; u < (int64_t)num_seqs * num_q_heads; u++) {
        const double inv_l = state_l[u] > 0.0 ? 1.0 / state_l[u] : 0.0;
        for (int64_t d = 0; d < head_dim; d++) out[u * head_dim + d] = state_o[u * head_dim + d] * inv_l;
    }
    return 0;
}

/* Gather of the visible pool rows of every sequence into a dense buffer
 * [S, max_blocks*BS, Hkv, D] (bf16 bit copies); rows t >= ctx are left as
 * the caller filled them.  This is the block-table indexing alone. */
int oracle_paged_gather(const uint16_t *pool, const int32_t *block_table, const int32_t *context_lens,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, uint16_t *dense)
{
    if (decode_check(num_seqs, num_kv_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, context_lens))
        return -1;
    decode_ctx c = {NULL, pool, NULL, block_table, context_lens, num_seqs, num_kv_heads, num_kv_heads,
                    head_dim, block_size, max_blocks_per_seq, 1.0, 0, NULL};
    const int64_t T = (int64_t)max_blocks_per_seq * block_size;
    for (int32_t s = 0; s < num_seqs; s++)
        for (int64_t t = 0; t < context_lens[s]; t++)
            for (int32_t kh = 0; kh < num_kv_heads; kh++)
                memcpy(dense + (((int64_t)s * T + t) * num_kv_heads + kh) * head_dim,
                       pool_row(&c, pool, s, t, kh), (size_t)head_dim * sizeof(uint16_t));
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Work list of the tiled forward pass (integer work).                      */
/*                                                                          */
/* Sequence b is cut into n_b = ceil(Lq_b / block_q) query tiles.  Tiles are */
/* listed level by level: level r holds tile index qt = r of every sequence */
/* with n_b > r; levels run from the highest r down to 0.  Under causal     */
/* masking with Lq == Lk a tile at level r sees r+1 key tiles, so this      */
/* lists the most expensive tiles first.  Inside a level the sequences come */
/* in ascending b when sort_grain is 0; otherwise in descending order of    */
/* ceil(Lq_b / sort_grain), ties in ascending b (the cost of a sequence's   */
/* last tile, in key tiles of sort_grain keys, when Lq == Lk).  Each tile   */
/* expands into num_heads items, head innermost: item = position * H + h.  */
/* The order is a scheduling choice (the pages leave the mapping of tiles   */
/* to thread blocks open); this is the list the GPU work decoder must       */
/* reproduce exactly.                                                       */
/* Output: items[3*w .. 3*w+2] = (b, qt, h).  Returns the item count, or    */
/* -1 if capacity is too small or arguments are bad.                        */
/* ------------------------------------------------------------------------ */
static int64_t seq_len_at(const int32_t *cu_q, int32_t b) { return (int64_t)cu_q[b + 1] - cu_q[b]; }

int64_t oracle_varlen_tile_map(const int32_t *cu_q, int32_t batch, int32_t num_heads, int32_t block_q,
                               int32_t sort_grain, int32_t *items, int64_t capacity)
{
    if (batch < 0 || num_heads <= 0 || block_q <= 0 || sort_grain < 0) return -1;
    int64_t max_tiles = 0;
    for (int32_t b = 0; b < batch; b++) {
        const int64_t L = (int64_t)cu_q[b + 1] - cu_q[b];
        if (L < 0) return -1;
        const int64_t n = (L + block_q - 1) / block_q;
        if (n > max_tiles) max_tiles = n;
    }
    /* the order of the sequences inside every level: ascending b, then (with
       a grain) a stable insertion sort by descending ceil(L / grain) */
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(batch > 0 ? batch : 1));
    if (!order) return -1;
    for (int32_t b = 0; b < batch; b++) order[b] = b;
    if (sort_grain > 0) {
        for (int32_t i = 1; i < batch; i++) {
            const int32_t x = order[i];
            const int64_t kx = (seq_len_at(cu_q, x) + sort_grain - 1) / sort_grain;
            int32_t j = i;
            while (j > 0 && (seq_len_at(cu_q, order[j - 1]) + sort_grain - 1) / sort_grain < kx) {
                order[j] = order[j - 1];
                j--;
            }
            order[j] = x;
        }
    }
    int64_t w = 0;
    for (int64_t r = max_tiles - 1; r >= 0; r--) {
        for (int32_t i = 0; i < batch; i++) {
            const int32_t b = order[i];
            const int64_t n = (seq_len_at(cu_q, b) + block_q - 1) / block_q;
            if (n <= r) continue;
            for (int32_t h = 0; h < num_heads; h++) {
                if (w >= capacity) {
                    free(order);
                    return -1;
                }
                items[3 * w + 0] = b;
                items[3 * w + 1] = (int32_t)r;
                items[3 * w + 2] = h;
                w++;
            }
        }
    }
    free(order);
    return w;
}
