/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for causal scaled dot-product
 * attention and for the three steps of the unfused pipeline.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code with the HIP library.
 *
 * What it computes (sources are the four web pages on attention profiling):
 *   - The backward pass (gradients of q, k, v), derived from the forward
 *     definition below by the chain rule; see the backward section.
 *   - Queries against a longer key/value sequence (a decode step against a
 *     key/value cache, computed by the split-KV path): the queries are the
 *     last Sq of the Skv positions.
 *   - A causal sliding-window mask (each query sees its own key and the
 *     window - 1 keys before it), one of the special masks the ai-manual.ru
 *     tutorial names (section 5's conclusions, section 7) as the reason to
 *     write custom attention kernels.
 *   - A block mask: one flag per block of 64 queries x 64 keys says whether
 *     the pairs in that block may attend (combined with the causal mask when
 *     causal is set) -- the block-sparse masks of the same passages.  Rows
 *     left with no visible key give out = 0 and lse = -inf.
 *   - The attention formula softmax(Q K^T / sqrt(d_k)) V, as stated in the
 *     "technical deep-dive" of the ainews.cool AttentionProfiler article.
 *   - The five-step causal pipeline of the Hugging Face "Profiling in PyTorch
 *     (Part 3)" rendering on insight.aitobox.com, section "Naive Attention":
 *     (1) scores = q k^T, (2) scores * scale, (3) masked_fill(mask, -inf),
 *     (4) softmax over the key axis, (5) attn v.  The same list appears in the
 *     chaosnode.de summary, section "Attention unter der Lupe".
 *   - The scale 1/sqrt(head_dim) of the NaiveCausalAttention class in that same
 *     section; here scale is an explicit argument.
 *   - Layout [B, H, S, D], D fastest, from the naive_attention comment in
 *     section 1 of the ai-manual.ru tutorial.
 *
 * Readings where the pages leave a step open:
 *   - mask: key j is masked for query i when j > i (square S_q = S_k = S);
 *     masked logits are exactly -inf, so their weight is exactly 0.  The
 *     masked keys are therefore left out of the max and the sum.
 *   - grouped-query attention: query head h reads key/value head
 *     h / (Hq / Hkv) (contiguous groups); Hq must be a multiple of Hkv.
 *   - lse (log-sum-exp of a row, not on the pages): ln(sum_j exp(s_ij)) over
 *     the unmasked keys, with s already scaled.
 *   - a row with no unmasked key cannot occur under the causal or window
 *     masks (key i is always visible to query i) but can under a block mask;
 *     it gets out = 0 and lse = -inf, like the "safe softmax" of the math
 *     backend described in the SDPA section of the Hugging Face article.
 *
 * Arithmetic: every product and sum is in double; inputs are float32 arrays
 * holding the exact values the GPU sees (bf16 values are exact in float32).
 * Work is split over rows (b, h, i) between POSIX threads.
 *
 * Mutation hooks: when compiled with -DORACLE_PLANT=<n> the oracle carries a
 * deliberate mistake (see the PLANT blocks).  The test suite builds those
 * variants to check that its pins catch each kind of mistake.  The normal
 * build defines nothing and carries none of them.
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

/* ------------------------------------------------------------------------ */
/* shape and row bookkeeping                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t B, Hq, Hkv, S, D;
} shape_t;

/* Row r of the flattened [B, Hq, S] index space -> (b, h, i). */
static void split_row(const shape_t* sh, int64_t r, int64_t* b, int64_t* h, int64_t* i) {
    *i = r % sh->S;
    int64_t bh = r / sh->S;
    *h = bh % sh->Hq;
    *b = bh / sh->Hq;
}

/* Key/value head read by query head h (contiguous GQA groups). */
static int64_t kv_head(const shape_t* sh, int64_t h) {
#if ORACLE_PLANT == 5
    return h % sh->Hkv; /* planted: strided instead of contiguous groups */
#else
    return h / (sh->Hq / sh->Hkv);
#endif
}

/* First visible key for query i under a causal sliding window of `window`
 * keys (the query's own position and the window - 1 before it); window <= 0
 * means no window. */
static int64_t first_key(int64_t i, int64_t window) {
    if (window <= 0) return 0;
#if ORACLE_PLANT == 13
    const int64_t f = i - window; /* planted: window one key too wide */
#else
    const int64_t f = i - window + 1;
#endif
    return f > 0 ? f : 0;
}

/* Last visible key for query i: i when causal (mask j > i), S-1 otherwise. */
static int64_t last_key(const shape_t* sh, int64_t i, int causal) {
#if ORACLE_PLANT == 3
    if (causal) return (i + 1 < sh->S) ? i + 1 : i; /* planted: off-by-one mask */
#endif
    return causal ? i : sh->S - 1;
}

/* ------------------------------------------------------------------------ */
/* work distribution                                                        */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void* ctx, int64_t n, double* scratch);

typedef struct {
    row_fn fn;
    void* ctx;
    int64_t nrows;
    int64_t scratch_len;
    atomic_llong next;
    atomic_int failed;
} pool_t;

static void* pool_worker(void* arg) {
    pool_t* p = (pool_t*)arg;
    double* scratch = (double*)malloc((size_t)(p->scratch_len > 0 ? p->scratch_len : 1) * sizeof(double));
    if (!scratch) {
        atomic_store(&p->failed, 1);
        return NULL;
    }
    for (;;) {
        int64_t n = atomic_fetch_add(&p->next, 1);
        if (n >= p->nrows) break;
        p->fn(p->ctx, n, scratch);
    }
    free(scratch);
    return NULL;
}

/* Runs fn(ctx, n, scratch) for n in [0, nrows) on nthreads threads. */
static int run_rows(row_fn fn, void* ctx, int64_t nrows, int64_t scratch_len, int nthreads) {
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.nrows = nrows;
    p.scratch_len = scratch_len;
    atomic_init(&p.next, 0);
    atomic_init(&p.failed, 0);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -1;
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, pool_worker, &p) != 0) break;
        started = t;
    }
    pool_worker(&p);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    free(th);
    return atomic_load(&p.failed) ? -1 : 0;
}

static int check_shape(const shape_t* sh) {
    if (sh->B < 1 || sh->Hq < 1 || sh->Hkv < 1 || sh->S < 1 || sh->D < 1) return -2;
    if (sh->Hq % sh->Hkv != 0) return -2;
    return 0;
}

static int check_rows(const shape_t* sh, const int64_t* rows, int64_t nrows) {
    int64_t total = sh->B * sh->Hq * sh->S;
    for (int64_t n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= total) return -3;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* attention, one row at a time (the definition written out)                */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *q, *k, *v;
    shape_t sh;
    double scale;
    int causal;
    int64_t window; /* > 0: causal sliding window of this many keys */
    /* block mask (NULL: none): flag (b, h, qb, kb) at
     * mask[b * msb + h * msh + qb * nkb + kb], blocks of ORACLE_MASK_BLOCK */
    const uint8_t* mask;
    int64_t msb, msh;
    const int64_t* rows;
    double *out, *lse;
} attn_ctx;

#define ORACLE_MASK_BLOCK 64

/* Whether the block mask lets query i of (b, h) see key j. */
static int block_visible(const attn_ctx* c, int64_t b, int64_t h, int64_t i, int64_t j) {
    if (!c->mask) return 1;
    const int64_t nkb = (c->sh.S + ORACLE_MASK_BLOCK - 1) / ORACLE_MASK_BLOCK;
#if ORACLE_PLANT == 15
    const int64_t qb = j / ORACLE_MASK_BLOCK, kb = i / ORACLE_MASK_BLOCK; /* planted: blocks transposed */
#else
    const int64_t qb = i / ORACLE_MASK_BLOCK, kb = j / ORACLE_MASK_BLOCK;
#endif
#if ORACLE_PLANT == 16
    const int64_t base = b * c->msh + h * c->msb; /* planted: batch and head strides swapped */
#else
    const int64_t base = b * c->msb + h * c->msh;
#endif
    return c->mask[base + qb * nkb + kb] != 0;
}

/*
 * For query row (b, h, i):
 *   s_j   = scale * sum_d q[b,h,i,d] k[b,g,j,d]          j in J(i)
 *   m     = max_j s_j
 *   l     = sum_j exp(s_j - m)
 *   out_d = sum_j exp(s_j - m) v[b,g,j,d] / l
 *   lse   = m + ln l
 * with g the key/value head of h and J(i) = {0..i} (causal) or {0..S-1};
 * with a sliding window of W keys, J(i) = {max(0, i-W+1)..i}; with a block
 * mask, J(i) keeps only the keys whose (query block, key block) flag is set.
 * Subtracting m changes nothing mathematically; it only keeps exp finite.
 */
static void attn_row(void* vctx, int64_t n, double* s) {
    const attn_ctx* c = (const attn_ctx*)vctx;
    const shape_t* sh = &c->sh;
    int64_t b, h, i;
    split_row(sh, c->rows[n], &b, &h, &i);
    const int64_t g = kv_head(sh, h);
    const int64_t S = sh->S, D = sh->D;
    const float* qi = c->q + ((b * sh->Hq + h) * S + i) * D;
    const float* kb = c->k + (b * sh->Hkv + g) * S * D;
    const float* vb = c->v + (b * sh->Hkv + g) * S * D;
    double* o = c->out + n * D;
    const int64_t jl = last_key(sh, i, c->causal);
    const int64_t j0 = first_key(i, c->window);

    double m = -INFINITY;
    for (int64_t j = j0; j <= jl; ++j) {
        if (!block_visible(c, b, h, i, j)) {
            s[j] = -INFINITY; /* weight exactly 0 below */
            continue;
        }
        const float* kj = kb + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) {
#if ORACLE_PLANT == 2
            dot += (double)qi[d] * (double)kb[d * S + j]; /* planted: K read transposed */
#else
            dot += (double)qi[d] * (double)kj[d];
#endif
        }
#if ORACLE_PLANT == 1
        s[j] = dot; /* planted: scale dropped */
#else
        s[j] = c->scale * dot;
#endif
        if (s[j] > m) m = s[j];
    }
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    if (jl < 0 || m == -INFINITY) { /* no visible key: only under a block mask */
        c->lse[n] = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = j0; j <= jl; ++j) {
        if (s[j] == -INFINITY) continue;
#if ORACLE_PLANT == 4
        const double w = exp(m - s[j]); /* planted: sign flipped in the exponent */
#else
        const double w = exp(s[j] - m);
#endif
        l += w;
        const float* vj = vb + j * D;
        for (int64_t d = 0; d < D; ++d) o[d] += w * (double)vj[d];
    }
    for (int64_t d = 0; d < D; ++d) {
#if ORACLE_PLANT == 6
        (void)l; /* planted: normalisation dropped */
#else
        o[d] /= l;
#endif
    }
#if ORACLE_PLANT == 7
    c->lse[n] = m + log2(l); /* planted: wrong logarithm base */
#else
    c->lse[n] = m + log(l);
#endif
}

int oracle_attn_fwd_local_rows(const float* q, const float* k, const float* v,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                               double scale, int causal, int64_t window,
                               const int64_t* rows, int64_t nrows,
                               double* out, double* lse, int nthreads);

/*
 * Attention forward for the listed rows.  rows[n] indexes the flattened
 * [B, Hq, S] row space; out is [nrows, D], lse is [nrows].
 * q is [B,Hq,S,D], k and v are [B,Hkv,S,D], all float32, contiguous.
 * Returns 0, or a negative code on a bad shape (-2), bad row (-3) or
 * allocation failure (-1).
 */
int oracle_attn_fwd_rows(const float* q, const float* k, const float* v,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                         double scale, int causal,
                         const int64_t* rows, int64_t nrows,
                         double* out, double* lse, int nthreads) {
    return oracle_attn_fwd_local_rows(q, k, v, B, Hq, Hkv, S, D, scale, causal, 0, rows, nrows, out, lse,
                                      nthreads);
}

/*
 * As oracle_attn_fwd_rows, with a causal sliding window: query i sees keys
 * max(0, i - window + 1) .. i.  window <= 0 means no window (then causal
 * selects plain causal or full attention); window >= 1 requires causal = 1.
 */
int oracle_attn_fwd_local_rows(const float* q, const float* k, const float* v,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                               double scale, int causal, int64_t window,
                               const int64_t* rows, int64_t nrows,
                               double* out, double* lse, int nthreads) {
    attn_ctx c;
    if (window > 0 && !causal) return -2;
    c.window = window;
    c.mask = NULL;
    c.msb = c.msh = 0;
    c.q = q; c.k = k; c.v = v;
    c.sh.B = B; c.sh.Hq = Hq; c.sh.Hkv = Hkv; c.sh.S = S; c.sh.D = D;
    c.scale = scale;
    c.causal = causal ? 1 : 0;
    c.rows = rows;
    c.out = out;
    c.lse = lse;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    rc = check_rows(&c.sh, rows, nrows);
    if (rc) return rc;
    return run_rows(attn_row, &c, nrows, S, nthreads);
}

/*
 * As oracle_attn_fwd_rows, with a block mask: query i of (b, h) sees key j
 * only if mask[b * msb + h * msh + (i / 64) * nkb + j / 64] != 0, with
 * nkb = ceil(S / 64) (and j <= i when causal).  msb, msh >= 0 are element
 * strides (0 broadcasts the mask over batches or heads).  A row with no
 * visible key gets out = 0 and lse = -inf.
 */
int oracle_attn_fwd_blockmask_rows(const float* q, const float* k, const float* v,
                                   int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                                   double scale, int causal,
                                   const uint8_t* mask, int64_t msb, int64_t msh,
                                   const int64_t* rows, int64_t nrows,
                                   double* out, double* lse, int nthreads) {
    attn_ctx c;
    if (!mask || msb < 0 || msh < 0) return -2;
    c.window = 0;
    c.mask = mask;
    c.msb = msb;
    c.msh = msh;
    c.q = q; c.k = k; c.v = v;
    c.sh.B = B; c.sh.Hq = Hq; c.sh.Hkv = Hkv; c.sh.S = S; c.sh.D = D;
    c.scale = scale;
    c.causal = causal ? 1 : 0;
    c.rows = rows;
    c.out = out;
    c.lse = lse;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    rc = check_rows(&c.sh, rows, nrows);
    if (rc) return rc;
    return run_rows(attn_row, &c, nrows, S, nthreads);
}

/* ------------------------------------------------------------------------ */
/* spread of v around out (ingredient of the fp8 error bound)                */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *q, *k, *v;
    shape_t sh;
    double scale;
    int causal;
    const int64_t* rows;
    double *sw, *su;
} spread_ctx;

/*
 * With p_j = exp(s_j - m) (so max p = 1), l = sum p_j and out = sum p_j v_j / l
 * as in attn_row:
 *   sw_d = sum_j p_j |v_jd - out_d| / l      (weighted spread)
 *   su_d = sum_j     |v_jd - out_d| / l      (unweighted spread)
 * If every weight p_j is perturbed to p_j (1 + e_j) + a_j, the weighted mean
 * moves by sum_j (p_j e_j + a_j)(v_jd - out_d) / sum_j p'_j, so
 * |out' - out| <= (max|e| sw + max|a| su) / (1 - max|e| - S max|a| / l).
 */
static void spread_row(void* vctx, int64_t n, double* s) {
    const spread_ctx* c = (const spread_ctx*)vctx;
    const shape_t* sh = &c->sh;
    int64_t b, h, i;
    split_row(sh, c->rows[n], &b, &h, &i);
    const int64_t g = kv_head(sh, h);
    const int64_t S = sh->S, D = sh->D;
    const float* qi = c->q + ((b * sh->Hq + h) * S + i) * D;
    const float* kb = c->k + (b * sh->Hkv + g) * S * D;
    const float* vb = c->v + (b * sh->Hkv + g) * S * D;
    const int64_t jl = last_key(sh, i, c->causal);
    double m = -INFINITY;
    for (int64_t j = 0; j <= jl; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kb[j * D + d];
        s[j] = c->scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j <= jl; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t d = 0; d < D; ++d) {
        double o = 0.0;
        for (int64_t j = 0; j <= jl; ++j) o += s[j] * (double)vb[j * D + d];
        o /= l;
        double sw = 0.0, su = 0.0;
        for (int64_t j = 0; j <= jl; ++j) {
            const double dv = fabs((double)vb[j * D + d] - o);
            sw += s[j] * dv;
            su += dv;
        }
        c->sw[n * D + d] = sw / l;
        c->su[n * D + d] = su / l;
    }
}

int oracle_attn_fwd_spread_rows(const float* q, const float* k, const float* v,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                                double scale, int causal, const int64_t* rows, int64_t nrows,
                                double* sw, double* su, int nthreads) {
    spread_ctx c;
    c.q = q; c.k = k; c.v = v;
    c.sh.B = B; c.sh.Hq = Hq; c.sh.Hkv = Hkv; c.sh.S = S; c.sh.D = D;
    c.scale = scale;
    c.causal = causal ? 1 : 0;
    c.rows = rows;
    c.sw = sw;
    c.su = su;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    rc = check_rows(&c.sh, rows, nrows);
    if (rc) return rc;
    return run_rows(spread_row, &c, nrows, S, nthreads);
}

/* ------------------------------------------------------------------------ */
/* queries against a longer key/value sequence (decode, split-KV)            */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *q, *k, *v;
    int64_t B, Hq, Hkv, Sq, Skv, D;
    double scale;
    int causal;
    const int64_t* rows;
    double *out, *lse;
} kv_ctx;

/*
 * Query i of Sq (0-based) is the sequence position Skv - Sq + i: the queries
 * are the last Sq positions of a sequence whose keys and values are all Skv
 * positions (a decode step against a key/value cache).  Causal: it sees keys
 * 0 .. Skv - Sq + i; otherwise all Skv keys.  Then the same definition as
 * attn_row: s_j = scale q_i . k_j, out = sum_j exp(s_j - m) v_j / l,
 * lse = m + ln l.
 */
static void kv_row(void* vctx, int64_t n, double* s) {
    const kv_ctx* c = (const kv_ctx*)vctx;
    const int64_t r = c->rows[n];
    const int64_t i = r % c->Sq, bh = r / c->Sq;
    const int64_t h = bh % c->Hq, b = bh / c->Hq;
    const int64_t g = h / (c->Hq / c->Hkv);
    const int64_t D = c->D;
    const float* qi = c->q + r * D;
    const float* kb = c->k + (b * c->Hkv + g) * c->Skv * D;
    const float* vb = c->v + (b * c->Hkv + g) * c->Skv * D;
    double* o = c->out + n * D;
#if ORACLE_PLANT == 14
    const int64_t jl = c->causal ? i : c->Skv - 1; /* planted: top-left alignment */
#else
    const int64_t jl = c->causal ? c->Skv - c->Sq + i : c->Skv - 1;
#endif
    double m = -INFINITY;
    for (int64_t j = 0; j <= jl; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kb[j * D + d];
        s[j] = c->scale * dot;
        if (s[j] > m) m = s[j];
    }
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    double l = 0.0;
    for (int64_t j = 0; j <= jl; ++j) {
        const double w = exp(s[j] - m);
        l += w;
        for (int64_t d = 0; d < D; ++d) o[d] += w * (double)vb[j * D + d];
    }
    for (int64_t d = 0; d < D; ++d) o[d] /= l;
    c->lse[n] = m + log(l);
}

/*
 * Attention of q [B, Hq, Sq, D] against k, v [B, Hkv, Skv, D] for the listed
 * rows of the flattened [B, Hq, Sq] space; out [nrows, D], lse [nrows].
 * Requires 1 <= Sq <= Skv.
 */
int oracle_attn_fwd_kv_rows(const float* q, const float* k, const float* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                            double scale, int causal, const int64_t* rows, int64_t nrows,
                            double* out, double* lse, int nthreads) {
    kv_ctx c;
    c.q = q; c.k = k; c.v = v;
    c.B = B; c.Hq = Hq; c.Hkv = Hkv; c.Sq = Sq; c.Skv = Skv; c.D = D;
    c.scale = scale;
    c.causal = causal ? 1 : 0;
    c.rows = rows;
    c.out = out;
    c.lse = lse;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < Sq || D < 1 || Hq % Hkv != 0) return -2;
    const int64_t total = B * Hq * Sq;
    for (int64_t n = 0; n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= total) return -3;
    return run_rows(kv_row, &c, nrows, Skv, nthreads);
}

/* ------------------------------------------------------------------------ */
/* the unfused pipeline, step by step                                       */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *a, *b;
    shape_t sh;
    double scale;
    int causal;
    const int64_t* rows;
    double *out, *lse;
} step_ctx;

/* Step 1 for one row: scores[b,h,i,j] = sum_d q[b,h,i,d] k[b,g,j,d], all j. */
static void qk_row(void* vctx, int64_t n, double* unused) {
    (void)unused;
    const step_ctx* c = (const step_ctx*)vctx;
    const shape_t* sh = &c->sh;
    int64_t b, h, i;
    split_row(sh, c->rows[n], &b, &h, &i);
    const int64_t g = kv_head(sh, h);
    const int64_t S = sh->S, D = sh->D;
    const float* qi = c->a + ((b * sh->Hq + h) * S + i) * D;
    const float* kb = c->b + (b * sh->Hkv + g) * S * D;
    double* o = c->out + n * S;
    for (int64_t j = 0; j < S; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kb[j * D + d];
        o[j] = dot;
    }
}

/* Unscaled scores q k^T for the listed rows; out is [nrows, S]. */
int oracle_qk_scores_rows(const float* q, const float* k,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                          const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    step_ctx c;
    memset(&c, 0, sizeof c);
    c.a = q; c.b = k;
    c.sh.B = B; c.sh.Hq = Hq; c.sh.Hkv = Hkv; c.sh.S = S; c.sh.D = D;
    c.rows = rows;
    c.out = out;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    rc = check_rows(&c.sh, rows, nrows);
    if (rc) return rc;
    return run_rows(qk_row, &c, nrows, 0, nthreads);
}

/*
 * Steps 2-4 for one row of an [B,H,S,S] score matrix: t_j = scale * x_j;
 * t_j = -inf for masked j; p_j = exp(t_j - max t) / sum exp(t - max t).
 * Masked entries get p = 0 exactly.  lse = max t + ln(sum exp(t - max t)).
 */
static void softmax_row(void* vctx, int64_t n, double* t) {
    const step_ctx* c = (const step_ctx*)vctx;
    const shape_t* sh = &c->sh;
    int64_t b, h, i;
    split_row(sh, c->rows[n], &b, &h, &i);
    const int64_t S = sh->S;
    const float* x = c->a + ((b * sh->Hq + h) * S + i) * S;
    double* p = c->out + n * S;
    const int64_t jl = last_key(sh, i, c->causal);
    double m = -INFINITY;
    for (int64_t j = 0; j < S; ++j) {
        t[j] = (j <= jl) ? c->scale * (double)x[j] : -INFINITY;
        if (t[j] > m) m = t[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        p[j] = (j <= jl) ? exp(t[j] - m) : 0.0;
        l += p[j];
    }
    for (int64_t j = 0; j < S; ++j) p[j] /= l;
    if (c->lse) c->lse[n] = m + log(l);
}

/* Masked row softmax of fp32 scores [B,H,S,S] for the listed rows (H = Hq);
 * p is [nrows, S]; lse is [nrows] or NULL. */
int oracle_masked_softmax_rows(const float* scores,
                               int64_t B, int64_t H, int64_t S,
                               double scale, int causal,
                               const int64_t* rows, int64_t nrows,
                               double* p, double* lse, int nthreads) {
    step_ctx c;
    memset(&c, 0, sizeof c);
    c.a = scores;
    c.sh.B = B; c.sh.Hq = H; c.sh.Hkv = H; c.sh.S = S; c.sh.D = 1;
    c.scale = scale;
    c.causal = causal ? 1 : 0;
    c.rows = rows;
    c.out = p;
    c.lse = lse;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    rc = check_rows(&c.sh, rows, nrows);
    if (rc) return rc;
    return run_rows(softmax_row, &c, nrows, S, nthreads);
}

/* Step 5 for one row: out[b,h,i,d] = sum_j p[b,h,i,j] v[b,g,j,d]. */
static void pv_row(void* vctx, int64_t n, double* unused) {
    (void)unused;
    const step_ctx* c = (const step_ctx*)vctx;
    const shape_t* sh = &c->sh;
    int64_t b, h, i;
    split_row(sh, c->rows[n], &b, &h, &i);
    const int64_t g = kv_head(sh, h);
    const int64_t S = sh->S, D = sh->D;
    const float* pi = c->a + ((b * sh->Hq + h) * S + i) * S;
    const float* vb = c->b + (b * sh->Hkv + g) * S * D;
    double* o = c->out + n * D;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        const double w = (double)pi[j];
        for (int64_t d = 0; d < D; ++d) o[d] += w * (double)vb[j * D + d];
    }
}

/* P V for the listed rows; p is [B,Hq,S,S], v is [B,Hkv,S,D]; out [nrows, D]. */
int oracle_pv_rows(const float* p, const float* v,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                   const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    step_ctx c;
    memset(&c, 0, sizeof c);
    c.a = p; c.b = v;
    c.sh.B = B; c.sh.Hq = Hq; c.sh.Hkv = Hkv; c.sh.S = S; c.sh.D = D;
    c.rows = rows;
    c.out = out;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    rc = check_rows(&c.sh, rows, nrows);
    if (rc) return rc;
    return run_rows(pv_row, &c, nrows, 0, nthreads);
}

/* ------------------------------------------------------------------------ */
/* backward: gradients of the forward above                                  */
/* ------------------------------------------------------------------------ */

/*
 * The forward is out_i = sum_j p_ij v_j with p_ij = exp(s_ij) / sum_j' exp(s_ij')
 * and s_ij = scale * q_i . k_j over the visible keys.  For a loss with
 * dL/dout = dout (and no gradient reaching lse), the chain rule gives
 *   dv_j  = sum_i p_ij dout_i
 *   dp_ij = dout_i . v_j
 *   ds_ij = p_ij (dp_ij - delta_i),  delta_i = sum_j p_ij dp_ij
 *   dq_i  = scale * sum_j ds_ij k_j
 *   dk_j  = scale * sum_i ds_ij q_i
 * where the sums over i run over every query (of every query head sharing
 * key/value head g) that sees key j.  The pages only say that the flash
 * backward is harder to get right than the forward (ai-manual.ru tutorial,
 * section 6); the formulas are the derivative of the forward definition.
 *
 * Pass 1 (one query row at a time): lse_i, delta_i and dq_i.
 * Pass 2 (one key row at a time): dk_j and dv_j, recomputing p_ij from the
 * lse_i and delta_i of pass 1.
 */
typedef struct {
    const float *q, *k, *v, *dout;
    shape_t sh;
    double scale;
    int causal;
    const int64_t* rows;
    double *lse, *delta, *dq;          /* pass 1 outputs, one per listed row */
    const double *lse_all, *delta_all; /* pass 2 inputs, [B, Hq, S]          */
    double *dk, *dv;                   /* pass 2 outputs, one per listed key */
} bwd_ctx;

/* scratch: s[S] then dp[S] */
static void bwd_query_row(void* vctx, int64_t n, double* scratch) {
    const bwd_ctx* c = (const bwd_ctx*)vctx;
    const shape_t* sh = &c->sh;
    int64_t b, h, i;
    split_row(sh, c->rows[n], &b, &h, &i);
    const int64_t g = kv_head(sh, h);
    const int64_t S = sh->S, D = sh->D;
    const float* qi = c->q + ((b * sh->Hq + h) * S + i) * D;
    const float* doi = c->dout + ((b * sh->Hq + h) * S + i) * D;
    const float* kb = c->k + (b * sh->Hkv + g) * S * D;
    const float* vb = c->v + (b * sh->Hkv + g) * S * D;
    double* s = scratch;
    double* dp = scratch + S;
    double* dq = c->dq + n * D;
    const int64_t jl = last_key(sh, i, c->causal);
    double m = -INFINITY;
    for (int64_t j = 0; j <= jl; ++j) {
        double dot = 0.0, dpj = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            dot += (double)qi[d] * (double)kb[j * D + d];
            dpj += (double)doi[d] * (double)vb[j * D + d];
        }
        s[j] = c->scale * dot;
        dp[j] = dpj;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j <= jl; ++j) l += exp(s[j] - m);
    const double lse = m + log(l);
    double delta = 0.0;
    for (int64_t j = 0; j <= jl; ++j) delta += exp(s[j] - lse) * dp[j];
    for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
    for (int64_t j = 0; j <= jl; ++j) {
        const double p = exp(s[j] - lse);
#if ORACLE_PLANT == 8
        const double ds = p * dp[j]; /* planted: delta left out */
#else
        const double ds = p * (dp[j] - delta);
#endif
        for (int64_t d = 0; d < D; ++d) {
#if ORACLE_PLANT == 10
            dq[d] += ds * (double)vb[j * D + d]; /* planted: v in place of k */
#else
            dq[d] += ds * (double)kb[j * D + d];
#endif
        }
    }
    for (int64_t d = 0; d < D; ++d) dq[d] *= c->scale;
    c->lse[n] = lse;
    c->delta[n] = delta;
}

static void bwd_key_row(void* vctx, int64_t n, double* unused) {
    (void)unused;
    const bwd_ctx* c = (const bwd_ctx*)vctx;
    const shape_t* sh = &c->sh;
    const int64_t S = sh->S, D = sh->D;
    const int64_t j = c->rows[n] % S;
    const int64_t bg = c->rows[n] / S;
    const int64_t g = bg % sh->Hkv, b = bg / sh->Hkv;
    const float* kj = c->k + (bg * S + j) * D;
    const float* vj = c->v + (bg * S + j) * D;
    double* dk = c->dk + n * D;
    double* dv = c->dv + n * D;
    for (int64_t d = 0; d < D; ++d) dk[d] = dv[d] = 0.0;
    for (int64_t h = 0; h < sh->Hq; ++h) {
        if (kv_head(sh, h) != g) continue;
#if ORACLE_PLANT == 12
        if (h != g * (sh->Hq / sh->Hkv)) continue; /* planted: only the group's first head */
#endif
        for (int64_t i = 0; i < S; ++i) {
#if ORACLE_PLANT == 11
            if (c->causal && i > j) continue; /* planted: mask direction flipped */
#else
            if (last_key(sh, i, c->causal) < j) continue; /* query i does not see key j */
#endif
            const int64_t row = (b * sh->Hq + h) * S + i;
            const float* qi = c->q + row * D;
            const float* doi = c->dout + row * D;
            double dot = 0.0, dp = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                dot += (double)qi[d] * (double)kj[d];
                dp += (double)doi[d] * (double)vj[d];
            }
            const double p = exp(c->scale * dot - c->lse_all[row]);
            const double ds = p * (dp - c->delta_all[row]);
            for (int64_t d = 0; d < D; ++d) {
                dv[d] += p * (double)doi[d];
#if ORACLE_PLANT == 9
                dk[d] += ds * (double)qi[d]; /* planted: scale dropped */
#else
                dk[d] += c->scale * ds * (double)qi[d];
#endif
            }
        }
    }
}

/*
 * Pass 1 for the listed query rows (indices into [B, Hq, S]): lse [nrows],
 * delta [nrows], dq [nrows, D].  dout has the shape of q.
 */
int oracle_attn_bwd_rows(const float* q, const float* k, const float* v, const float* dout,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                         double scale, int causal, const int64_t* rows, int64_t nrows,
                         double* lse, double* delta, double* dq, int nthreads) {
    bwd_ctx c;
    memset(&c, 0, sizeof c);
    c.q = q; c.k = k; c.v = v; c.dout = dout;
    c.sh.B = B; c.sh.Hq = Hq; c.sh.Hkv = Hkv; c.sh.S = S; c.sh.D = D;
    c.scale = scale;
    c.causal = causal ? 1 : 0;
    c.rows = rows;
    c.lse = lse; c.delta = delta; c.dq = dq;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    rc = check_rows(&c.sh, rows, nrows);
    if (rc) return rc;
    return run_rows(bwd_query_row, &c, nrows, 2 * S, nthreads);
}

/*
 * Pass 2 for the listed key rows (indices into [B, Hkv, S]): dk, dv
 * [nkeys, D].  lse_all and delta_all are pass 1's results for every query
 * row, [B, Hq, S].
 */
int oracle_attn_bwd_keys(const float* q, const float* k, const float* v, const float* dout,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t S, int64_t D,
                         double scale, int causal, const double* lse_all, const double* delta_all,
                         const int64_t* keys, int64_t nkeys, double* dk, double* dv, int nthreads) {
    bwd_ctx c;
    memset(&c, 0, sizeof c);
    c.q = q; c.k = k; c.v = v; c.dout = dout;
    c.sh.B = B; c.sh.Hq = Hq; c.sh.Hkv = Hkv; c.sh.S = S; c.sh.D = D;
    c.scale = scale;
    c.causal = causal ? 1 : 0;
    c.rows = keys;
    c.lse_all = lse_all; c.delta_all = delta_all;
    c.dk = dk; c.dv = dv;
    int rc = check_shape(&c.sh);
    if (rc) return rc;
    const int64_t total = B * Hkv * S;
    for (int64_t n = 0; n < nkeys; ++n)
        if (keys[n] < 0 || keys[n] >= total) return -3;
    return run_rows(bwd_key_row, &c, nkeys, 0, nthreads);
}

/* Which mistake (0 = none) this build carries; lets a test confirm a variant. */
int oracle_plant_id(void) { return ORACLE_PLANT; }
