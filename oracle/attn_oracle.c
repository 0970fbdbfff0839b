/*
 * attn_oracle.c — plain, slow fp64 CPU reference for scaled-dot-product
 * attention. TEST INFRASTRUCTURE ONLY: it is called by the tests, by the
 * smoke check and by the bench's CPU-baseline leg, never by the product path.
 * It shares no code with the GPU library.
 *
 * Pages, cited by title and section:
 *  [p1] "AI Infra 入门：RMSNorm、Softmax、Causal Mask、Sampling 的数学与底层优化"
 *  [p2] "05 · Tích vô hướng, Softmax và toán của Attention" (inference-notes)
 *  [p3] "MLA 矩阵乘法吸收的数值稳定性治理" (gsyq.cn)
 *  [p4] "Bộ 06 · Bên trong model" (inference-notes revision cards)
 *  [p5] "第11节：Attention 实现（Flash vs Fallback）" (minimind course notes)
 *
 * What it computes, for one query row q against keys K[0..n) and values
 * V[0..n), all held exactly in double:
 *
 *   s_j  = scale · Σ_t q_t · K_jt        dot product, ÷√d folded into scale
 *                                        [p2] §1, [p5] §4
 *   s_j  = −∞ where the explicit mask is set (future key j > i)
 *                                        [p1] §3, [p4] Q2, [p5] §3
 *   pass 1  m   = max_j s_j              safe softmax, [p1] §2, [p4] Q1
 *   pass 2  ℓ   = Σ_j exp(s_j − m)
 *   pass 3  P_j = exp(s_j − m) / ℓ ;  O_d = Σ_j P_j · V_jd     [p2] §3
 *   LSE = m + ln ℓ   natural log, so softmax_j = exp(s_j − LSE)  [p1] §3
 *
 * These are the three passes of the safe softmax (maximum, denominator,
 * result) that [p1] §3 contrasts with the one-pass online form: the oracle
 * states the definition, the GPU kernels implement the online algorithm.
 *
 * Prefill builds a dense boolean mask M[r][j] = (j > row_r) for the rows it
 * evaluates (the full N×N matrix when all rows are asked for) and sets the
 * score to −∞ where it is set, in the order of the fallback flow of [p5] §6
 * (scores, causal mask, softmax, weighted values; no padding, no dropout).
 * Decode uses no mask (the single query sees only history, [p1] §3) and
 * reads only the first kv_len cache slots, never unfilled ones ([p4] Q3).
 *
 * Backward of the causal prefill: the forward weights P are recomputed by
 * the same definition, then the gradients of the softmax and of the two
 * products follow the chain rule written out (the LSE kept by the forward
 * is what lets a fused kernel recompute P exactly, [p1] §3).
 *
 * Chunked prefill: a chunk of Nq new tokens whose K/V were appended to a
 * cache, so a sequence's keys are [history | chunk] ([p5] §3: K = past K
 * followed by current K). The score matrix [Nq][kv_len] gets the triu(1)
 * mask on its last Nq columns only: chunk row i sees every history key and
 * chunk keys 0..i ([p5] §3). Ragged batches give every sequence its own
 * kv_len; a sequence with kv_len = 0 attends to nothing, so its sums are
 * empty: O = 0 and LSE = ln 0 = −∞.
 *
 * GQA: query head hq reads K/V head hq / (Hq/Hkv): contiguous groups of
 * Hq/Hkv query heads share one K/V head ([p2] §4).
 * MLA absorbed: one latent head shared by every query head; the key is the
 * whole Dqk-wide row (latent | rope), the value its first Dv channels
 * ([p3] §一, §三).
 *
 * Parallelism: rows are independent; they are split into contiguous ranges
 * over `threads` POSIX threads. Summation order inside a row is fixed
 * (ascending t, ascending j), so results do not depend on the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread -lm (no fused
 * multiply-add contraction, no fast-math reassociation).
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* One query row against n keys (three-pass safe softmax). `mask` is NULL or
 * n flags (nonzero = masked). `s` is caller scratch of n doubles. `p_out`
 * is NULL or n doubles receiving the softmax weights. */
static void attend_row(const double *q, const double *k, long k_stride, int dk,
                       const double *v, long v_stride, int dv, int n,
                       const unsigned char *mask, double scale, double *s,
                       double *o, double *lse, double *p_out)
{
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        const double *kj = k + (long)j * k_stride;
        for (int t = 0; t < dk; ++t)
            dot += q[t] * kj[t];
        s[j] = scale * dot;
        if (mask && mask[j])
            s[j] = -INFINITY;
    }
    /* pass 1: row maximum */
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (s[j] > m)
            m = s[j];
    /* pass 2: denominator */
    double l = 0.0;
    for (int j = 0; j < n; ++j)
        l += exp(s[j] - m);
    /* pass 3: normalised weights and weighted sum of values */
    for (int d = 0; d < dv; ++d)
        o[d] = 0.0;
    for (int j = 0; j < n; ++j) {
        double p = exp(s[j] - m) / l;
        if (p_out)
            p_out[j] = p;
        const double *vj = v + (long)j * v_stride;
        for (int d = 0; d < dv; ++d)
            o[d] += p * vj[d];
    }
    *lse = m + log(l);
}

/* ------------------------------------------------------------ threading --- */
typedef void (*row_fn)(void *ctx, long unit, double *scratch);

typedef struct {
    row_fn fn;
    void *ctx;
    long begin, end;
    int scratch_n;
} range_job;

static void *run_range(void *arg)
{
    range_job *job = (range_job *)arg;
    double *scratch = (double *)malloc(sizeof(double) * (size_t)(job->scratch_n > 0 ? job->scratch_n : 1));
    if (!scratch)
        return (void *)1;
    for (long u = job->begin; u < job->end; ++u)
        job->fn(job->ctx, u, scratch);
    free(scratch);
    return NULL;
}

static int run_units(row_fn fn, void *ctx, long units, int scratch_n, int threads)
{
    if (threads < 1)
        threads = 1;
    if (threads > units)
        threads = units > 0 ? (int)units : 1;
    range_job *jobs = (range_job *)calloc((size_t)threads, sizeof(range_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -1;
    }
    int rc = 0;
    for (int t = 0; t < threads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = units * t / threads;
        jobs[t].end = units * (t + 1) / threads;
        jobs[t].scratch_n = scratch_n;
    }
    for (int t = 1; t < threads; ++t)
        if (pthread_create(&tids[t], NULL, run_range, &jobs[t]) != 0)
            rc = -1;
    if (run_range(&jobs[0]) != NULL)
        rc = -1;
    for (int t = 1; t < threads; ++t) {
        void *ret = NULL;
        pthread_join(tids[t], &ret);
        if (ret != NULL)
            rc = -1;
    }
    free(jobs);
    free(tids);
    return rc;
}

/* --------------------------------------------------------------- prefill --- */
typedef struct {
    const double *q, *k, *v;
    int B, Hq, Hkv, N, D, n_rows;
    double scale;
    const unsigned char *mask; /* [n_rows][N] */
    double *o, *lse, *p;
} prefill_ctx;

static void prefill_unit(void *vctx, long unit, double *scratch)
{
    prefill_ctx *c = (prefill_ctx *)vctx;
    long r = unit % c->n_rows;
    long bh = unit / c->n_rows;
    int hq = (int)(bh % c->Hq);
    int b = (int)(bh / c->Hq);
    int hkv = hq / (c->Hq / c->Hkv);
    const double *q = c->q + ((long)bh * c->n_rows + r) * c->D;
    const double *k = c->k + ((long)b * c->Hkv + hkv) * (long)c->N * c->D;
    const double *v = c->v + ((long)b * c->Hkv + hkv) * (long)c->N * c->D;
    attend_row(q, k, c->D, c->D, v, c->D, c->D, c->N, c->mask + r * (long)c->N,
               c->scale, scratch, c->o + ((long)bh * c->n_rows + r) * c->D,
               c->lse + (long)bh * c->n_rows + r,
               c->p ? c->p + ((long)bh * c->n_rows + r) * c->N : NULL);
}

/* Causal prefill, N queries against N keys (mask M[i][j] = j > i).
 * q:   [B][Hq][n_rows][D]  — only the evaluated rows, in `rows` order
 * k,v: [B][Hkv][N][D]
 * rows: n_rows query indices in [0, N)
 * o: [B][Hq][n_rows][D], lse: [B][Hq][n_rows], p: NULL or [B][Hq][n_rows][N]
 * Returns 0, or -1 on bad arguments / allocation failure. */
int oracle_prefill_causal(const double *q, const double *k, const double *v,
                          int B, int Hq, int Hkv, int N, int D, double scale,
                          const int *rows, int n_rows, double *o, double *lse,
                          double *p, int threads)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1 || n_rows < 1 || Hq % Hkv)
        return -1;
    unsigned char *mask = (unsigned char *)malloc((size_t)n_rows * (size_t)N);
    if (!mask)
        return -1;
    for (long r = 0; r < n_rows; ++r) {
        if (rows[r] < 0 || rows[r] >= N) {
            free(mask);
            return -1;
        }
        for (int j = 0; j < N; ++j)
            mask[r * N + j] = (unsigned char)(j > rows[r]);
    }
    prefill_ctx c = {q, k, v, B, Hq, Hkv, N, D, n_rows, scale, mask, o, lse, p};
    int rc = run_units(prefill_unit, &c, (long)B * Hq * n_rows, N, threads);
    free(mask);
    return rc;
}

/* ------------------------------------------------ causal prefill backward --- */
typedef struct {
    const double *q, *k, *v, *dout;
    int B, Hq, Hkv, N, D;
    double scale;
    double *dq, *dk, *dv;
} bwd_ctx;

/* One (b, K/V head): every query head of its group in turn. Scratch: the
 * N×N weights P and the N×N dP of one head, and the causal mask row. */
static void bwd_unit(void *vctx, long unit, double *scratch)
{
    bwd_ctx *c = (bwd_ctx *)vctx;
    const int N = c->N, D = c->D, G = c->Hq / c->Hkv;
    const int b = (int)(unit / c->Hkv), hkv = (int)(unit % c->Hkv);
    double *P = scratch, *dP = scratch + (long)N * N, *s = dP + (long)N * N;
    unsigned char *mask = (unsigned char *)(s + N);
    const long kv_off = ((long)b * c->Hkv + hkv) * (long)N * D;
    const double *K = c->k + kv_off, *V = c->v + kv_off;
    double *dK = c->dk + kv_off, *dV = c->dv + kv_off;
    for (long x = 0; x < (long)N * D; ++x)
        dK[x] = dV[x] = 0.0;
    for (int g = 0; g < G; ++g) {
        const long q_off = ((long)b * c->Hq + hkv * G + g) * (long)N * D;
        const double *Q = c->q + q_off, *dO = c->dout + q_off;
        double *dQ = c->dq + q_off;
        /* forward weights, row by row: the same definition as the prefill */
        for (int i = 0; i < N; ++i) {
            double o_unused[1], lse_unused;
            for (int j = 0; j < N; ++j)
                mask[j] = (unsigned char)(j > i);
            attend_row(Q + (long)i * D, K, D, D, V, D, 0, N, mask, c->scale, s, o_unused,
                       &lse_unused, P + (long)i * N);
        }
        /* dP_ij = dO_i · V_j ;  dV_j += Σ_i P_ij dO_i */
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j) {
                double acc = 0.0;
                for (int t = 0; t < D; ++t)
                    acc += dO[(long)i * D + t] * V[(long)j * D + t];
                dP[(long)i * N + j] = acc;
            }
        for (int j = 0; j < N; ++j)
            for (int i = 0; i < N; ++i) {
                const double p = P[(long)i * N + j];
                for (int t = 0; t < D; ++t)
                    dV[(long)j * D + t] += p * dO[(long)i * D + t];
            }
        /* softmax Jacobian: dS_ij = P_ij (dP_ij − Σ_l P_il dP_il), kept in dP */
        for (int i = 0; i < N; ++i) {
            double Di = 0.0;
            for (int j = 0; j < N; ++j)
                Di += P[(long)i * N + j] * dP[(long)i * N + j];
            for (int j = 0; j < N; ++j)
                dP[(long)i * N + j] = P[(long)i * N + j] * (dP[(long)i * N + j] - Di);
        }
        /* S = scale·Q·Kᵀ:  dQ_i = scale Σ_j dS_ij K_j ;  dK_j += scale Σ_i dS_ij Q_i */
        for (int i = 0; i < N; ++i)
            for (int t = 0; t < D; ++t) {
                double acc = 0.0;
                for (int j = 0; j < N; ++j)
                    acc += dP[(long)i * N + j] * K[(long)j * D + t];
                dQ[(long)i * D + t] = c->scale * acc;
            }
        for (int j = 0; j < N; ++j)
            for (int t = 0; t < D; ++t) {
                double acc = 0.0;
                for (int i = 0; i < N; ++i)
                    acc += dP[(long)i * N + j] * Q[(long)i * D + t];
                dK[(long)j * D + t] += c->scale * acc;
            }
    }
}

/* Gradients of the causal prefill (N queries against N keys, mask j > i)
 * for an upstream gradient dout = ∂L/∂O:
 *   dV = Pᵀ·dO,  dP = dO·Vᵀ,  dS = P ∘ (dP − rowsum(P ∘ dP)),
 *   dQ = scale·dS·K,  dK = scale·dSᵀ·Q,
 * with dK and dV summed over the query heads that share a K/V head.
 * q, dout, dq: [B][Hq][N][D]; k, v, dk, dv: [B][Hkv][N][D]. */
int oracle_prefill_causal_backward(const double *q, const double *k, const double *v,
                                   const double *dout, int B, int Hq, int Hkv, int N, int D,
                                   double scale, double *dq, double *dk, double *dv,
                                   int threads)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1 || Hq % Hkv)
        return -1;
    bwd_ctx c = {q, k, v, dout, B, Hq, Hkv, N, D, scale, dq, dk, dv};
    /* scratch: P and dP (N×N each), the score row, and N mask bytes */
    const long scratch = 2L * N * N + N + (N + 7) / 8 + 1;
    return run_units(bwd_unit, &c, (long)B * Hkv, (int)scratch, threads);
}

/* ------------------------------------------- chunked prefill on a cache --- */
typedef struct {
    const double *q, *k, *v;
    int B, Hq, Hkv, kv_cap, D, n_rows;
    const int *kv_lens;
    double scale;
    const unsigned char *mask; /* [B][n_rows][kv_cap] */
    double *o, *lse;
} chunk_ctx;

static void chunk_unit(void *vctx, long unit, double *scratch)
{
    chunk_ctx *c = (chunk_ctx *)vctx;
    long r = unit % c->n_rows;
    long bh = unit / c->n_rows;
    int hq = (int)(bh % c->Hq);
    int b = (int)(bh / c->Hq);
    int hkv = hq / (c->Hq / c->Hkv);
    const double *k = c->k + ((long)b * c->Hkv + hkv) * (long)c->kv_cap * c->D;
    const double *v = c->v + ((long)b * c->Hkv + hkv) * (long)c->kv_cap * c->D;
    attend_row(c->q + ((long)bh * c->n_rows + r) * c->D, k, c->D, c->D, v, c->D, c->D,
               c->kv_lens[b], c->mask + ((long)b * c->n_rows + r) * c->kv_cap, c->scale,
               scratch, c->o + ((long)bh * c->n_rows + r) * c->D,
               c->lse + (long)bh * c->n_rows + r, NULL);
}

/* Chunked prefill against a cache: sequence b holds kv_lens[b] keys, the
 * last Nq of which belong to the chunk (Nq <= kv_lens[b] <= kv_cap).
 * Mask (triu(1) on the last Nq columns, [p5] §3): with P = kv_lens[b] − Nq
 * history keys, key j is masked for chunk row i iff j >= P and j − P > i.
 * q:   [B][Hq][n_rows][D] — the evaluated chunk rows, in `rows` order
 * k,v: [B][Hkv][kv_cap][D]
 * rows: n_rows chunk row indices in [0, Nq)
 * o: [B][Hq][n_rows][D], lse: [B][Hq][n_rows]. */
int oracle_prefill_chunked(const double *q, const double *k, const double *v,
                           int B, int Hq, int Hkv, int Nq, const int *kv_lens,
                           int kv_cap, int D, double scale, const int *rows,
                           int n_rows, double *o, double *lse, int threads)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || D < 1 || n_rows < 1 || Hq % Hkv || kv_cap < Nq)
        return -1;
    for (int b = 0; b < B; ++b)
        if (kv_lens[b] < Nq || kv_lens[b] > kv_cap)
            return -1;
    for (int r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= Nq)
            return -1;
    unsigned char *mask = (unsigned char *)malloc((size_t)B * n_rows * (size_t)kv_cap);
    if (!mask)
        return -1;
    for (int b = 0; b < B; ++b) {
        const int past = kv_lens[b] - Nq;
        for (long r = 0; r < n_rows; ++r) {
            unsigned char *m = mask + ((long)b * n_rows + r) * kv_cap;
            for (int j = 0; j < kv_cap; ++j)
                m[j] = (unsigned char)(j >= past && j - past > rows[r]);
        }
    }
    chunk_ctx c = {q, k, v, B, Hq, Hkv, kv_cap, D, n_rows, kv_lens, scale, mask, o, lse};
    int rc = run_units(chunk_unit, &c, (long)B * Hq * n_rows, kv_cap, threads);
    free(mask);
    return rc;
}

/* ------------------------------------------------------------ GQA decode --- */
typedef struct {
    const double *q, *k, *v;
    int B, Hq, Hkv, kv_len, kv_cap, D;
    const int *kv_lens; /* NULL: every sequence is filled to kv_len */
    double scale;
    double *o, *lse, *p;
} decode_ctx;

static void decode_unit(void *vctx, long unit, double *scratch)
{
    decode_ctx *c = (decode_ctx *)vctx;
    int hq = (int)(unit % c->Hq);
    int b = (int)(unit / c->Hq);
    int hkv = hq / (c->Hq / c->Hkv);
    const double *k = c->k + ((long)b * c->Hkv + hkv) * (long)c->kv_cap * c->D;
    const double *v = c->v + ((long)b * c->Hkv + hkv) * (long)c->kv_cap * c->D;
    const int n = c->kv_lens ? c->kv_lens[b] : c->kv_len;
    attend_row(c->q + unit * c->D, k, c->D, c->D, v, c->D, c->D, n, NULL,
               c->scale, scratch, c->o + unit * c->D, c->lse + unit,
               c->p ? c->p + unit * c->kv_len : NULL);
}

/* Single-query decode over a K/V cache filled to kv_len (no mask).
 * q: [B][Hq][D]; k,v: [B][Hkv][kv_cap][D]; o: [B][Hq][D]; lse: [B][Hq];
 * p: NULL or [B][Hq][kv_len]. */
int oracle_decode_gqa(const double *q, const double *k, const double *v,
                      int B, int Hq, int Hkv, int kv_len, int kv_cap, int D,
                      double scale, double *o, double *lse, double *p, int threads)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv || kv_len < 1 || kv_len > kv_cap)
        return -1;
    decode_ctx c = {q, k, v, B, Hq, Hkv, kv_len, kv_cap, D, NULL, scale, o, lse, p};
    return run_units(decode_unit, &c, (long)B * Hq, kv_len, threads);
}

/* Ragged decode: sequence b is filled to kv_lens[b] (0 <= kv_lens[b] <=
 * kv_cap); otherwise as oracle_decode_gqa. No weights are returned. */
int oracle_decode_gqa_ragged(const double *q, const double *k, const double *v,
                             int B, int Hq, int Hkv, const int *kv_lens, int kv_cap,
                             int D, double scale, double *o, double *lse, int threads)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv || kv_cap < 1)
        return -1;
    for (int b = 0; b < B; ++b)
        if (kv_lens[b] < 0 || kv_lens[b] > kv_cap)
            return -1;
    decode_ctx c = {q, k, v, B, Hq, Hkv, 0, kv_cap, D, kv_lens, scale, o, lse, NULL};
    return run_units(decode_unit, &c, (long)B * Hq, kv_cap, threads);
}

/* ----------------------------------------------------- MLA absorbed decode --- */
typedef struct {
    const double *q, *c;
    int B, Hq, kv_len, kv_cap, Dqk, Dv;
    const int *kv_lens; /* NULL: every sequence is filled to kv_len */
    double scale;
    double *o, *lse;
} mla_ctx;

static void mla_unit(void *vctx, long unit, double *scratch)
{
    mla_ctx *c = (mla_ctx *)vctx;
    int b = (int)(unit / c->Hq);
    const double *lat = c->c + (long)b * c->kv_cap * c->Dqk;
    /* key = the whole row (latent | rope); value = its first Dv channels */
    attend_row(c->q + unit * c->Dqk, lat, c->Dqk, c->Dqk, lat, c->Dqk, c->Dv,
               c->kv_lens ? c->kv_lens[b] : c->kv_len, NULL, c->scale, scratch,
               c->o + unit * c->Dv, c->lse + unit, NULL);
}

/* q: [B][Hq][Dqk]; ckv: [B][kv_cap][Dqk]; o: [B][Hq][Dv]; lse: [B][Hq]. */
int oracle_decode_mla(const double *q, const double *ckv, int B, int Hq,
                      int kv_len, int kv_cap, int Dqk, int Dv, double scale,
                      double *o, double *lse, int threads)
{
    if (B < 1 || Hq < 1 || Dqk < 1 || Dv < 1 || Dv > Dqk || kv_len < 1 || kv_len > kv_cap)
        return -1;
    mla_ctx c = {q, ckv, B, Hq, kv_len, kv_cap, Dqk, Dv, NULL, scale, o, lse};
    return run_units(mla_unit, &c, (long)B * Hq, kv_len, threads);
}

/* Ragged absorbed-MLA decode: sequence b is filled to kv_lens[b]. */
int oracle_decode_mla_ragged(const double *q, const double *ckv, int B, int Hq,
                             const int *kv_lens, int kv_cap, int Dqk, int Dv,
                             double scale, double *o, double *lse, int threads)
{
    if (B < 1 || Hq < 1 || Dqk < 1 || Dv < 1 || Dv > Dqk || kv_cap < 1)
        return -1;
    for (int b = 0; b < B; ++b)
        if (kv_lens[b] < 0 || kv_lens[b] > kv_cap)
            return -1;
    mla_ctx c = {q, ckv, B, Hq, 0, kv_cap, Dqk, Dv, kv_lens, scale, o, lse};
    return run_units(mla_unit, &c, (long)B * Hq, kv_cap, threads);
}

/* ------------------------- causal prefill backward, selected rows / keys --- */
/* The same gradients as oracle_prefill_causal_backward, evaluated for chosen
 * query rows (dQ) and chosen keys (dK, dV) with the work spread over rows,
 * so one (b, K/V head) group of a long sequence takes seconds, not minutes.
 * It follows the definition in three passes:
 *   1. every row i: the forward weights P_i (the same attend_row as the
 *      prefill, with the causal mask row), its LSE_i, and
 *      Dsum_i = Σ_j P_ij · dP_ij with dP_ij = dO_i · V_j;
 *   2. each chosen row: dS_ij = P_ij (dP_ij − Dsum_i), dQ_i = scale Σ_j dS_ij K_j;
 *   3. each chosen key j, for every row i the mask leaves it visible to
 *      (i >= j), in every query head of its group: P_ij = exp(s_ij − LSE_i)
 *      (the softmax written through the log-sum-exp, [p1] §3), dS_ij as above,
 *      dV_j = Σ P_ij dO_i, dK_j = scale Σ dS_ij Q_i.
 * Per-row quantities are fixed before pass 2 and 3 read them, and every sum
 * runs in ascending index order inside one unit, so the thread count does not
 * change the result. */
typedef struct {
    const double *q, *k, *v, *dout;
    int B, Hq, Hkv, N, D;
    double scale;
    const int *rows, *keys;
    int n_rows, n_keys;
    double *lse, *dsum; /* [B][Hq][N] */
    double *dq;         /* [B][Hq][n_rows][D] */
    double *dk, *dv;    /* [B][Hkv][n_keys][D] */
} bwd_rows_ctx;

static double dot_d(const double *a, const double *b, int D)
{
    double acc = 0.0;
    for (int t = 0; t < D; ++t)
        acc += a[t] * b[t];
    return acc;
}

/* scratch: s[N], p[N], o[D], mask[N] bytes */
static void bwd_rows_stats(bwd_rows_ctx *c, int b, int hq, int i, double *scratch, double *lse_out,
                           double *dsum_out, double *p)
{
    const int N = c->N, D = c->D, hkv = hq / (c->Hq / c->Hkv);
    double *s = scratch, *o = scratch + 2L * N;
    unsigned char *mask = (unsigned char *)(o + D);
    const double *Q = c->q + ((long)b * c->Hq + hq) * (long)N * D;
    const double *dO = c->dout + ((long)b * c->Hq + hq) * (long)N * D;
    const double *K = c->k + ((long)b * c->Hkv + hkv) * (long)N * D;
    const double *V = c->v + ((long)b * c->Hkv + hkv) * (long)N * D;
    for (int j = 0; j < N; ++j)
        mask[j] = (unsigned char)(j > i);
    attend_row(Q + (long)i * D, K, D, D, V, D, D, N, mask, c->scale, s, o, lse_out, p);
    double acc = 0.0;
    for (int j = 0; j < N; ++j)
        if (!mask[j])
            acc += p[j] * dot_d(dO + (long)i * D, V + (long)j * D, D);
    *dsum_out = acc;
}

static void bwd_rows_pass1(void *vctx, long unit, double *scratch)
{
    bwd_rows_ctx *c = (bwd_rows_ctx *)vctx;
    const int i = (int)(unit % c->N), bh = (int)(unit / c->N);
    bwd_rows_stats(c, bh / c->Hq, bh % c->Hq, i, scratch, c->lse + unit, c->dsum + unit,
                   scratch + c->N);
}

static void bwd_rows_pass2(void *vctx, long unit, double *scratch)
{
    bwd_rows_ctx *c = (bwd_rows_ctx *)vctx;
    const int N = c->N, D = c->D;
    const int r = (int)(unit % c->n_rows), bh = (int)(unit / c->n_rows);
    const int b = bh / c->Hq, hq = bh % c->Hq, hkv = hq / (c->Hq / c->Hkv), i = c->rows[r];
    double *p = scratch + N, lse_i, dsum_i;
    bwd_rows_stats(c, b, hq, i, scratch, &lse_i, &dsum_i, p);
    const double *dO = c->dout + ((long)b * c->Hq + hq) * (long)N * D;
    const double *K = c->k + ((long)b * c->Hkv + hkv) * (long)N * D;
    const double *V = c->v + ((long)b * c->Hkv + hkv) * (long)N * D;
    const double Di = c->dsum[(long)bh * N + i];
    double *dq = c->dq + ((long)bh * c->n_rows + r) * D;
    for (int t = 0; t < D; ++t)
        dq[t] = 0.0;
    for (int j = 0; j <= i; ++j) {
        const double ds = p[j] * (dot_d(dO + (long)i * D, V + (long)j * D, D) - Di);
        for (int t = 0; t < D; ++t)
            dq[t] += ds * K[(long)j * D + t];
    }
    for (int t = 0; t < D; ++t)
        dq[t] *= c->scale;
}

static void bwd_rows_pass3(void *vctx, long unit, double *scratch)
{
    (void)scratch;
    bwd_rows_ctx *c = (bwd_rows_ctx *)vctx;
    const int N = c->N, D = c->D, G = c->Hq / c->Hkv;
    const int u = (int)(unit % c->n_keys), bk = (int)(unit / c->n_keys);
    const int b = bk / c->Hkv, hkv = bk % c->Hkv, j = c->keys[u];
    const double *K = c->k + ((long)b * c->Hkv + hkv) * (long)N * D + (long)j * D;
    const double *V = c->v + ((long)b * c->Hkv + hkv) * (long)N * D + (long)j * D;
    double *dk = c->dk + ((long)bk * c->n_keys + u) * D;
    double *dv = c->dv + ((long)bk * c->n_keys + u) * D;
    for (int t = 0; t < D; ++t)
        dk[t] = dv[t] = 0.0;
    for (int g = 0; g < G; ++g) {
        const long bh = (long)b * c->Hq + hkv * G + g;
        const double *Q = c->q + bh * N * D, *dO = c->dout + bh * N * D;
        for (int i = 0; i < N; ++i) {
            if (j > i) /* the causal mask: key j is in row i's future */
                continue;
            const double s = c->scale * dot_d(Q + (long)i * D, K, D);
            const double p = exp(s - c->lse[bh * N + i]);
            const double ds = p * (dot_d(dO + (long)i * D, V, D) - c->dsum[bh * N + i]);
            for (int t = 0; t < D; ++t) {
                dv[t] += p * dO[(long)i * D + t];
                dk[t] += c->scale * ds * Q[(long)i * D + t];
            }
        }
    }
}

/* q, dout: [B][Hq][N][D]; k, v: [B][Hkv][N][D]; rows: n_rows query indices,
 * keys: n_keys key indices, each in [0, N).
 * dq: [B][Hq][n_rows][D]; dk, dv: [B][Hkv][n_keys][D]. */
int oracle_prefill_causal_backward_rows(const double *q, const double *k, const double *v,
                                        const double *dout, int B, int Hq, int Hkv, int N, int D,
                                        double scale, const int *rows, int n_rows, const int *keys,
                                        int n_keys, double *dq, double *dk, double *dv,
                                        int threads)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1 || Hq % Hkv || n_rows < 0 || n_keys < 0)
        return -1;
    for (int r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= N)
            return -1;
    for (int u = 0; u < n_keys; ++u)
        if (keys[u] < 0 || keys[u] >= N)
            return -1;
    double *stats = (double *)malloc(sizeof(double) * 2 * (size_t)B * Hq * N);
    if (!stats)
        return -1;
    bwd_rows_ctx c = {q, k, v, dout, B, Hq, Hkv, N, D, scale, rows, keys, n_rows, n_keys,
                      stats, stats + (size_t)B * Hq * N, dq, dk, dv};
    /* scratch: s[N], p[N], o[D], and N mask bytes */
    const int scratch = 2 * N + D + (N + 7) / 8 + 1;
    int rc = run_units(bwd_rows_pass1, &c, (long)B * Hq * N, scratch, threads);
    if (rc == 0 && n_rows > 0)
        rc = run_units(bwd_rows_pass2, &c, (long)B * Hq * n_rows, scratch, threads);
    if (rc == 0 && n_keys > 0)
        rc = run_units(bwd_rows_pass3, &c, (long)B * Hkv * n_keys, 1, threads);
    free(stats);
    return rc;
}
