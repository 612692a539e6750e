/*
 * attn_oracle.c -- fp64 CPU oracle for exact softmax attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product:
 * only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
 * may load or call it.  It shares no code, header, table or constant with
 * the HIP library under exact_io_aware_27_amd/csrc, and it never touches a GPU.
 *
 * What it computes is the plain definition of attention, written out with
 * no tiling, no online softmax, no fusion and no reordering:
 *
 *   O = softmax(scale * Q K^T) V          per (batch, head)
 *
 *   - "FlashAttention evolution" (letsgetai.github.io), section on why
 *     attention is slow: the attention equation, S = Q K^T in R^{N x N},
 *     softmax over each row, then the product with V.
 *   - "FlashAttention" concept page (compassingai.com), section 3, the
 *     memory-wall listing: S is formed in full, P = softmax(S) is formed in
 *     full, then O = P V.  This oracle does exactly that, one query row at
 *     a time: it materialises the row of S and the row of P in host memory.
 *
 * Readings where the pages are silent (each is also listed in the design doc):
 *   - the scale is an explicit argument; every workload passes 1/sqrt(d),
 *     the value in the attention equation;
 *   - causal: key j is visible to query i iff j <= i + (Nk - Nq).  With
 *     Nq == Nk that is j <= i; with fewer queries than keys the queries are
 *     the LAST Nq positions of the sequence (each new token sees every key
 *     before it, as in decoding with the keys and values of earlier tokens
 *     kept); masked keys take no part in max, sum or output;
 *   - LSE (the saved softmax statistics, m and l, folded into one number) is
 *     the natural-log logsumexp of the scaled, masked logits: m + ln(l);
 *   - inputs are bfloat16 bit patterns; each is widened exactly to fp64.
 *
 * Every floating-point step runs in fp64 in ascending index order.
 * Parity: pinned by tests/test_oracle.py against closed forms (equal keys,
 * causal row 0, N = 1, two-key logistic weights with huge logits), against an
 * independent library routine (PyTorch's CPU scaled_dot_product_attention in
 * float64) and against the pages' two-block merge identity.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status codes of oracle_attn(). */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2
#define ORACLE_PSUM 3 /* a row of P failed to sum to 1 within 1e-12 */

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q;         /* [BH][Nq][d] bf16 bits */
    const uint16_t *k, *v;     /* [BH][Nk][d] bf16 bits */
    int64_t BH, Nq, Nk, d;
    int causal;
    double scale;
    const int64_t *rows; /* [BH][R] query-row indices, or NULL = all rows */
    int64_t R;           /* rows per (batch, head) */
    double *o;           /* [BH][R][d] */
    double *lse;         /* [BH][R] */
    double *psum_dev;    /* [BH][R] |sum_j P_ij - 1|, may be NULL */
    int64_t next_job;    /* shared job counter, taken under the lock */
    int64_t n_jobs;
    int status;
    pthread_mutex_t lock;
} oracle_ctx;

enum { ROWS_PER_JOB = 64 };

/*
 * One query row i of one (batch, head):
 *   J    = {0..Nk-1}, or {0..i+Nk-Nq} when causal
 *   S_j  = scale * sum_t q_it k_jt            (the S row, materialised)
 *   m    = max_j S_j
 *   e_j  = exp(S_j - m),  l = sum_j e_j,  P_j = e_j / l   (the P row)
 *   O_t  = sum_j P_j v_jt
 *   LSE  = m + ln(l)
 */
static int one_row(const oracle_ctx *c, int64_t bh, int64_t i, double *qrow,
                   double *S, double *P, double *o_out, double *lse_out,
                   double *dev_out)
{
    const int64_t Nq = c->Nq, Nk = c->Nk, d = c->d;
    const uint16_t *q = c->q + bh * Nq * d;
    const uint16_t *k = c->k + bh * Nk * d;
    const uint16_t *v = c->v + bh * Nk * d;
    const int64_t nkeys = c->causal ? i + (Nk - Nq) + 1 : Nk;

    for (int64_t t = 0; t < d; ++t)
        qrow[t] = widen_bf16(q[i * d + t]);

    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int64_t t = 0; t < d; ++t)
            dot += qrow[t] * widen_bf16(k[j * d + t]);
        S[j] = c->scale * dot;
    }

    double m = S[0];
    for (int64_t j = 1; j < nkeys; ++j)
        if (S[j] > m)
            m = S[j];

    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        P[j] = exp(S[j] - m);
        l += P[j];
    }
    double psum = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        P[j] = P[j] / l;
        psum += P[j];
    }
    const double dev = fabs(psum - 1.0);

    for (int64_t t = 0; t < d; ++t)
        o_out[t] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        const double p = P[j];
        for (int64_t t = 0; t < d; ++t)
            o_out[t] += p * widen_bf16(v[j * d + t]);
    }
    *lse_out = m + log(l);
    if (dev_out)
        *dev_out = dev;
    return dev <= 1e-12 ? ORACLE_OK : ORACLE_PSUM;
}

static void *worker(void *arg)
{
    oracle_ctx *c = (oracle_ctx *)arg;
    const int64_t jobs_per_bh = (c->R + ROWS_PER_JOB - 1) / ROWS_PER_JOB;
    double *qrow = malloc((size_t)c->d * sizeof(double));
    double *S = malloc((size_t)c->Nk * sizeof(double));
    double *P = malloc((size_t)c->Nk * sizeof(double));
    int status = ORACLE_OK;
    if (!qrow || !S || !P)
        status = ORACLE_NO_MEMORY;

    while (status == ORACLE_OK) {
        pthread_mutex_lock(&c->lock);
        const int64_t job = c->next_job++;
        pthread_mutex_unlock(&c->lock);
        if (job >= c->n_jobs)
            break;
        const int64_t bh = job / jobs_per_bh;
        const int64_t r0 = (job % jobs_per_bh) * ROWS_PER_JOB;
        const int64_t r1 = r0 + ROWS_PER_JOB < c->R ? r0 + ROWS_PER_JOB : c->R;
        for (int64_t r = r0; r < r1 && status == ORACLE_OK; ++r) {
            const int64_t i = c->rows ? c->rows[bh * c->R + r] : r;
            const int64_t slot = bh * c->R + r;
            status = one_row(c, bh, i, qrow, S, P, c->o + slot * c->d,
                             c->lse + slot,
                             c->psum_dev ? c->psum_dev + slot : NULL);
        }
    }
    free(qrow);
    free(S);
    free(P);
    if (status != ORACLE_OK) {
        pthread_mutex_lock(&c->lock);
        if (c->status == ORACLE_OK)
            c->status = status;
        c->next_job = c->n_jobs; /* stop the other threads early */
        pthread_mutex_unlock(&c->lock);
    }
    return NULL;
}

/*
 * oracle_attn_qk: exact attention for the selected query rows of every
 * (batch, head), Nq queries against Nk keys.
 *   q         bf16 bit patterns, contiguous [BH][Nq][d]
 *   k, v      bf16 bit patterns, contiguous [BH][Nk][d]
 *   causal    requires Nq <= Nk (every query then sees at least key 0)
 *   rows      [BH][R] query indices in [0, Nq), or NULL for R == Nq, all rows
 *   o         out: fp64 [BH][R][d];  lse: out, fp64 [BH][R]
 *   psum_dev  out (optional): fp64 [BH][R], |sum_j P_ij - 1|
 *   nthreads  worker threads (>= 1)
 * Returns ORACLE_OK, or ORACLE_BAD_ARG / ORACLE_NO_MEMORY / ORACLE_PSUM.
 */
int oracle_attn_qk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   int64_t BH, int64_t Nq, int64_t Nk, int64_t d, int causal,
                   double scale, const int64_t *rows, int64_t R, double *o,
                   double *lse, double *psum_dev, int nthreads)
{
    if (!q || !k || !v || !o || !lse || BH < 0 || Nq < 1 || Nk < 1 || d < 1 ||
        R < 0 || nthreads < 1 || !isfinite(scale) || (causal && Nq > Nk))
        return ORACLE_BAD_ARG;
    if (!rows && R != Nq)
        return ORACLE_BAD_ARG;
    if (rows)
        for (int64_t x = 0; x < BH * R; ++x)
            if (rows[x] < 0 || rows[x] >= Nq)
                return ORACLE_BAD_ARG;
    if (BH == 0 || R == 0)
        return ORACLE_OK;

    oracle_ctx c;
    c.q = q;
    c.k = k;
    c.v = v;
    c.BH = BH;
    c.Nq = Nq;
    c.Nk = Nk;
    c.d = d;
    c.causal = causal ? 1 : 0;
    c.scale = scale;
    c.rows = rows;
    c.R = R;
    c.o = o;
    c.lse = lse;
    c.psum_dev = psum_dev;
    c.next_job = 0;
    c.n_jobs = BH * ((R + ROWS_PER_JOB - 1) / ROWS_PER_JOB);
    c.status = ORACLE_OK;
    pthread_mutex_init(&c.lock, NULL);

    if (nthreads > c.n_jobs)
        nthreads = (int)c.n_jobs;
    pthread_t *tid = malloc((size_t)nthreads * sizeof(pthread_t));
    if (!tid) {
        pthread_mutex_destroy(&c.lock);
        return ORACLE_NO_MEMORY;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, &c) != 0)
            break;
        ++started;
    }
    if (started == 0)
        worker(&c); /* no thread could be created: run on the caller */
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&c.lock);
    return c.status;
}

/* oracle_attn: the same with Nq == Nk == N (queries and keys of one sequence). */
int oracle_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                int64_t BH, int64_t N, int64_t d, int causal, double scale,
                const int64_t *rows, int64_t R, double *o, double *lse,
                double *psum_dev, int nthreads)
{
    return oracle_attn_qk(q, k, v, BH, N, N, d, causal, scale, rows, R, o, lse,
                          psum_dev, nthreads);
}
