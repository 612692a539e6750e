/*
 * attn_bwd_oracle.c -- fp64 CPU oracle for the gradients of exact softmax
 * attention (the backward pass).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product:
 * only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
 * may load or call it.  It shares no code, header, table or constant with
 * the HIP library under exact_io_aware_27_amd/csrc, and it never touches a GPU.
 *
 * The pages say that the backward pass recomputes S and P block by block
 * from the softmax statistics saved by the forward pass instead of storing
 * the N x N matrices ("FlashAttention evolution", letsgetai.github.io,
 * recomputation paragraph of the FlashAttention-1 results; "FlashAttention"
 * concept page, compassingai.com, section 3, mechanisms).  They do not write
 * the gradients out.  What the backward pass computes is the plain
 * derivative of the forward definition O = softmax(scale * Q K^T) V, which
 * this oracle writes out with no tiling and no recomputation, one query row
 * at a time, for an upstream gradient dO:
 *
 *   S_ij  = scale * q_i . k_j          (j visible to i; causal: j <= i + Nk - Nq)
 *   P_ij  = exp(S_ij - m_i) / l_i      (the softmax row, materialised)
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij           (= dO_i . O_i)
 *   dS_ij = P_ij (dP_ij - D_i)         (the softmax Jacobian applied to dP)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * Every floating-point step runs in fp64 in ascending index order; the
 * inputs are bf16 bit patterns widened exactly.  One thread per
 * (batch, head): dK and dV sum over the rows of their own head only.
 * Parity: pinned in tests/test_bwd_oracle.py against PyTorch autograd in
 * float64 on the CPU, against central finite differences of the forward
 * oracle's definition, and against closed forms.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BWD_OK 0
#define BWD_BAD_ARG 1
#define BWD_NO_MEMORY 2

static double widen(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v, *dout; /* q, dout: [BH][Nq][d]; k, v: [BH][Nk][d] */
    int64_t BH, Nq, Nk, d;
    int causal;
    double scale;
    double *dq, *dk, *dv; /* dq: [BH][Nq][d]; dk, dv: [BH][Nk][d] */
    double *dsum;         /* D: [BH][Nq] */
    int64_t next;
    int status;
    pthread_mutex_t lock;
} bwd_ctx;

static int one_head(bwd_ctx *c, int64_t bh)
{
    const int64_t Nq = c->Nq, Nk = c->Nk, d = c->d;
    const uint16_t *q = c->q + bh * Nq * d, *dout = c->dout + bh * Nq * d;
    const uint16_t *k = c->k + bh * Nk * d, *v = c->v + bh * Nk * d;
    double *dq = c->dq + bh * Nq * d, *dk = c->dk + bh * Nk * d, *dv = c->dv + bh * Nk * d;
    double *S = malloc((size_t)Nk * sizeof(double));
    double *P = malloc((size_t)Nk * sizeof(double));
    double *dP = malloc((size_t)Nk * sizeof(double));
    double *qi = malloc((size_t)d * sizeof(double));
    double *gi = malloc((size_t)d * sizeof(double));
    if (!S || !P || !dP || !qi || !gi) {
        free(S); free(P); free(dP); free(qi); free(gi);
        return BWD_NO_MEMORY;
    }
    for (int64_t x = 0; x < Nk * d; ++x)
        dk[x] = dv[x] = 0.0;
    for (int64_t i = 0; i < Nq; ++i) {
        const int64_t nkeys = c->causal ? i + (Nk - Nq) + 1 : Nk;
        for (int64_t t = 0; t < d; ++t) {
            qi[t] = widen(q[i * d + t]);
            gi[t] = widen(dout[i * d + t]);
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < nkeys; ++j) {
            double dot = 0.0;
            for (int64_t t = 0; t < d; ++t)
                dot += qi[t] * widen(k[j * d + t]);
            S[j] = c->scale * dot;
            if (S[j] > m)
                m = S[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            P[j] = exp(S[j] - m);
            l += P[j];
        }
        double Di = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            P[j] /= l;
            double dot = 0.0;
            for (int64_t t = 0; t < d; ++t)
                dot += gi[t] * widen(v[j * d + t]);
            dP[j] = dot;
            Di += P[j] * dP[j];
        }
        c->dsum[bh * Nq + i] = Di;
        for (int64_t t = 0; t < d; ++t)
            dq[i * d + t] = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            const double ds = P[j] * (dP[j] - Di);
            for (int64_t t = 0; t < d; ++t) {
                dv[j * d + t] += P[j] * gi[t];
                dq[i * d + t] += c->scale * ds * widen(k[j * d + t]);
                dk[j * d + t] += c->scale * ds * qi[t];
            }
        }
    }
    free(S); free(P); free(dP); free(qi); free(gi);
    return BWD_OK;
}

static void *worker(void *arg)
{
    bwd_ctx *c = (bwd_ctx *)arg;
    for (;;) {
        pthread_mutex_lock(&c->lock);
        const int64_t bh = c->status == BWD_OK ? c->next++ : c->BH;
        pthread_mutex_unlock(&c->lock);
        if (bh >= c->BH)
            break;
        const int st = one_head(c, bh);
        if (st != BWD_OK) {
            pthread_mutex_lock(&c->lock);
            c->status = st;
            pthread_mutex_unlock(&c->lock);
        }
    }
    return NULL;
}

/*
 * oracle_attn_bwd: gradients dQ, dK, dV (and D) of exact attention for an
 * upstream gradient dO, Nq queries against Nk keys (causal: Nq <= Nk, query
 * i sees key j iff j <= i + Nk - Nq).
 *   q, dout  bf16 bits [BH][Nq][d];  k, v: bf16 bits [BH][Nk][d]
 *   dq       out fp64 [BH][Nq][d];   dk, dv: out fp64 [BH][Nk][d]
 *   dsum     out fp64 [BH][Nq] (D_i = sum_j P_ij dP_ij)
 * Returns BWD_OK, BWD_BAD_ARG or BWD_NO_MEMORY.
 */
int oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                    int64_t BH, int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                    double *dq, double *dk, double *dv, double *dsum, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !dsum || BH < 0 || Nq < 1 || Nk < 1 ||
        d < 1 || nthreads < 1 || !isfinite(scale) || (causal && Nq > Nk))
        return BWD_BAD_ARG;
    if (BH == 0)
        return BWD_OK;
    bwd_ctx c;
    c.q = q; c.k = k; c.v = v; c.dout = dout;
    c.BH = BH; c.Nq = Nq; c.Nk = Nk; c.d = d;
    c.causal = causal ? 1 : 0;
    c.scale = scale;
    c.dq = dq; c.dk = dk; c.dv = dv; c.dsum = dsum;
    c.next = 0;
    c.status = BWD_OK;
    pthread_mutex_init(&c.lock, NULL);
    if (nthreads > BH)
        nthreads = (int)BH;
    pthread_t *tid = malloc((size_t)nthreads * sizeof(pthread_t));
    int started = 0;
    if (tid)
        for (int t = 0; t < nthreads; ++t) {
            if (pthread_create(&tid[t], NULL, worker, &c) != 0)
                break;
            ++started;
        }
    if (started == 0)
        worker(&c);
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&c.lock);
    return c.status;
}

/*
 * oracle_attn_bwd_dq_rows: dQ_i (and D_i) for R given query rows i of every
 * head, by the same per-row steps as oracle_attn_bwd: O(Nk d) per row, so
 * rows of long sequences can be checked one by one (dK and dV need every row).
 *   rows   int64 [BH][R] query indices;  dq: out fp64 [BH][R][d];  dsum: out [BH][R]
 *   term2  out fp64 [BH][R][d] or NULL: sum_j (scale dS_ij k_jt)^2, the sum of
 *          squared terms of each dQ element (the scale of its rounding error
 *          when every dS_ij is rounded before the product)
 *   pk, o  out fp64 [BH][R][d] or NULL: sum_j P_ij k_jt and the output row
 *          O_i = sum_j P_ij v_j (a change dD of D_i moves dQ_i by
 *          -scale dD (P K)_i, and D is formed from O)
 *   pv2    out fp64 [BH][R][d] or NULL: sum_j P_ij^2 (v_jt - O_it)^2, the
 *          scale of the error the forward pass's rounding of P puts into O
 */
int oracle_attn_bwd_dq_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                            int64_t BH, int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                            const int64_t *rows, int64_t R, double *dq, double *dsum, double *term2,
                            double *pk, double *o, double *pv2)
{
    if (!q || !k || !v || !dout || !rows || !dq || !dsum || BH < 0 || Nq < 1 || Nk < 1 || d < 1 || R < 0 ||
        !isfinite(scale) || (causal && Nq > Nk))
        return BWD_BAD_ARG;
    double *S = malloc((size_t)Nk * sizeof(double));
    double *P = malloc((size_t)Nk * sizeof(double));
    double *dP = malloc((size_t)Nk * sizeof(double));
    if (!S || !P || !dP) {
        free(S); free(P); free(dP);
        return BWD_NO_MEMORY;
    }
    int status = BWD_OK;
    for (int64_t bh = 0; bh < BH && status == BWD_OK; ++bh) {
        const uint16_t *qh = q + bh * Nq * d, *gh = dout + bh * Nq * d;
        const uint16_t *kh = k + bh * Nk * d, *vh = v + bh * Nk * d;
        for (int64_t x = 0; x < R; ++x) {
            const int64_t i = rows[bh * R + x];
            if (i < 0 || i >= Nq) {
                status = BWD_BAD_ARG;
                break;
            }
            const int64_t nkeys = causal ? i + (Nk - Nq) + 1 : Nk;
            double m = -INFINITY;
            for (int64_t j = 0; j < nkeys; ++j) {
                double dot = 0.0;
                for (int64_t t = 0; t < d; ++t)
                    dot += widen(qh[i * d + t]) * widen(kh[j * d + t]);
                S[j] = scale * dot;
                if (S[j] > m)
                    m = S[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                P[j] = exp(S[j] - m);
                l += P[j];
            }
            double Di = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                P[j] /= l;
                double dot = 0.0;
                for (int64_t t = 0; t < d; ++t)
                    dot += widen(gh[i * d + t]) * widen(vh[j * d + t]);
                dP[j] = dot;
                Di += P[j] * dP[j];
            }
            dsum[bh * R + x] = Di;
            double *out = dq + (bh * R + x) * d;
            double *t2 = term2 ? term2 + (bh * R + x) * d : NULL;
            double *pko = pk ? pk + (bh * R + x) * d : NULL;
            double *oo = o ? o + (bh * R + x) * d : NULL;
            double *p2 = pv2 ? pv2 + (bh * R + x) * d : NULL;
            for (int64_t t = 0; t < d; ++t) {
                out[t] = 0.0;
                if (t2)
                    t2[t] = 0.0;
                if (pko)
                    pko[t] = 0.0;
                if (oo)
                    oo[t] = 0.0;
            }
            for (int64_t j = 0; j < nkeys; ++j) {
                const double ds = P[j] * (dP[j] - Di);
                for (int64_t t = 0; t < d; ++t) {
                    const double kt = widen(kh[j * d + t]);
                    const double term = scale * ds * kt;
                    out[t] += term;
                    if (t2)
                        t2[t] += term * term;
                    if (pko)
                        pko[t] += P[j] * kt;
                    if (oo)
                        oo[t] += P[j] * widen(vh[j * d + t]);
                }
            }
            if (p2 && oo) {  /* second pass: O is known now */
                for (int64_t t = 0; t < d; ++t)
                    p2[t] = 0.0;
                for (int64_t j = 0; j < nkeys; ++j)
                    for (int64_t t = 0; t < d; ++t) {
                        const double dv = widen(vh[j * d + t]) - oo[t];
                        p2[t] += P[j] * P[j] * dv * dv;
                    }
            }
        }
    }
    free(S); free(P); free(dP);
    return status;
}
