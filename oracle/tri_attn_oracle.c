/*
 * FP64 CPU oracle for triangle attention (starting node), forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the HIP
 * path is checked against.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product path never calls it and
 * shares no code, header or constant with it.
 *
 * What it computes (TurboPairFormer pages: the Lambda post "Как работает
 * TurboPairFormer", and the biocloudservice page "它优化了什么"):
 *   For every batch b, row i and head h, queries q[b,i,j,h,:] attend over keys
 *   k[b,i,k,h,:] of the same row.  With alpha the softmax scale (1/sqrt(D) unless
 *   given), mu[b,i,k] = 0 for an attended key and -inf for a masked one:
 *     s[j,k]  = alpha * <q[b,i,j,h,:], k[b,i,k,h,:]> + bias[b,h,j,k] + mu[b,i,k]
 *     P[j,k]  = exp(s[j,k] - m_j) / sum_k' exp(s[j,k'] - m_j),  m_j = max_k s[j,k]
 *     o[b,i,j,h,:] = sum_k P[j,k] v[b,i,k,h,:]
 *     lse[b,i,h,j] = m_j + log sum_k exp(s[j,k] - m_j)
 *   The pair bias is shared by every row i, so its gradient is a reduction over
 *   all rows: dbias[b,h,j,k] = sum_i dS_i[j,k].
 *   Backward with g = dO:
 *     dP[j,k] = <g[b,i,j,h,:], v[b,i,k,h,:]>,  Dj = sum_k P[j,k] dP[j,k]
 *     dS[j,k] = P[j,k] (dP[j,k] - Dj)
 *     dq[j] = alpha sum_k dS[j,k] k[k],  dk[k] = alpha sum_j dS[j,k] q[j],
 *     dv[k] = sum_j P[j,k] g[j]
 *   These are the plain definitions written out in double precision.
 *
 * Readings where the pages are silent:
 *   - a row whose keys are all masked gets o = 0, lse = +inf and zero gradients;
 *   - the mask is [B,N,N] (row i, key k), broadcast over heads and queries, and
 *     gets no gradient; masked keys get exactly zero weight.
 *
 * Layouts (all row-major, last index fastest):
 *   q, k, v, dO : [B, N, N, H, D]   bias : [B, H, N, N]   mask : [B, N, N] u8 or NULL
 * Outputs are written compactly per selected row: for the r-th selected (b, i),
 *   o[r, j, h, c], lse[r, h, j], dq/dk/dv[r, j, h, c].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, N, H, D;
    double alpha;
    const double *q, *k, *v, *bias, *dout;
    const uint8_t *mask;
} problem_t;

static inline int64_t at5(const problem_t *p, int64_t b, int64_t i, int64_t j, int64_t h) {
    return (((b * p->N + i) * p->N + j) * p->H + h) * p->D;
}

static inline int attends(const problem_t *p, int64_t b, int64_t i, int64_t k) {
    return p->mask == NULL || p->mask[(b * p->N + i) * p->N + k] != 0;
}

static double dot(const double *x, const double *y, int64_t n) {
    double acc = 0.0;
    for (int64_t c = 0; c < n; ++c) acc += x[c] * y[c];
    return acc;
}

/*
 * Softmax row of query j in row (b, i), head h.  Fills prob[k] (0 for masked
 * keys) and returns the log-sum-exp; returns +inf (and prob = 0) when no key is
 * attended.
 */
static double softmax_row(const problem_t *p, int64_t b, int64_t i, int64_t h, int64_t j,
                          double *logit, double *prob) {
    const int64_t N = p->N;
    const double *qj = p->q + at5(p, b, i, j, h);
    const double *bias_row = p->bias + ((b * p->H + h) * N + j) * N;
    double m = -INFINITY;
    for (int64_t k = 0; k < N; ++k) {
        if (!attends(p, b, i, k)) { logit[k] = -INFINITY; continue; }
        logit[k] = p->alpha * dot(qj, p->k + at5(p, b, i, k, h), p->D) + bias_row[k];
        if (logit[k] > m) m = logit[k];
    }
    if (m == -INFINITY) {
        for (int64_t k = 0; k < N; ++k) prob[k] = 0.0;
        return INFINITY;
    }
    double l = 0.0;
    for (int64_t k = 0; k < N; ++k) {
        prob[k] = (logit[k] == -INFINITY) ? 0.0 : exp(logit[k] - m);
        l += prob[k];
    }
    for (int64_t k = 0; k < N; ++k) prob[k] /= l;
    return m + log(l);
}

/* dP[k] = <dO[j], v[k]> for attended keys; returns Dj = sum_k P dP. */
static double dprob_row(const problem_t *p, int64_t b, int64_t i, int64_t h, int64_t j,
                        const double *prob, double *dprob) {
    const double *gj = p->dout + at5(p, b, i, j, h);
    double Dj = 0.0;
    for (int64_t k = 0; k < p->N; ++k) {
        dprob[k] = attends(p, b, i, k) ? dot(gj, p->v + at5(p, b, i, k, h), p->D) : 0.0;
        Dj += prob[k] * dprob[k];
    }
    return Dj;
}

/*
 * Forward (and, when dout != NULL, backward for q, k and v) of the selected rows.
 * rows_b[r], rows_i[r] name the r-th selected row.  Any output pointer may be NULL.
 */
void oracle_rows(int64_t B, int64_t N, int64_t H, int64_t D, double alpha,
                 const double *q, const double *k, const double *v, const double *bias,
                 const uint8_t *mask, const double *dout,
                 int64_t nrows, const int64_t *rows_b, const int64_t *rows_i,
                 double *o, double *lse, double *dq, double *dk, double *dv, double *delta) {
    problem_t p = {B, N, H, D, alpha, q, k, v, bias, dout, mask};
    const int64_t row_elems = N * H * D;
#pragma omp parallel
    {
        double *logit = malloc(sizeof(double) * N);
        double *prob = malloc(sizeof(double) * N);
        double *dprob = malloc(sizeof(double) * N);
#pragma omp for schedule(dynamic)
        for (int64_t rh = 0; rh < nrows * H; ++rh) {
            const int64_t r = rh / H, h = rh % H;
            const int64_t b = rows_b[r], i = rows_i[r];
            for (int64_t j = 0; j < N; ++j) {
                const double L = softmax_row(&p, b, i, h, j, logit, prob);
                if (lse) lse[(r * H + h) * N + j] = L;
                if (o) {
                    double *oj = o + r * row_elems + (j * H + h) * D;
                    for (int64_t c = 0; c < D; ++c) oj[c] = 0.0;
                    for (int64_t kk = 0; kk < N; ++kk) {
                        if (prob[kk] == 0.0) continue;
                        const double *vk = v + at5(&p, b, i, kk, h);
                        for (int64_t c = 0; c < D; ++c) oj[c] += prob[kk] * vk[c];
                    }
                }
                if (dout == NULL) continue;
                const double Dj = dprob_row(&p, b, i, h, j, prob, dprob);
                if (delta) delta[(r * H + h) * N + j] = Dj;
                const double *qj = q + at5(&p, b, i, j, h);
                const double *gj = dout + at5(&p, b, i, j, h);
                double *dqj = dq ? dq + r * row_elems + (j * H + h) * D : NULL;
                if (dqj) for (int64_t c = 0; c < D; ++c) dqj[c] = 0.0;
                for (int64_t kk = 0; kk < N; ++kk) {
                    const double ds = prob[kk] * (dprob[kk] - Dj);
                    const double *kv = k + at5(&p, b, i, kk, h);
                    if (dqj) for (int64_t c = 0; c < D; ++c) dqj[c] += alpha * ds * kv[c];
                    if (dk) {
                        double *dkk = dk + r * row_elems + (kk * H + h) * D;
                        if (j == 0) for (int64_t c = 0; c < D; ++c) dkk[c] = 0.0;
                        for (int64_t c = 0; c < D; ++c) dkk[c] += alpha * ds * qj[c];
                    }
                    if (dv) {
                        double *dvk = dv + r * row_elems + (kk * H + h) * D;
                        if (j == 0) for (int64_t c = 0; c < D; ++c) dvk[c] = 0.0;
                        for (int64_t c = 0; c < D; ++c) dvk[c] += prob[kk] * gj[c];
                    }
                }
            }
        }
        free(logit);
        free(prob);
        free(dprob);
    }
}

/*
 * Pair-bias gradient of the selected (b, h, j): dbias[s, k] = sum over rows i in
 * ascending order of dS_i[j, k].  P_i and dP_i are recomputed for every row.
 */
void oracle_dbias(int64_t B, int64_t N, int64_t H, int64_t D, double alpha,
                  const double *q, const double *k, const double *v, const double *bias,
                  const uint8_t *mask, const double *dout,
                  int64_t nsel, const int64_t *sel_b, const int64_t *sel_h,
                  const int64_t *sel_j, double *dbias) {
    problem_t p = {B, N, H, D, alpha, q, k, v, bias, dout, mask};
#pragma omp parallel
    {
        double *logit = malloc(sizeof(double) * N);
        double *prob = malloc(sizeof(double) * N);
        double *dprob = malloc(sizeof(double) * N);
#pragma omp for schedule(dynamic)
        for (int64_t s = 0; s < nsel; ++s) {
            const int64_t b = sel_b[s], h = sel_h[s], j = sel_j[s];
            double *out = dbias + s * N;
            for (int64_t kk = 0; kk < N; ++kk) out[kk] = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                softmax_row(&p, b, i, h, j, logit, prob);
                const double Dj = dprob_row(&p, b, i, h, j, prob, dprob);
                for (int64_t kk = 0; kk < N; ++kk) out[kk] += prob[kk] * (dprob[kk] - Dj);
            }
        }
        free(logit);
        free(prob);
        free(dprob);
    }
}
