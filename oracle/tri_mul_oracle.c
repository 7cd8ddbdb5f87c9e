/*
 * FP64 CPU oracle for the triangle multiplicative update's contraction, forward and
 * backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, plain reference the HIP path is checked
 * against.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the product path never calls it and shares no code with it.
 *
 * What it computes.  The TurboPairFormer pages name the triangle multiplicative update
 * as the method's second kernel family next to triangle attention (biocloudservice
 * page, opening paragraph; Lambda post, opening section) without writing it out.  The
 * plainest reading of an AlphaFold3-style triangle multiplicative update is the
 * Pairformer block whose cubic-cost core contracts two projected pair tensors a and b
 * (channels c, pair positions (x, y)) over the third node k of every triangle, one
 * channel at a time:
 *   outgoing edges: z[b, i, j, c] = sum_k a[b, i, k, c] * bb[b, j, k, c]
 *   incoming edges: z[b, i, j, c] = sum_k a[b, k, i, c] * bb[b, k, j, c]
 * With g = dL/dz the gradients are the two other contractions of the same triangle:
 *   outgoing: da[b, i, k, c] = sum_j g[b, i, j, c] * bb[b, j, k, c]
 *             dbb[b, j, k, c] = sum_i g[b, i, j, c] * a[b, i, k, c]
 *   incoming: da[b, k, i, c] = sum_j g[b, i, j, c] * bb[b, k, j, c]
 *             dbb[b, k, j, c] = sum_i g[b, i, j, c] * a[b, k, i, c]
 * These are the plain definitions written out in double precision, one output value
 * at a time.  (The projections, gates, masks and layer norms of the whole block act
 * elementwise or per position before and after this contraction.)
 *
 * Layout (row-major, last index fastest): a, bb, g, z, da, dbb : [B, N, N, C].
 * Outputs are written compactly per selected row: for the r-th selected (b, x), the
 * values [r, y, c] of the output tensor's row x (its first pair index).
 */
#include <stdint.h>

static inline int64_t at4(int64_t N, int64_t C, int64_t b, int64_t x, int64_t y) {
    return ((b * N + x) * N + y) * C;
}

/* Rows x of z: z[b, x, y, c] for every y, c. */
void oracle_trimul_rows(int64_t B, int64_t N, int64_t C, int incoming, const double *a, const double *bb,
                        int64_t nrows, const int64_t *rows_b, const int64_t *rows_x, double *z) {
    (void)B;
#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows_b[r], i = rows_x[r];
        double *zr = z + r * N * C;
        for (int64_t j = 0; j < N; ++j)
            for (int64_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int64_t k = 0; k < N; ++k) {
                    if (incoming)
                        acc += a[at4(N, C, b, k, i) + c] * bb[at4(N, C, b, k, j) + c];
                    else
                        acc += a[at4(N, C, b, i, k) + c] * bb[at4(N, C, b, j, k) + c];
                }
                zr[j * C + c] = acc;
            }
    }
}

/* Rows x of da (which = 0) or dbb (which = 1): out[r, y, c] = grad[b, x, y, c]. */
void oracle_trimul_grad_rows(int64_t B, int64_t N, int64_t C, int incoming, int which, const double *a,
                             const double *bb, const double *g, int64_t nrows, const int64_t *rows_b,
                             const int64_t *rows_x, double *out) {
    (void)B;
#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows_b[r], x = rows_x[r];
        double *o = out + r * N * C;
        for (int64_t y = 0; y < N; ++y)
            for (int64_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int64_t t = 0; t < N; ++t) {
                    if (!incoming && which == 0)       /* da[i=x, k=y] = sum_j g[i, j] bb[j, k] */
                        acc += g[at4(N, C, b, x, t) + c] * bb[at4(N, C, b, t, y) + c];
                    else if (!incoming && which == 1)  /* dbb[j=x, k=y] = sum_i g[i, j] a[i, k] */
                        acc += g[at4(N, C, b, t, x) + c] * a[at4(N, C, b, t, y) + c];
                    else if (incoming && which == 0)   /* da[k=x, i=y] = sum_j g[i, j] bb[k, j] */
                        acc += g[at4(N, C, b, y, t) + c] * bb[at4(N, C, b, x, t) + c];
                    else                               /* dbb[k=x, j=y] = sum_i g[i, j] a[k, i] */
                        acc += g[at4(N, C, b, t, y) + c] * a[at4(N, C, b, x, t) + c];
                }
                o[y * C + c] = acc;
            }
    }
}
