/*
 * Plain fp64 CPU oracle for the Differential Attention forward operator.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the GPU path is
 * checked against.  It shares no code, header or constant with the GPU library,
 * and nothing on the product path may call it.
 *
 * What it computes, for one head and one query row i (all in double):
 *
 *   visible keys      j = 0 .. n_vis-1, where n_vis = i+1 under a causal mask
 *                     (a query sees itself and earlier keys) and n_vis = n_k
 *                     otherwise;
 *   scores            s1_j = <q1_i, k1_j> / sqrt(d),  s2_j = <q2_i, k2_j> / sqrt(d)
 *                     -- the two scaled dot products of the DiffAttn formula
 *                     (iloveeagents.com, "Mathematical Formula"; llmbytes.dev,
 *                     "How Differential Attention Cancels Common-Mode Noise",
 *                     step 2), with d the query/key head dimension;
 *   softmax maps      a1_j = exp(s1_j - max s1) / sum_j exp(s1_j - max s1), and
 *                     a2 likewise (same sources, step 2; subtracting the max does
 *                     not change the exact value);
 *   differential row  w_j = a1_j - lambda * a2_j  (step 3 of the llmbytes.dev list);
 *   pre-norm output   D_c = sum_j w_j * v_jc,  c = 0 .. dv-1  (step 3);
 *   per-head norm     mu = mean_c D_c, var = mean_c (D_c - mu)^2 (population
 *                     variance), out_c = (1 - lambda_init) * (D_c - mu) /
 *                     sqrt(var + eps)  (step 4: GroupNorm over the head's
 *                     channels, then the (1 - lambda_init) scale; no affine
 *                     parameters).
 *
 * The row of w is materialised once per query; there is no tiling, fusion or
 * reordering beyond that definition.  Rows are independent and are spread over
 * OpenMP threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Softmax of x[0..n-1] in place (n >= 1). */
static void softmax_inplace(double* x, int64_t n) {
    double m = x[0];
    for (int64_t j = 1; j < n; ++j)
        if (x[j] > m) m = x[j];
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        x[j] = exp(x[j] - m);
        z += x[j];
    }
    for (int64_t j = 0; j < n; ++j) x[j] /= z;
}

static double dot(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += a[t] * b[t];
    return s;
}

/*
 * One head.  Row-major arrays:
 *   q1, q2 [n_q][d]   k1, k2 [n_k][d]   v [n_k][dv]
 * rows[r] (0 <= rows[r] < n_q) names the query rows to compute; out is
 * [n_rows][dv].  For a causal mask, query row i is at sequence position
 * i (queries and keys share positions; n_q must equal n_k).
 * pre_norm != 0 writes D instead of the normalised output.
 * rowsum, if not NULL, receives sum_j w_j for each computed row.
 * Returns 0, or -1 on a bad argument or an allocation failure.
 */
int oracle_diffattn_rows(const double* q1, const double* q2,
                         const double* k1, const double* k2, const double* v,
                         int64_t n_q, int64_t n_k, int d, int dv,
                         const int64_t* rows, int64_t n_rows,
                         int causal, double lam, double lambda_init, double eps,
                         int pre_norm, double* out, double* rowsum) {
    if (!q1 || !q2 || !k1 || !k2 || !v || !rows || !out) return -1;
    if (n_q < 1 || n_k < 1 || d < 1 || dv < 1 || n_rows < 0) return -1;
    if (causal && n_q != n_k) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= n_q) return -1;

    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int failed = 0;

#pragma omp parallel
    {
        double* a1 = (double*)malloc(sizeof(double) * (size_t)n_k);
        double* a2 = (double*)malloc(sizeof(double) * (size_t)n_k);
        double* D = (double*)malloc(sizeof(double) * (size_t)dv);
        const int have_buffers = a1 && a2 && D;
        /* every thread reaches the work-sharing loop, buffers or not */
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!have_buffers) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            {
                const int64_t i = rows[r];
                const int64_t n_vis = causal ? i + 1 : n_k;
                const double* q1i = q1 + i * d;
                const double* q2i = q2 + i * d;

                for (int64_t j = 0; j < n_vis; ++j) {
                    a1[j] = dot(q1i, k1 + j * d, d) * inv_sqrt_d;
                    a2[j] = dot(q2i, k2 + j * d, d) * inv_sqrt_d;
                }
                softmax_inplace(a1, n_vis);
                softmax_inplace(a2, n_vis);

                /* w_j = a1_j - lambda a2_j, kept in a1 */
                double wsum = 0.0;
                for (int64_t j = 0; j < n_vis; ++j) {
                    a1[j] = a1[j] - lam * a2[j];
                    wsum += a1[j];
                }
                if (rowsum) rowsum[r] = wsum;

                for (int c = 0; c < dv; ++c) D[c] = 0.0;
                for (int64_t j = 0; j < n_vis; ++j) {
                    const double wj = a1[j];
                    const double* vj = v + j * dv;
                    for (int c = 0; c < dv; ++c) D[c] += wj * vj[c];
                }

                double* o = out + r * dv;
                if (pre_norm) {
                    memcpy(o, D, sizeof(double) * (size_t)dv);
                } else {
                    double mu = 0.0;
                    for (int c = 0; c < dv; ++c) mu += D[c];
                    mu /= dv;
                    double var = 0.0;
                    for (int c = 0; c < dv; ++c) var += (D[c] - mu) * (D[c] - mu);
                    var /= dv;
                    const double inv_std = 1.0 / sqrt(var + eps);
                    for (int c = 0; c < dv; ++c)
                        o[c] = (1.0 - lambda_init) * (D[c] - mu) * inv_std;
                }
            }
        }
        free(a1);
        free(a2);
        free(D);
    }
    return failed ? -1 : 0;
}

/* Number of threads an OpenMP parallel region uses here (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
