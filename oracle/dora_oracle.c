/*
 * dora_oracle.c - plain, slow fp64 CPU reference for the DoRA module.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only code allowed to load this
 * library.  The HIP product library never calls it, and the two share no
 * source, header, table or helper.
 *
 * Sources (by page title and section):
 *   [SD]   "Scaling DoRA: High-Rank Adaptation via Factored Norms and Fused
 *          Kernels" (Zelenin, Zhuravlyova; arXiv 2603.22276), abstract.
 *   [DoRA] "DoRA: Weight-Decomposed Low-Rank Adaptation" (Liu et al. 2024),
 *          as summarised on its summary pages: "Method" and "Statistical
 *          analysis" sections, Key Point 3.
 *
 * What is computed, written out as plain definitions (no blocking, no
 * factoring, no reordering beyond the loops below):
 *   V   = W + s*B*A                dense [d_out, d_in]; this is exactly the
 *                                  materialised product that [SD] abstract
 *                                  says frameworks form and that the GPU
 *                                  path must avoid.
 *   n_i = ||V_i||_2                one norm per output row ([SD] abstract:
 *                                  "row-wise norm of W + sBA").
 *   y   = (m / n) (.) (x V^T)      magnitude times unit direction, the
 *                                  LoRA product supplying the direction
 *                                  ([DoRA] Method; Key Point 3).
 *   backward                       gradients of L = sum(dy (.) y) with the
 *                                  row norm n held constant (the reading
 *                                  of the training-memory modification in
 *                                  [DoRA] "Statistical analysis").
 *
 * Precision: every input element (fp32, or bf16 given as raw 16-bit
 * patterns) is promoted exactly to double; all arithmetic is double.
 * m, n and s are passed as doubles by the caller (promoted exactly from
 * the fp32 values the GPU receives).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Exact promotion of element idx of an fp32 or bf16 array to double. */
static double elem(const void *p, int dtype, int64_t idx)
{
    if (dtype == ORACLE_BF16) {
        uint32_t bits = ((const uint16_t *)p)[idx];
        bits <<= 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[idx];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Row i of the LoRA product, ba[j] = sum_k B[i,k] * A[k,j], and the dense
 * row v[j] = W[i,j] + s * ba[j]. */
static void dense_row(const void *W, const void *A, const void *B, int dt,
                      double s, int64_t d_in, int64_t r, int64_t i,
                      double *ba, double *v)
{
    for (int64_t j = 0; j < d_in; ++j)
        ba[j] = 0.0;
    for (int64_t k = 0; k < r; ++k) {
        double b = elem(B, dt, i * r + k);
        for (int64_t j = 0; j < d_in; ++j)
            ba[j] += b * elem(A, dt, k * d_in + j);
    }
    for (int64_t j = 0; j < d_in; ++j)
        v[j] = elem(W, dt, i * d_in + j) + s * ba[j];
}

/*
 * Row norms of V = W + s*B*A for the listed rows (rows == NULL: all d_out
 * rows in order).  Also returns, for each listed row, the three terms the
 * factored method sums ([SD] abstract: "base, cross, and Gram terms"):
 *   base_i  = sum_j W_ij^2
 *   cross_i = sum_j W_ij * (BA)_ij
 *   gram_i  = sum_j (BA)_ij^2
 * They are taken here from the dense rows, by their plain definitions.
 * Any of n, base, cross, gram may be NULL.
 */
int oracle_norm(const void *W, const void *A, const void *B, int dt, double s,
                int64_t d_out, int64_t d_in, int64_t r,
                const int64_t *rows, int64_t nrows,
                double *n, double *base, double *cross, double *gram)
{
    if (rows == NULL)
        nrows = d_out;
    int failed = 0;
#pragma omp parallel
    {
        double *ba = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        double *v = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        if (ba == NULL || v == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t q = 0; q < nrows; ++q) {
                int64_t i = rows ? rows[q] : q;
                dense_row(W, A, B, dt, s, d_in, r, i, ba, v);
                double vv = 0.0, ww = 0.0, wb = 0.0, bb = 0.0;
                for (int64_t j = 0; j < d_in; ++j) {
                    double w = elem(W, dt, i * d_in + j);
                    vv += v[j] * v[j];
                    ww += w * w;
                    wb += w * ba[j];
                    bb += ba[j] * ba[j];
                }
                if (n) n[q] = sqrt(vv);
                if (base) base[q] = ww;
                if (cross) cross[q] = wb;
                if (gram) gram[q] = bb;
            }
        }
        free(ba);
        free(v);
    }
    return failed ? -1 : 0;
}

/*
 * Forward: y[tt, q] = (m_i / n_i) * sum_j x[t, j] * V[i, j] for listed
 * tokens t = toks[tt] and rows i = rows[q] (NULL lists mean "all, in
 * order").  n_i is the dense row norm, or n_in[i] when n_in is given
 * (the norm held fixed, as a cached or detached norm is).  m and n_in are
 * indexed by the row index i.  y is [ntok][nrow]; n_out (nullable) gets
 * the n_i used, per listed row.
 */
int oracle_forward(const void *x, const void *W, const void *A, const void *B,
                   const double *m, int dt, double s,
                   int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                   const int64_t *toks, int64_t ntok,
                   const int64_t *rows, int64_t nrow,
                   const double *n_in, double *y, double *n_out)
{
    if (toks == NULL)
        ntok = T;
    if (rows == NULL)
        nrow = d_out;
    int failed = 0;
#pragma omp parallel
    {
        double *ba = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        double *v = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        if (ba == NULL || v == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t q = 0; q < nrow; ++q) {
                int64_t i = rows ? rows[q] : q;
                dense_row(W, A, B, dt, s, d_in, r, i, ba, v);
                double n;
                if (n_in) {
                    n = n_in[i];
                } else {
                    double vv = 0.0;
                    for (int64_t j = 0; j < d_in; ++j)
                        vv += v[j] * v[j];
                    n = sqrt(vv);
                }
                if (n_out) n_out[q] = n;
                double g = m[i] / n;
                for (int64_t tt = 0; tt < ntok; ++tt) {
                    int64_t t = toks ? toks[tt] : tt;
                    double h = 0.0;
                    for (int64_t j = 0; j < d_in; ++j)
                        h += elem(x, dt, t * d_in + j) * v[j];
                    y[tt * nrow + q] = g * h;
                }
            }
        }
        free(ba);
        free(v);
    }
    (void)d_out;
    return failed ? -1 : 0;
}

/*
 * Compose alone, by its plain definition (not the rearranged stable form
 * the GPU evaluates): y[t, i] = (m_i / n_i) * (base[t, i] + s * lora[t, i]).
 * base and lora are [T, d_out] in dtype dt; y is [T, d_out] double.
 */
int oracle_compose(const void *base, const void *lora, const double *m,
                   const double *n, int dt, double s, int64_t T, int64_t d_out,
                   double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < d_out; ++i) {
            double b = elem(base, dt, t * d_out + i);
            double l = elem(lora, dt, t * d_out + i);
            y[t * d_out + i] = (m[i] / n[i]) * (b + s * l);
        }
    }
    return 0;
}

/*
 * Merged weight, by its plain definition: W'[q, j] = (m_i / n_i) * V[i, j]
 * for the listed rows i = rows[q] (rows == NULL: all d_out rows), with
 * V = W + s*B*A and n_i its dense row norm, or n_in[i] when given.  The
 * adapted weight folds into one matrix, so inference runs a plain linear
 * layer ([DoRA] Key Points 3 and 5: no added inference latency).  Wm is
 * [nrows][d_in] double.
 */
int oracle_merge(const void *W, const void *A, const void *B, const double *m,
                 int dt, double s, int64_t d_out, int64_t d_in, int64_t r,
                 const int64_t *rows, int64_t nrows, const double *n_in, double *Wm)
{
    if (rows == NULL)
        nrows = d_out;
    int failed = 0;
#pragma omp parallel
    {
        double *ba = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        double *v = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        if (ba == NULL || v == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t q = 0; q < nrows; ++q) {
                int64_t i = rows ? rows[q] : q;
                dense_row(W, A, B, dt, s, d_in, r, i, ba, v);
                double ni = 0.0;
                if (n_in) {
                    ni = n_in[i];
                } else {
                    for (int64_t j = 0; j < d_in; ++j)
                        ni += v[j] * v[j];
                    ni = sqrt(ni);
                }
                for (int64_t j = 0; j < d_in; ++j)
                    Wm[q * d_in + j] = (m[i] / ni) * v[j];
            }
        }
        free(ba);
        free(v);
    }
    (void)d_out;
    return failed ? -1 : 0;
}

/*
 * Backward through the row norm (the gradient without the stop-gradient),
 * all outputs, by the plain chain rule on dense V = W + s*B*A.  Here n is
 * the dense row norm of V itself.  With h = x V^T, g = m / n and
 * dh = dy (.) g, the gradient with respect to V is
 *   dV[i,j] = sum_t dh[t,i] x[t,j] - cn_i V[i,j],
 *   cn_i    = (m_i / n_i^3) sum_t dy[t,i] h[t,i]      (from dn_i/dV_i = V_i / n_i),
 * and, as V depends on A and B through s*B*A,
 *   dA[k,j] = s * sum_i B[i,k] dV[i,j],   dB[i,k] = s * sum_j dV[i,j] A[k,j];
 * dx and dm are the same as with n held constant (n depends on neither).
 * Outputs are double: dx [T][d_in], dA [r][d_in], dB [d_out][r], dm [d_out].
 */
int oracle_backward_through_norm(const void *dy, const void *x, const void *W,
                                 const void *A, const void *B, const double *m,
                                 int dt, double s, int64_t T, int64_t d_in,
                                 int64_t d_out, int64_t r, double *dx, double *dA,
                                 double *dB, double *dm)
{
    size_t nv = (size_t)(d_out * d_in > 0 ? d_out * d_in : 1);
    size_t nh = (size_t)(T * d_out > 0 ? T * d_out : 1);
    size_t nr = (size_t)(d_out > 0 ? d_out : 1);
    double *V = malloc(sizeof(double) * nv);
    double *dV = malloc(sizeof(double) * nv);
    double *hv = malloc(sizeof(double) * nh);
    double *nn = malloc(sizeof(double) * nr);
    double *cn = malloc(sizeof(double) * nr);
    int rc = 0;
    if (!V || !dV || !hv || !nn || !cn) {
        rc = -1;
        goto done;
    }

    /* Dense V and its row norms. */
#pragma omp parallel
    {
        double *ba = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        if (ba != NULL) {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < d_out; ++i) {
                dense_row(W, A, B, dt, s, d_in, r, i, ba, V + i * d_in);
                double sq = 0.0;
                for (int64_t j = 0; j < d_in; ++j)
                    sq += V[i * d_in + j] * V[i * d_in + j];
                nn[i] = sqrt(sq);
            }
        } else {
#pragma omp atomic write
            rc = -1;
        }
        free(ba);
    }
    if (rc)
        goto done;

    /* h = x V^T. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < d_out; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < d_in; ++j)
                acc += elem(x, dt, t * d_in + j) * V[i * d_in + j];
            hv[t * d_out + i] = acc;
        }

    /* dm and the norm coefficient cn. */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d_out; ++i) {
        double dyh = 0.0;
        for (int64_t t = 0; t < T; ++t)
            dyh += elem(dy, dt, t * d_out + i) * hv[t * d_out + i];
        dm[i] = dyh / nn[i];
        cn[i] = m[i] / (nn[i] * nn[i] * nn[i]) * dyh;
    }

    /* dV. */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d_out; ++i)
        for (int64_t j = 0; j < d_in; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                acc += elem(dy, dt, t * d_out + i) * (m[i] / nn[i]) * elem(x, dt, t * d_in + j);
            dV[i * d_in + j] = acc - cn[i] * V[i * d_in + j];
        }

    /* dx = dh V. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < d_in; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < d_out; ++i)
                acc += elem(dy, dt, t * d_out + i) * (m[i] / nn[i]) * V[i * d_in + j];
            dx[t * d_in + j] = acc;
        }

    /* dA = s B^T dV, dB = s dV A^T. */
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < r; ++k)
        for (int64_t j = 0; j < d_in; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < d_out; ++i)
                acc += elem(B, dt, i * r + k) * dV[i * d_in + j];
            dA[k * d_in + j] = acc * s;
        }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d_out; ++i)
        for (int64_t k = 0; k < r; ++k) {
            double acc = 0.0;
            for (int64_t j = 0; j < d_in; ++j)
                acc += dV[i * d_in + j] * elem(A, dt, k * d_in + j);
            dB[i * r + k] = acc * s;
        }

done:
    free(V);
    free(dV);
    free(hv);
    free(nn);
    free(cn);
    return rc;
}

/*
 * Backward with the row norm n held constant, all outputs, for sizes the
 * dense [d_out, d_in] V fits in host memory.  With g_i = m_i / n_i,
 * h = x V^T and dh = dy (.) g:
 *   dm_i    = sum_t dy[t,i] * h[t,i] / n_i
 *   dx[t,j] = sum_i dh[t,i] * V[i,j]
 *   dB[i,k] = s * sum_t dh[t,i] * P[t,k],   P[t,k] = sum_j x[t,j] * A[k,j]
 *   dA[k,j] = s * sum_t Q[t,k] * x[t,j],    Q[t,k] = sum_i dh[t,i] * B[i,k]
 * Outputs are double: dx [T][d_in], dA [r][d_in], dB [d_out][r], dm [d_out].
 */
int oracle_backward_full(const void *dy, const void *x, const void *W,
                         const void *A, const void *B, const double *m,
                         const double *n, int dt, double s,
                         int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                         double *dx, double *dA, double *dB, double *dm)
{
    size_t nv = (size_t)(d_out * d_in > 0 ? d_out * d_in : 1);
    size_t nh = (size_t)(T * d_out > 0 ? T * d_out : 1);
    size_t np = (size_t)(T * r > 0 ? T * r : 1);
    double *V = malloc(sizeof(double) * nv);
    double *h = malloc(sizeof(double) * nh);
    double *dh = malloc(sizeof(double) * nh);
    double *P = malloc(sizeof(double) * np);
    double *Q = malloc(sizeof(double) * np);
    int rc = 0;
    if (!V || !h || !dh || !P || !Q) {
        rc = -1;
        goto out;
    }

    /* Dense V, row by row. */
#pragma omp parallel
    {
        double *ba = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        if (ba != NULL) {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < d_out; ++i)
                dense_row(W, A, B, dt, s, d_in, r, i, ba, V + i * d_in);
        } else {
#pragma omp atomic write
            rc = -1;
        }
        free(ba);
    }
    if (rc)
        goto out;

    /* h = x V^T and dh = dy (.) g. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < d_out; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < d_in; ++j)
                acc += elem(x, dt, t * d_in + j) * V[i * d_in + j];
            h[t * d_out + i] = acc;
            dh[t * d_out + i] = elem(dy, dt, t * d_out + i) * (m[i] / n[i]);
        }
    }

    /* dm. */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d_out; ++i) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t)
            acc += elem(dy, dt, t * d_out + i) * h[t * d_out + i];
        dm[i] = acc / n[i];
    }

    /* dx. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < d_in; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < d_out; ++i)
                acc += dh[t * d_out + i] * V[i * d_in + j];
            dx[t * d_in + j] = acc;
        }
    }

    /* P = x A^T and Q = dh B. */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < r; ++k) {
            double p = 0.0, qv = 0.0;
            for (int64_t j = 0; j < d_in; ++j)
                p += elem(x, dt, t * d_in + j) * elem(A, dt, k * d_in + j);
            for (int64_t i = 0; i < d_out; ++i)
                qv += dh[t * d_out + i] * elem(B, dt, i * r + k);
            P[t * r + k] = p;
            Q[t * r + k] = qv;
        }
    }

    /* dB and dA. */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d_out; ++i) {
        for (int64_t k = 0; k < r; ++k) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                acc += dh[t * d_out + i] * P[t * r + k];
            dB[i * r + k] = s * acc;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < r; ++k) {
        for (int64_t j = 0; j < d_in; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                acc += Q[t * r + k] * elem(x, dt, t * d_in + j);
            dA[k * d_in + j] = s * acc;
        }
    }

out:
    free(V);
    free(h);
    free(dh);
    free(P);
    free(Q);
    return rc;
}

/*
 * Backward with n held constant, selected entries only, each computed on
 * its own from the definitions above (for module shapes where dense V or
 * full gradients would be too slow on the CPU).  Index lists are pairs,
 * row-major: dx_idx = {t0, j0, t1, j1, ...}, dA_idx = {k, j, ...},
 * dB_idx = {i, k, ...}; dm_idx = {i, ...}.
 */
int oracle_backward_sampled(const void *dy, const void *x, const void *W,
                            const void *A, const void *B, const double *m,
                            const double *n, int dt, double s,
                            int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                            const int64_t *dx_idx, int64_t n_dx, double *dx,
                            const int64_t *dA_idx, int64_t n_dA, double *dA,
                            const int64_t *dB_idx, int64_t n_dB, double *dB,
                            const int64_t *dm_idx, int64_t n_dm, double *dm)
{
    int failed = 0;

    /* dx[t,j] = sum_i dy[t,i] g_i V[i,j],  V[i,j] = W[i,j] + s sum_k B[i,k] A[k,j]. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_dx; ++q) {
        int64_t t = dx_idx[2 * q], j = dx_idx[2 * q + 1];
        double acc = 0.0;
        for (int64_t i = 0; i < d_out; ++i) {
            double ba = 0.0;
            for (int64_t k = 0; k < r; ++k)
                ba += elem(B, dt, i * r + k) * elem(A, dt, k * d_in + j);
            double vij = elem(W, dt, i * d_in + j) + s * ba;
            acc += elem(dy, dt, t * d_out + i) * (m[i] / n[i]) * vij;
        }
        dx[q] = acc;
    }

    /* dA[k,j] = s sum_t (sum_i dy[t,i] g_i B[i,k]) x[t,j]. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_dA; ++q) {
        int64_t k = dA_idx[2 * q], j = dA_idx[2 * q + 1];
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double qtk = 0.0;
            for (int64_t i = 0; i < d_out; ++i)
                qtk += elem(dy, dt, t * d_out + i) * (m[i] / n[i]) * elem(B, dt, i * r + k);
            acc += qtk * elem(x, dt, t * d_in + j);
        }
        dA[q] = s * acc;
    }

    /* dB[i,k] = s sum_t dy[t,i] g_i (sum_j x[t,j] A[k,j]). */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_dB; ++q) {
        int64_t i = dB_idx[2 * q], k = dB_idx[2 * q + 1];
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double ptk = 0.0;
            for (int64_t j = 0; j < d_in; ++j)
                ptk += elem(x, dt, t * d_in + j) * elem(A, dt, k * d_in + j);
            acc += elem(dy, dt, t * d_out + i) * (m[i] / n[i]) * ptk;
        }
        dB[q] = s * acc;
    }

    /* dm_i = sum_t dy[t,i] (sum_j x[t,j] V[i,j]) / n_i. */
#pragma omp parallel
    {
        double *ba = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        double *v = malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        if (ba == NULL || v == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t q = 0; q < n_dm; ++q) {
                int64_t i = dm_idx[q];
                dense_row(W, A, B, dt, s, d_in, r, i, ba, v);
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    double h = 0.0;
                    for (int64_t j = 0; j < d_in; ++j)
                        h += elem(x, dt, t * d_in + j) * v[j];
                    acc += elem(dy, dt, t * d_out + i) * h;
                }
                dm[q] = acc / n[i];
            }
        }
        free(ba);
        free(v);
    }
    return failed ? -1 : 0;
}
