/*
 * Reference SGEMM oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow definition that the GPU library is checked
 * against.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg load it; the product library never links, calls or includes
 * anything here, and this file includes nothing from the product.
 *
 * What it computes (row-major storage, A is M x K, B is K x N, C is M x N):
 *
 *     C[i][j] <- alpha * sum_k A[i][k] * B[k][j]  +  beta * C[i][j]
 *
 * Sources:
 *   - The triple loop over i, j, k and row-major indexing follow the CPU
 *     reference function of "matmul_opt.cu" (cnblogs post, page 3), which
 *     sums A[i*K+k]*B[k*N+j] over k for every (i, j).
 *   - The alpha/beta epilogue follows the naive kernel of the
 *     NVIDIA_SGEMM_PRACTICE README ("kernel 1" section), which writes
 *     alpha*tmp + beta*C.
 *   - Leading dimensions follow that README's OFFSET(row, col, ld) macro
 *     ("kernel 6" section): element (r, c) lives at r*ld + c.
 *
 * Readings where the pages are silent:
 *   - Products and sums are taken in double precision and rounded to float
 *     once at the end (the page-3 reference sums in float; the spec of this
 *     library asks for fp64 accumulation).  A product of two floats is exact
 *     in double, so only the k-summation rounds.
 *   - k is summed in ascending order for every element.
 *   - beta == 0 means C is not read (BLAS convention), so NaN in C does not
 *     leak into the result.
 *   - alpha == 0 or K == 0 means A and B are not read.
 *   - Every partial sum is computed without fused multiply-add; build with
 *     -ffp-contract=off.
 *
 * Parallelism: rows of C are split across OpenMP threads.  Each output
 * element is owned by exactly one thread and its k-order is fixed, so the
 * bits do not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Epilogue for one element, one rounding from double to float at the end.
 * With alpha == 0 the product term is absent (A and B were not read); with
 * beta == 0 the old value of C is absent (C was not read).
 */
static float finish(double alpha, double s, double beta, const float *c)
{
    double r = 0.0;
    if (alpha != 0.0)
        r = alpha * s;
    if (beta != 0.0)
        r = (alpha != 0.0) ? r + beta * (double)(*c) : beta * (double)(*c);
    return (float)r;
}

/*
 * Full product.  On return C holds the new values; if absdot is not NULL,
 * absdot[i*ldt + j] = sum_k |A[i][k] * B[k][j]| (the scale used by the
 * tolerance test).  Returns 0, or -1 if scratch memory could not be had.
 *
 * Loop order is i, then k, then j with one double accumulator per column:
 * every element still sums its K products in ascending k, exactly as the
 * i-j-k loop does, but B is walked row by row.
 */
int oracle_sgemm(int M, int N, int K, float alpha, const float *A, int lda,
                 const float *B, int ldb, float beta, float *C, int ldc,
                 double *absdot, int ldt)
{
    int failed = 0;
    if (M <= 0 || N <= 0)
        return 0;

#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N);
        double *mag = (double *)malloc(sizeof(double) * (size_t)N);
        if (acc == NULL || mag == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int i = 0; i < M; ++i) {
                for (int j = 0; j < N; ++j) {
                    acc[j] = 0.0;
                    mag[j] = 0.0;
                }
                if (alpha != 0.0f) {
                    for (int k = 0; k < K; ++k) {
                        const double a = (double)A[(size_t)i * lda + k];
                        const float *brow = B + (size_t)k * ldb;
                        for (int j = 0; j < N; ++j) {
                            const double p = a * (double)brow[j];
                            acc[j] = acc[j] + p;
                            mag[j] = mag[j] + fabs(p);
                        }
                    }
                }
                float *crow = C + (size_t)i * ldc;
                for (int j = 0; j < N; ++j)
                    crow[j] = finish((double)alpha, acc[j], (double)beta, &crow[j]);
                if (absdot != NULL) {
                    double *trow = absdot + (size_t)i * ldt;
                    for (int j = 0; j < N; ++j)
                        trow[j] = mag[j];
                }
            }
        }
        free(acc);
        free(mag);
    }
    return failed ? -1 : 0;
}

/*
 * Selected elements only, for shapes too large to compute whole.  For each
 * p < npts, with (i, j) = (rows[p], cols[p]):
 *     out[p]    = float(alpha * sum_k A[i][k]*B[k][j] + beta * Cin[i][j])
 *     absdot[p] = sum_k |A[i][k]*B[k][j]|          (if absdot is not NULL)
 * Cin is read only when beta != 0.  This is the i-j-k loop written out.
 */
void oracle_sgemm_points(int K, float alpha, const float *A, int lda,
                         const float *B, int ldb, float beta,
                         const float *Cin, int ldc, int npts,
                         const int *rows, const int *cols, float *out,
                         double *absdot)
{
#pragma omp parallel for schedule(static)
    for (int p = 0; p < npts; ++p) {
        const size_t i = (size_t)rows[p];
        const size_t j = (size_t)cols[p];
        double s = 0.0, t = 0.0;
        if (alpha != 0.0f) {
            for (int k = 0; k < K; ++k) {
                const double prod = (double)A[i * lda + k] * (double)B[(size_t)k * ldb + j];
                s = s + prod;
                t = t + fabs(prod);
            }
        }
        out[p] = finish((double)alpha, s, (double)beta,
                        beta != 0.0f ? Cin + i * (size_t)ldc + j : NULL);
        if (absdot != NULL)
            absdot[p] = t;
    }
}

/* Number of threads the OpenMP runtime will use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
