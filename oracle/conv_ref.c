/*
 * Reference 2-D convolution and im2col -- TEST INFRASTRUCTURE ONLY.
 *
 * Like sgemm_ref.c, this file is the plain, slow definition that the GPU
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product library never links,
 * calls or includes anything here, and this file includes nothing from the
 * product.
 *
 * Where the operation comes from: the UNIVERSAL_SGEMM_CUDA README
 * ("Results" section) times six GEMM shapes of convolution layers lowered
 * to matrix products; the page names neither the layers nor the lowering.
 * This file states the convolution those shapes stand for, as image
 * networks define it (cross-correlation: the filter is not flipped), and
 * the im2col lowering that turns it into C = W * B:
 *
 *   input   X[b][c][ih][iw]   b < batch, c < C, ih < H, iw < W   (NCHW, packed)
 *   filter  F[m][c][r][s]     m < M, r < R, s < S; row m of the weight matrix
 *                             is F[m] flattened, k = (c*R + r)*S + s,
 *                             at Wt[m*ldw + k]
 *   output  OH = (H + 2*ph - R) / sh + 1,  OW = (W + 2*pw - S) / sw + 1
 *           n = (b*OH + oh)*OW + ow,  Y[m*ldy + n]
 *   tap     x(b, c, oh*sh - ph + r, ow*sw - pw + s), zero outside the image
 *
 *   Y[m][n] <- alpha * sum_k Wt[m][k] * B[k][n] + beta * Y[m][n]
 *   B[k][n] =  the tap of (c, r, s) for output position n  (im2col)
 *
 * Readings of the pages (where they leave the convolution open):
 *   - Zero padding holds real zeros: a tap outside the image contributes
 *     w * 0, which is 0 for finite w and NaN for an infinite or NaN weight,
 *     exactly as the product with the im2col matrix does.
 *   - The output is left in the layout the lowered product writes: one row
 *     per output channel, columns in (b, oh, ow) order.
 *   - As in sgemm_ref.c: products and sums in double, k ascending, one
 *     rounding to float; beta == 0 means Y is not read; alpha == 0 means
 *     neither X nor the weights are read.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Output extent along one axis; the caller checks in + 2 pad >= k. */
int oracle_conv_out_size(int in, int k, int stride, int pad)
{
    return (in + 2 * pad - k) / stride + 1;
}

/* The tap value: X at (b, c, ih, iw), or 0 outside the image. */
static float tap(const float *X, int C, int H, int W, int b, int c, int ih, int iw)
{
    if (ih < 0 || ih >= H || iw < 0 || iw >= W)
        return 0.0f;
    return X[(((size_t)b * C + c) * H + ih) * W + iw];
}

/* Epilogue for one element (the same rule as the GEMM reference). */
static float conv_finish(double alpha, double s, double beta, const float *y)
{
    double v = 0.0;
    if (alpha != 0.0)
        v = alpha * s;
    if (beta != 0.0)
        v = (alpha != 0.0) ? v + beta * (double)(*y) : beta * (double)(*y);
    return (float)v;
}

/*
 * im2col: B[k*ldb + n] for k < C*R*S, n < batch*OH*OW, as defined above.
 */
void oracle_im2col(int batch, int C, int H, int W, int R, int S, int sh, int sw, int ph,
                   int pw, const float *X, float *B, long ldb)
{
    const int OH = oracle_conv_out_size(H, R, sh, ph);
    const int OW = oracle_conv_out_size(W, S, sw, pw);
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c)
        for (int r = 0; r < R; ++r)
            for (int s = 0; s < S; ++s) {
                const size_t k = ((size_t)c * R + r) * S + s;
                float *brow = B + k * (size_t)ldb;
                for (int b = 0; b < batch; ++b)
                    for (int oh = 0; oh < OH; ++oh)
                        for (int ow = 0; ow < OW; ++ow) {
                            const size_t n = ((size_t)b * OH + oh) * OW + ow;
                            brow[n] = tap(X, C, H, W, b, c, oh * sh - ph + r, ow * sw - pw + s);
                        }
            }
}

/*
 * Direct convolution.  For every output channel m and output position n, the
 * taps are summed in ascending k = (c, r, s) with a double accumulator, then
 * rounded once.  absdot, if not NULL, receives sum_k |w * x| at
 * absdot[m*ldt + n].  Returns 0, or -1 if scratch memory could not be had.
 */
int oracle_conv2d(int batch, int C, int H, int W, int M, int R, int S, int sh, int sw,
                  int ph, int pw, float alpha, const float *X, const float *Wt, long ldw,
                  float beta, float *Y, long ldy, double *absdot, long ldt)
{
    const int OH = oracle_conv_out_size(H, R, sh, ph);
    const int OW = oracle_conv_out_size(W, S, sw, pw);
    const int K = C * R * S;
    int failed = 0;
    if (M <= 0 || batch <= 0 || OH <= 0 || OW <= 0)
        return 0;

#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)OW);
        double *mag = (double *)malloc(sizeof(double) * (size_t)OW);
        if (acc == NULL || mag == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for collapse(2) schedule(static)
            for (int m = 0; m < M; ++m)
                for (int b = 0; b < batch; ++b)
                    for (int oh = 0; oh < OH; ++oh) {
                        for (int ow = 0; ow < OW; ++ow) {
                            acc[ow] = 0.0;
                            mag[ow] = 0.0;
                        }
                        if (alpha != 0.0f) {
                            for (int k = 0; k < K; ++k) {
                                const int c = k / (R * S), r = (k / S) % R, s = k % S;
                                const double w = (double)Wt[(size_t)m * ldw + k];
                                for (int ow = 0; ow < OW; ++ow) {
                                    const double x = (double)tap(X, C, H, W, b, c,
                                                                 oh * sh - ph + r,
                                                                 ow * sw - pw + s);
                                    const double p = w * x;
                                    acc[ow] = acc[ow] + p;
                                    mag[ow] = mag[ow] + fabs(p);
                                }
                            }
                        }
                        const size_t n0 = ((size_t)b * OH + oh) * OW;
                        float *yrow = Y + (size_t)m * ldy + n0;
                        for (int ow = 0; ow < OW; ++ow)
                            yrow[ow] = conv_finish((double)alpha, acc[ow], (double)beta,
                                                   &yrow[ow]);
                        if (absdot != NULL) {
                            double *trow = absdot + (size_t)m * ldt + n0;
                            for (int ow = 0; ow < OW; ++ow)
                                trow[ow] = mag[ow];
                        }
                    }
        }
        free(acc);
        free(mag);
    }
    return failed ? -1 : 0;
}
