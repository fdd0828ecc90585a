/*
 * libsgemm -- 2-D convolution for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The UNIVERSAL_SGEMM_CUDA README ("Results" section) times six GEMM shapes
 * of convolution layers lowered to matrix products by im2col; the page names
 * neither the layers nor the lowering.  These entry points compute such
 * layers from the input itself, and the im2col matrix for the lowered
 * product (sgemm_f32 on it gives the same result), as image networks define
 * the convolution (cross-correlation, the filter not flipped):
 *
 *   input   X: batch x channels x height x width floats, packed (NCHW),
 *           X[((b*channels + c)*height + ih)*width + iw]
 *   filters Wt: out_channels rows, row m = filter m flattened, tap
 *           k = (c*kernel_h + r)*kernel_w + s at Wt[m*ldw + k]
 *           (K = channels*kernel_h*kernel_w taps, ldw >= K)
 *   output  OH = (height + 2 pad_h - kernel_h) / stride_h + 1, OW likewise;
 *           Y: out_channels rows of N = batch*OH*OW positions, row m at
 *           Y[m*ldy], position n = (b*OH + oh)*OW + ow (the layout the
 *           lowered product C = Wt * B writes; ldy >= N)
 *   tap     X at (b, c, oh*stride_h - pad_h + r, ow*stride_w - pad_w + s),
 *           zero outside the image (the zeros are multiplied like any tap)
 *
 *   Y[m][n] <- alpha * sum_k Wt[m][k] * tap_k(n) + beta * Y[m][n]
 *
 * All pointers are device pointers on the current HIP device, owned by the
 * caller; Y must not overlap X or Wt.  Calls queue kernels on `stream` and
 * return; they allocate, free, copy and synchronise nothing, so they may be
 * captured into a HIP graph.  Results are visible once the stream has been
 * synchronised.
 */
#ifndef LIBSGEMM_SCONV_H
#define LIBSGEMM_SCONV_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel forms for sconv2d_f32_variant(). */
enum sconv_variant {
    SCONV_VARIANT_AUTO = 0,   /* a pointwise layer (1x1 filter, stride 1, no
                               * padding) as one sgemm_f32 per image on X in
                               * place; else the stem kernel where it applies,
                               * else the tile kernel (its tap form, else its
                               * direct form, where those apply) where its
                               * tiles keep the CUs busier, else general */
    SCONV_VARIANT_STEM = 1,   /* input rows staged in LDS once per 256 output
                               * positions; only the geometries it is built for
                               * (3 channels, 7x7 or 3x3 filters at stride 2,
                               * pad <= 4, images up to 224 + padding wide,
                               * out_channels <= 64, X and Y under 4 GiB);
                               * others return
                               * SGEMM_ERR_VARIANT_SHAPE (include/sgemm.h) */
    SCONV_VARIANT_GENERAL = 2, /* any geometry: 64 x 64 output tiles, taps gathered
                                * from X into LDS in slabs of 16 */
    SCONV_VARIANT_TILE = 3,    /* matrix-core tiles (64, 128 or 192 x 128) with
                                * taps gathered into a three-slab LDS ring, the
                                * contraction walked tap by tap over blocks of 16
                                * channels; any geometry with X and the filter
                                * rows under 2^31 bytes; others return
                                * SGEMM_ERR_VARIANT_SHAPE */
    SCONV_VARIANT_DIRECT = 4,  /* the tile kernel's fast form: both operands loaded
                                * straight into LDS; 3x3 and 1x1 filters, K a
                                * multiple of 16, Wt 16-byte aligned with ldw a
                                * multiple of 4, and the tile form's limits;
                                * others return SGEMM_ERR_VARIANT_SHAPE */
    SCONV_VARIANT_TAP = 5      /* the direct form with one filter tap per matrix
                                * k-step (slabs of 4 channels x 9 taps); 3x3
                                * filters, channels a multiple of 4, Wt as for
                                * SCONV_VARIANT_DIRECT; others return
                                * SGEMM_ERR_VARIANT_SHAPE */
};

/*
 * sconv2d_f32 -- Y <- alpha * conv(X, filters) + beta * Y, as defined above.
 *
 *   batch, channels, height, width   input extent (batch >= 0, others >= 1)
 *   out_channels                     M >= 0, rows of Wt and Y
 *   kernel_h, kernel_w               filter extent, >= 1
 *   stride_h, stride_w               >= 1
 *   pad_h, pad_w                     zero padding on each side, >= 0
 *   alpha                            alpha == 0: X and Wt are not read
 *   X, Wt, ldw                       input and filters (ldw >= K)
 *   beta                             beta == 0: Y is written, not read
 *   Y, ldy                           output (ldy >= max(1, N))
 *
 * Returns 0; -p for the first invalid parameter p, counting batch as 1:
 *   -1 batch < 0 (or N > INT_MAX), -2 channels < 1 (or K > INT_MAX),
 *   -3 height < 1, -4 width < 1, -5 out_channels < 0,
 *   -6 kernel_h < 1 or > height + 2 pad_h, -7 kernel_w likewise,
 *   -8 stride_h < 1, -9 stride_w < 1, -10 pad_h < 0 (or height + 2 pad_h
 *   > INT_MAX), -11 pad_w likewise,
 *  -13 X NULL or not 4-byte aligned (while it is read), -14 Wt likewise,
 *  -15 ldw < K, -17 Y NULL or not 4-byte aligned (while M*N > 0),
 *  -18 ldy < max(1, N);
 * checked before any HIP call.  A positive value is the hipError_t of a
 * failed HIP call (nothing was queued then).  batch, out_channels or N
 * zero: nothing to do.
 *
 * Accuracy: as sgemm_f32, each output is a fp32 sum of fp32 products of
 * K terms; within 1e-5 * (|alpha| sum_k |w x| + |beta y|) + 1e-6 of the
 * exact value for data like the benchmark's, exact for integer data whose
 * partial sums stay below 2^24 (then equal, bit for bit, to sgemm_f32 on
 * the im2col matrix).
 *
 * Thread safety: re-entrant; the shared state is a per-device cache of the
 * compute-unit count and, for pointwise layers (run through sgemm_f32), the
 * stream-K workspace slots sgemm_f32 documents.
 */
int sconv2d_f32(int batch, int channels, int height, int width, int out_channels,
                int kernel_h, int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w,
                float alpha, const float *X, const float *Wt, int ldw, float beta, float *Y,
                int ldy, hipStream_t stream);

/* As sconv2d_f32 with the kernel form forced (enum sconv_variant); returns
 * SGEMM_ERR_BAD_VARIANT for an unknown variant (checked first), then the
 * argument checks, then SGEMM_ERR_VARIANT_SHAPE when the stem form cannot
 * run the geometry.  For tests and measurement. */
int sconv2d_f32_variant(int variant, int batch, int channels, int height, int width,
                        int out_channels, int kernel_h, int kernel_w, int stride_h,
                        int stride_w, int pad_h, int pad_w, float alpha, const float *X,
                        const float *Wt, int ldw, float beta, float *Y, int ldy,
                        hipStream_t stream);

/*
 * sgemm_im2col_f32 -- write B, the K x N im2col matrix of X (K =
 * channels*kernel_h*kernel_w, N = batch*OH*OW): B[k*ldb + n] is tap k of
 * output position n, zero outside the image.  sgemm_f32(M, N, K, alpha, Wt,
 * ldw, B, ldb, beta, Y, ldy) then computes what sconv2d_f32 computes.  B is
 * written with non-temporal stores (it is read once, later).  Returns 0,
 * -p as sconv2d_f32 for the parameters it shares (counting batch as 1:
 * -1 .. -4, then -5 kernel_h .. -10 pad_w), -11 X, -12 B (NULL or not
 * 4-byte aligned while N > 0), -13 ldb < max(1, N); or a hipError_t.
 */
int sgemm_im2col_f32(int batch, int channels, int height, int width, int kernel_h,
                     int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w,
                     const float *X, float *B, int ldb, hipStream_t stream);

/*
 * sconv2d_plan -- describe, without touching any GPU, the kernel
 * sconv2d_f32_variant would launch on a device with num_cus compute units
 * (for packed filters, 16-byte aligned):
 *   "stem mb=2 k=147 window=3x13x232 strip=256 strips=6272 grid=512 oh=112 ow=112"
 *   "gemm images=1 m=256 n=50176 k=1024 oh=224 ow=224"   (one sgemm_f32 per image)
 *   "tap bm=192 bn=128 waves=8 k=1152 grid=222 oh=119 ow=119"
 *   "direct bm=128 bn=128 waves=4 k=256 grid=1568 oh=56 ow=56"
 *   "tile bm=64 bn=128 waves=4 k=255 grid=3 oh=21 ow=9"
 *   "general tile=64x64 k=1152 grid=... oh=... ow=..."   or "none".
 * Writes at most buflen bytes (NUL-terminated).  Returns 0, the argument
 * codes of sconv2d_f32 for the geometry, SGEMM_ERR_BAD_VARIANT,
 * SGEMM_ERR_VARIANT_SHAPE, or -12 when num_cus < 1 or buf is NULL with
 * buflen > 0.
 */
int sconv2d_plan(int variant, int batch, int channels, int height, int width, int out_channels,
                 int kernel_h, int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w,
                 int num_cus, char *buf, int buflen);

/* Number of stem kernels built (geometries the stem form takes). */
int sconv2d_num_stem_kernels(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSGEMM_SCONV_H */
