// libsgemm convolution entry points: argument checks, the choice between
// the stem kernel and the general implicit-GEMM kernel, and the im2col
// producer, behind the C ABI declared in include/sconv.h.  Like the GEMM
// entry points, nothing here allocates, frees, copies or synchronises: work
// is queued on the caller's stream.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/sconv.h"
#include "../../include/sgemm.h"
#include "conv.hpp"

namespace sgemm {
namespace {

struct Geometry {
    int batch, C, H, W, M, R, S, sh, sw, ph, pw;
};

// Checks shared by the entry points (no HIP call).  Returns 0 or -p, p the
// position of the first bad parameter in sconv2d_f32's list.
int check_geometry(const Geometry &q, int *OH, int *OW, int64_t *N)
{
    if (q.batch < 0) return -1;
    if (q.C < 1) return -2;
    if (q.H < 1) return -3;
    if (q.W < 1) return -4;
    if (q.M < 0) return -5;
    if (q.R < 1) return -6;
    if (q.S < 1) return -7;
    if (q.sh < 1) return -8;
    if (q.sw < 1) return -9;
    if (q.ph < 0) return -10;
    if (q.pw < 0) return -11;
    if ((int64_t)q.H + 2 * q.ph < q.R) return -6;
    if ((int64_t)q.W + 2 * q.pw < q.S) return -7;
    if ((int64_t)q.C * q.R * q.S > INT_MAX) return -2;
    *OH = (q.H + 2 * q.ph - q.R) / q.sh + 1;
    *OW = (q.W + 2 * q.pw - q.S) / q.sw + 1;
    *N = (int64_t)q.batch * *OH * *OW;
    if (*N > INT_MAX) return -1;
    return 0;
}

// The stem kernels built: geometry, row blocks, window shape, waves per SIMD.
struct StemEntry {
    int C, R, S, sh, sw, mb, wpitch, rows, wpe;
    ConvKernelFn fn;
};

#define SGEMM_STEM(MB, CH, R, S, SH, SW, WP, ROWS, WPE) \
    {CH, R, S, SH, SW, MB, WP, ROWS, WPE, conv_stem_kernel<MB, CH, R, S, SH, SW, WP, ROWS, WPE>}

// Windows for 224-wide images: 232 columns hold the image and its padding
// (column 4 is input column 0); 13 rows (7 x 7, stride 2) or 9 (3 x 3,
// stride 2) cover the four output rows a 256-position strip of a 112-wide
// output touches.  LDS: 75 KB (7 x 7) and 30 KB (3 x 3); two workgroups
// per CU (four waves each: the register budget of two waves per SIMD).
const StemEntry kStems[] = {
    SGEMM_STEM(2, 3, 7, 7, 2, 2, 232, 13, 2),
    SGEMM_STEM(1, 3, 7, 7, 2, 2, 232, 13, 2),
    SGEMM_STEM(2, 3, 3, 3, 2, 2, 232, 9, 2),
    SGEMM_STEM(1, 3, 3, 3, 2, 2, 232, 9, 2),
};
constexpr int kNumStems = (int)(sizeof(kStems) / sizeof(kStems[0]));

// The stem entry that can run this problem, or null: same filter, channels
// and strides, M within its row blocks (the smallest that fits), the padded
// image inside the window's width, and every strip's input rows inside the
// window's height.
const StemEntry *stem_for(const Geometry &q, int OH, int OW)
{
    const StemEntry *best = nullptr;
    for (const StemEntry &e : kStems) {
        if (e.C != q.C || e.R != q.R || e.S != q.S || e.sh != q.sh || e.sw != q.sw) continue;
        if (q.M > 32 * e.mb) continue;
        if (q.pw > kStemCol0) continue;
        const int64_t last_col = (int64_t)(OW - 1) * q.sw - q.pw + q.S - 1 + kStemCol0;
        if (last_col >= e.wpitch) continue;
        const int64_t out_rows = (kStemStrip + OW - 2) / OW;  // output rows a strip spans - 1
        if (out_rows * q.sh + q.R > e.rows) continue;
        (void)OH;
        if (best == nullptr || e.mb < best->mb) best = &e;
    }
    return best;
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Per-device compute-unit count, cached.
constexpr int kConvMaxDevices = 64;
int g_conv_cus[kConvMaxDevices];

hipError_t conv_device_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kConvMaxDevices && g_conv_cus[dev] > 0) {
        *cus = g_conv_cus[dev];
        return hipSuccess;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    if (dev >= 0 && dev < kConvMaxDevices) g_conv_cus[dev] = n;
    *cus = n;
    return hipSuccess;
}

int conv_launch(int variant, const Geometry &q, float alpha, const float *X, const float *Wt,
                int ldw, float beta, float *Y, int ldy, hipStream_t stream)
{
    if (variant < SCONV_VARIANT_AUTO || variant > SCONV_VARIANT_GENERAL) return SGEMM_ERR_BAD_VARIANT;
    int OH = 0, OW = 0;
    int64_t N = 0;
    const int bad = check_geometry(q, &OH, &OW, &N);
    if (bad != 0) return bad;
    const int K = q.C * q.R * q.S;
    const bool reads = alpha != 0.0f && q.M > 0 && N > 0;
    if (reads && (X == nullptr || ((uintptr_t)X & 3u) != 0)) return -13;
    if (reads && (Wt == nullptr || ((uintptr_t)Wt & 3u) != 0)) return -14;
    if (ldw < K) return -15;
    if (q.M > 0 && N > 0 && (Y == nullptr || ((uintptr_t)Y & 3u) != 0)) return -17;
    if ((int64_t)ldy < (N > 1 ? N : 1)) return -18;
    const StemEntry *stem = stem_for(q, OH, OW);
    // The stem kernel addresses X and Y with 32-bit byte offsets.
    const int64_t x_bytes = 4 * (int64_t)q.batch * q.C * q.H * q.W;
    const int64_t y_bytes = 4 * (int64_t)q.M * ldy;
    if (x_bytes >= (1ll << 32) || y_bytes >= (1ll << 32)) stem = nullptr;
    if (variant == SCONV_VARIANT_STEM && stem == nullptr) return SGEMM_ERR_VARIANT_SHAPE;
    if (q.M == 0 || N == 0) return 0;

    if (alpha == 0.0f) {
        int64_t blocks = ceil_div64((int64_t)q.M * N, 256);
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(conv_scale_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, Y,
                           (int64_t)ldy, q.M, N, beta);
        return (int)hipGetLastError();
    }

    ConvArgs a;
    a.X = X;
    a.Wt = Wt;
    a.Y = Y;
    a.ldw = ldw;
    a.ldy = ldy;
    a.batch = q.batch;
    a.C = q.C;
    a.H = q.H;
    a.W = q.W;
    a.M = q.M;
    a.R = q.R;
    a.S = q.S;
    a.sh = q.sh;
    a.sw = q.sw;
    a.ph = q.ph;
    a.pw = q.pw;
    a.OH = OH;
    a.OW = OW;
    a.K = K;
    a.N = N;
    a.alpha = alpha;
    a.beta = beta;

    if (stem != nullptr && variant != SCONV_VARIANT_GENERAL) {
        int cus = 0;
        const hipError_t e = conv_device_cus(&cus);
        if (e != hipSuccess) return (int)e;
        const int spi = (int)ceil_div64((int64_t)OH * OW, kStemStrip);
        const int64_t total = (int64_t)spi * q.batch;
        if (total > INT_MAX) return (int)hipErrorInvalidConfiguration;
        // A workgroup is four waves, one per SIMD: wpe of them fit a CU.
        const int64_t resident = (int64_t)cus * stem->wpe;
        const int64_t grid = total < resident ? total : resident;
        hipLaunchKernelGGL(stem->fn, dim3((unsigned)grid), dim3(256), 0, stream, a, spi,
                           (int)total);
        return (int)hipGetLastError();
    }
    const int tiles_m = (int)ceil_div64(q.M, kConvTile);
    const int64_t blocks = (int64_t)tiles_m * ceil_div64(N, kConvTile);
    if (blocks > INT_MAX) return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(conv_gemm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, tiles_m,
                       0);
    return (int)hipGetLastError();
}

}  // namespace
}  // namespace sgemm

using sgemm::Geometry;

extern "C" int sconv2d_f32_variant(int variant, int batch, int channels, int height, int width,
                                   int out_channels, int kernel_h, int kernel_w, int stride_h,
                                   int stride_w, int pad_h, int pad_w, float alpha,
                                   const float *X, const float *Wt, int ldw, float beta, float *Y,
                                   int ldy, hipStream_t stream)
{
    const Geometry q = {batch,    channels, height,   width,    out_channels, kernel_h,
                        kernel_w, stride_h, stride_w, pad_h,    pad_w};
    return sgemm::conv_launch(variant, q, alpha, X, Wt, ldw, beta, Y, ldy, stream);
}

extern "C" int sconv2d_f32(int batch, int channels, int height, int width, int out_channels,
                           int kernel_h, int kernel_w, int stride_h, int stride_w, int pad_h,
                           int pad_w, float alpha, const float *X, const float *Wt, int ldw,
                           float beta, float *Y, int ldy, hipStream_t stream)
{
    return sconv2d_f32_variant(SCONV_VARIANT_AUTO, batch, channels, height, width, out_channels,
                               kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w, alpha, X, Wt,
                               ldw, beta, Y, ldy, stream);
}

extern "C" int sgemm_im2col_f32(int batch, int channels, int height, int width, int kernel_h,
                                int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w,
                                const float *X, float *B, int ldb, hipStream_t stream)
{
    using namespace sgemm;
    const Geometry q = {batch, channels, height, width, 1, kernel_h, kernel_w,
                        stride_h, stride_w, pad_h, pad_w};
    int OH = 0, OW = 0;
    int64_t N = 0;
    const int bad = check_geometry(q, &OH, &OW, &N);
    if (bad != 0) return bad > -5 ? bad : bad + 1;  // no out_channels in this list
    if (N > 0 && (X == nullptr || ((uintptr_t)X & 3u) != 0)) return -11;
    if (N > 0 && (B == nullptr || ((uintptr_t)B & 3u) != 0)) return -12;
    if ((int64_t)ldb < (N > 1 ? N : 1)) return -13;
    if (N == 0) return 0;
    ConvArgs a = {};
    a.X = X;
    a.batch = batch;
    a.C = channels;
    a.H = height;
    a.W = width;
    a.R = kernel_h;
    a.S = kernel_w;
    a.sh = stride_h;
    a.sw = stride_w;
    a.ph = pad_h;
    a.pw = pad_w;
    a.OH = OH;
    a.OW = OW;
    a.K = channels * kernel_h * kernel_w;
    a.N = N;
    const int64_t gx = ceil_div64(N, 1024);
    const int64_t gy = ceil_div64(a.K, kIm2colRows);
    if (gx > INT_MAX || gy > 65535) return (int)hipErrorInvalidConfiguration;
    const int vec = (((uintptr_t)B & 15u) == 0 && ldb % 4 == 0) ? 1 : 0;
    hipLaunchKernelGGL(im2col_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, a,
                       B, (int64_t)ldb, 0, vec);
    return (int)hipGetLastError();
}

extern "C" int sconv2d_plan(int variant, int batch, int channels, int height, int width,
                            int out_channels, int kernel_h, int kernel_w, int stride_h,
                            int stride_w, int pad_h, int pad_w, int num_cus, char *buf, int buflen)
{
    using namespace sgemm;
    if (variant < SCONV_VARIANT_AUTO || variant > SCONV_VARIANT_GENERAL) return SGEMM_ERR_BAD_VARIANT;
    const Geometry q = {batch,    channels, height,   width,    out_channels, kernel_h,
                        kernel_w, stride_h, stride_w, pad_h,    pad_w};
    int OH = 0, OW = 0;
    int64_t N = 0;
    const int bad = check_geometry(q, &OH, &OW, &N);
    if (bad != 0) return bad;
    if (num_cus < 1 || (buf == nullptr && buflen > 0) || buflen < 0) return -12;
    const StemEntry *stem = stem_for(q, OH, OW);
    // Packed output (ldy = N) assumed, as for the call's own size check.
    if (4 * (int64_t)batch * channels * height * width >= (1ll << 32) ||
        4 * (int64_t)out_channels * N >= (1ll << 32))
        stem = nullptr;
    if (variant == SCONV_VARIANT_STEM && stem == nullptr) return SGEMM_ERR_VARIANT_SHAPE;
    char text[200];
    if (out_channels == 0 || N == 0) {
        std::snprintf(text, sizeof text, "none");
    } else if (stem != nullptr && variant != SCONV_VARIANT_GENERAL) {
        const int spi = (int)ceil_div64((int64_t)OH * OW, kStemStrip);
        const int64_t total = (int64_t)spi * batch;
        const int64_t resident = (int64_t)num_cus * stem->wpe;
        std::snprintf(text, sizeof text,
                      "stem mb=%d k=%d window=%dx%dx%d strip=%d strips=%lld grid=%lld oh=%d ow=%d",
                      stem->mb, channels * kernel_h * kernel_w, channels, stem->rows, stem->wpitch,
                      kStemStrip, (long long)total, (long long)(total < resident ? total : resident),
                      OH, OW);
    } else {
        const int64_t tiles = ceil_div64(out_channels, kConvTile) * ceil_div64(N, kConvTile);
        std::snprintf(text, sizeof text, "general tile=%dx%d k=%d grid=%lld oh=%d ow=%d",
                      kConvTile, kConvTile, channels * kernel_h * kernel_w, (long long)tiles, OH,
                      OW);
    }
    if (buflen > 0) {
        std::strncpy(buf, text, (size_t)buflen - 1);
        buf[buflen - 1] = '\0';
    }
    return 0;
}

extern "C" int sconv2d_num_stem_kernels(void) { return sgemm::kNumStems; }
