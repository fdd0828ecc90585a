// libsgemm convolution entry points: argument checks, the choice among the
// stem kernel, the MFMA tile kernels and the general implicit-GEMM kernel,
// and the im2col producer, behind the C ABI declared in include/sconv.h.  Like the GEMM
// entry points, nothing here allocates, frees, copies or synchronises: work
// is queued on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
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
    if ((int64_t)q.H + 2 * (int64_t)q.ph < q.R) return -6;
    if ((int64_t)q.W + 2 * (int64_t)q.pw < q.S) return -7;
    // Padded extents stay in int, so every input coordinate a kernel forms does.
    if ((int64_t)q.H + 2 * (int64_t)q.ph > INT_MAX) return -10;
    if ((int64_t)q.W + 2 * (int64_t)q.pw > INT_MAX) return -11;
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
// output touches.  LDS: 75 KB (7 x 7) and 30 KB (3 x 3).  Workgroups of
// four waves; the last column is the waves per SIMD the register budget is
// set for, i.e. workgroups per CU: two, or three for the 3 x 3 kernel with
// one row block (168 registers; 70.9 -> 68.0 us on the 3 x 3 stem reading
// when it was introduced, and a four-wave budget spills).
const StemEntry kStems[] = {
    SGEMM_STEM(2, 3, 7, 7, 2, 2, 232, 13, 2),
    SGEMM_STEM(1, 3, 7, 7, 2, 2, 232, 13, 2),
    SGEMM_STEM(2, 3, 3, 3, 2, 2, 232, 9, 2),
    SGEMM_STEM(1, 3, 3, 3, 2, 2, 232, 9, 3),
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

// A pointwise layer: 1 x 1 filter, stride 1, no padding (then OH = H, OW = W,
// and image b's im2col matrix is its own C x (H W) block of X).  H W must fit
// the GEMM's int N, which N = batch H W <= INT_MAX already ensures.
bool pointwise(const Geometry &q)
{
    return q.R == 1 && q.S == 1 && q.sh == 1 && q.sw == 1 && q.ph == 0 && q.pw == 0;
}

// The MFMA tile kernels built: tile and waves; all run two waves per SIMD
// (two 4-wave workgroups or one 8-wave workgroup per CU).
struct TileEntry {
    int bm, bn, waves;
    ConvKernelFn fn;
};

#define SGEMM_CONV_TILE(BM, BN, WM, WN) {BM, BN, WM * WN, conv_tile_kernel<BM, BN, WM, WN, 2>}

const TileEntry kTiles[] = {
    SGEMM_CONV_TILE(128, 128, 2, 2),
    SGEMM_CONV_TILE(192, 128, 4, 2),
    SGEMM_CONV_TILE(64, 128, 1, 4),
};

// The direct-to-LDS forms: filter, tile, waves (two waves per SIMD too).
struct DlEntry {
    int R, S, bm, bn, waves;
    ConvKernelFn fn;
};

#define SGEMM_CONV_DL(BM, BN, WM, WN, R, S) \
    {R, S, BM, BN, WM * WN, conv_dl_kernel<BM, BN, WM, WN, 2, R, S>}

const DlEntry kDlTiles[] = {
    SGEMM_CONV_DL(128, 128, 2, 2, 3, 3), SGEMM_CONV_DL(192, 128, 4, 2, 3, 3),
    SGEMM_CONV_DL(64, 128, 1, 4, 3, 3),  SGEMM_CONV_DL(128, 128, 2, 2, 1, 1),
    SGEMM_CONV_DL(192, 128, 4, 2, 1, 1), SGEMM_CONV_DL(64, 128, 1, 4, 1, 1),
};

// The one-tap-per-k-step forms (3 x 3 filters), all at two waves per SIMD:
// four waves with a two-slab ring (70-78 KB of LDS, two workgroups per CU)
// or eight waves with a three-slab ring (145 KB, one per CU).  At equal
// busiest-CU work the earlier entry is taken: (256,43264,1152) runs the
// four-wave 128 x 128 tile (223.4 us; the eight-wave one, three-slab ring,
// 232.5), (384,14161,1152) the 192 x 128 tile (112.6 us; 96 x 128 two per
// CU, 114.2).  The 96-row tile serves M <= 96.
#define SGEMM_CONV_TAP(BM, BN, WM, WN, NB, R, S) \
    {R, S, BM, BN, WM * WN, conv_tap_kernel<BM, BN, WM, WN, 2, R, S, NB>}

const DlEntry kTapTiles[] = {
    SGEMM_CONV_TAP(128, 128, 2, 2, 2, 3, 3),
    SGEMM_CONV_TAP(192, 128, 4, 2, 3, 3, 3),
    SGEMM_CONV_TAP(96, 128, 2, 2, 2, 3, 3),
};

// The general kernel's rate relative to the tile kernels' (measured on the
// 3 x 3 readings: about 0.3 against 0.6 and more of the matrix peak).
constexpr int64_t kGeneralCost = 2;

// Work of the busiest CU, in multiply-adds per tap: ceil(tiles / CUs)
// tiles of bm x bn each (the tiles are spread evenly over the CUs, and
// those sharing a CU share its matrix cores).
int64_t tile_cost(int64_t M, int64_t N, int bm, int bn, int cus)
{
    const int64_t tiles = ceil_div64(M, bm) * ceil_div64(N, bn);
    return ceil_div64(tiles, cus) * bm * bn;
}

// Whether the tile kernels can address the problem: X and the filter rows
// it reads under 2^31 bytes (raw buffer offsets), N short of INT_MAX by a
// tile.
bool tile_fits(const Geometry &q, int64_t N, int ldw)
{
    const int64_t x_bytes = 4 * (int64_t)q.batch * q.C * q.H * q.W;
    const int64_t w_bytes = 4 * ((int64_t)(q.M > 0 ? q.M - 1 : 0) * ldw + (int64_t)q.C * q.R * q.S);
    return x_bytes < (1ll << 31) && w_bytes < (1ll << 31) && N <= INT_MAX - 256;
}

// The tile kernel for this problem, or null for the general kernel: among
// those built, the least busiest-CU work, scaled by the channel padding of
// the tile kernels' 16-channel slabs, against the general kernel's 64 x 64
// tiles at kGeneralCost.
const TileEntry *tile_for(const Geometry &q, int64_t N, int cus)
{
    const int64_t K = (int64_t)q.C * q.R * q.S;
    const int64_t Kpad = (int64_t)((q.C + 15) / 16) * 16 * q.R * q.S;
    const TileEntry *best = nullptr;
    // Compared in units of work * K.
    int64_t best_cost = kGeneralCost * tile_cost(q.M, N, kConvTile, kConvTile, cus) * K;
    for (const TileEntry &e : kTiles) {
        const int64_t c = tile_cost(q.M, N, e.bm, e.bn, cus) * Kpad;
        if (c < best_cost) {
            best = &e;
            best_cost = c;
        }
    }
    return best;
}

// Whether the filter rows are 16-byte aligned (base and row pitch), as the
// direct-to-LDS forms load them.
bool rows_aligned(const float *Wt, int ldw) { return ldw % 4 == 0 && ((uintptr_t)Wt & 15u) == 0; }

// The direct-to-LDS kernel for this problem, or null: the filter must be one
// built, K a multiple of 16, the filter rows 16-byte aligned (w_aligned), and
// the tile kernels' limits hold; among those built, the least busiest-CU work.
const DlEntry *dl_for(const Geometry &q, int64_t N, bool w_aligned, int ldw, int cus)
{
    const int64_t K = (int64_t)q.C * q.R * q.S;
    if (K % 16 != 0 || !w_aligned || !tile_fits(q, N, ldw)) return nullptr;
    const DlEntry *best = nullptr;
    for (const DlEntry &e : kDlTiles) {
        if (e.R != q.R || e.S != q.S) continue;
        if (best == nullptr ||
            tile_cost(q.M, N, e.bm, e.bn, cus) < tile_cost(q.M, N, best->bm, best->bn, cus))
            best = &e;
    }
    return best;
}

// The one-tap-per-k-step kernel for this problem, or null: a filter built,
// C a multiple of 4, the filter rows 16-byte aligned (w_aligned), and the
// tile kernels' limits; among those built, the least busiest-CU work.
const DlEntry *tap_for(const Geometry &q, int64_t N, bool w_aligned, int ldw, int cus)
{
    if (q.C % 4 != 0 || !w_aligned || !tile_fits(q, N, ldw)) return nullptr;
    const DlEntry *best = nullptr;
    for (const DlEntry &e : kTapTiles) {
        if (e.R != q.R || e.S != q.S) continue;
        if (best == nullptr ||
            tile_cost(q.M, N, e.bm, e.bn, cus) < tile_cost(q.M, N, best->bm, best->bn, cus))
            best = &e;
    }
    return best;
}

// The tile kernel with the least busiest-CU work, for the forced tile form.
const TileEntry *tile_forced(const Geometry &q, int64_t N, int cus)
{
    const TileEntry *best = nullptr;
    for (const TileEntry &e : kTiles)
        if (best == nullptr ||
            tile_cost(q.M, N, e.bm, e.bn, cus) < tile_cost(q.M, N, best->bm, best->bn, cus))
            best = &e;
    return best;
}

// Per-device compute-unit count, cached.
constexpr int kConvMaxDevices = 64;
std::atomic<int> g_conv_cus[kConvMaxDevices];

hipError_t conv_device_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int cached =
        dev >= 0 && dev < kConvMaxDevices ? g_conv_cus[dev].load(std::memory_order_relaxed) : 0;
    if (cached > 0) {
        *cus = cached;
        return hipSuccess;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    if (dev >= 0 && dev < kConvMaxDevices) g_conv_cus[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return hipSuccess;
}

int conv_launch(int variant, const Geometry &q, float alpha, const float *X, const float *Wt,
                int ldw, float beta, float *Y, int ldy, hipStream_t stream)
{
    if (variant < SCONV_VARIANT_AUTO || variant > SCONV_VARIANT_TAP) return SGEMM_ERR_BAD_VARIANT;
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
    const bool tile_ok = tile_fits(q, N, ldw);
    if (variant == SCONV_VARIANT_TILE && !tile_ok) return SGEMM_ERR_VARIANT_SHAPE;
    const bool w_aligned = rows_aligned(Wt, ldw);
    if (variant == SCONV_VARIANT_DIRECT && dl_for(q, N, w_aligned, ldw, 1) == nullptr)
        return SGEMM_ERR_VARIANT_SHAPE;
    if (variant == SCONV_VARIANT_TAP && tap_for(q, N, w_aligned, ldw, 1) == nullptr)
        return SGEMM_ERR_VARIANT_SHAPE;
    if (q.M == 0 || N == 0) return 0;

    if (alpha == 0.0f) {
        int64_t blocks = ceil_div64((int64_t)q.M * N, 256);
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(conv_scale_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, Y,
                           (int64_t)ldy, q.M, N, beta);
        return (int)hipGetLastError();
    }

    // A 1 x 1 filter at stride 1 without padding: the taps of image b are
    // its C x (H W) block of X itself, so the convolution is one product
    // per image, Y[:, b H W ..] = Wt X_b, run by the GEMM path on X in place.
    if (variant == SCONV_VARIANT_AUTO && pointwise(q)) {
        const int hw = q.H * q.W;
        for (int b = 0; b < q.batch; ++b) {
            const int rc = sgemm_f32(q.M, hw, q.C, alpha, Wt, ldw, X + (int64_t)b * q.C * hw, hw,
                                     beta, Y + (int64_t)b * hw, ldy, stream);
            if (rc != 0) return rc;
        }
        return 0;
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

    int cus = 0;
    const hipError_t ce = conv_device_cus(&cus);
    if (ce != hipSuccess) return (int)ce;
    if (stem != nullptr && (variant == SCONV_VARIANT_AUTO || variant == SCONV_VARIANT_STEM)) {
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
    const TileEntry *tile = !tile_ok                          ? nullptr
                            : variant == SCONV_VARIANT_TILE ? tile_forced(q, N, cus)
                            : variant == SCONV_VARIANT_AUTO ? tile_for(q, N, cus)
                                                            : nullptr;
    // The direct-to-LDS forms where they apply, in the tile kernels' place:
    // one tap per k-step first, then 16-tap slabs.
    const DlEntry *tap = tap_for(q, N, w_aligned, ldw, cus);
    const DlEntry *dl = variant == SCONV_VARIANT_DIRECT ? dl_for(q, N, w_aligned, ldw, cus)
                        : variant == SCONV_VARIANT_TAP  ? tap
                        : (variant == SCONV_VARIANT_AUTO && tile != nullptr)
                            ? (tap != nullptr ? tap : dl_for(q, N, w_aligned, ldw, cus))
                            : nullptr;
    if (dl != nullptr) {
        const int tiles_m = (int)ceil_div64(q.M, dl->bm);
        const int tiles_n = (int)ceil_div64(N, dl->bn);
        const int64_t blocks = (int64_t)tiles_m * tiles_n;
        if (blocks > INT_MAX) return (int)hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(dl->fn, dim3((unsigned)blocks), dim3(64 * dl->waves), 0, stream, a,
                           tiles_m, tiles_n);
        return (int)hipGetLastError();
    }
    if (tile != nullptr) {
        const int tiles_m = (int)ceil_div64(q.M, tile->bm);
        const int tiles_n = (int)ceil_div64(N, tile->bn);
        const int64_t blocks = (int64_t)tiles_m * tiles_n;
        if (blocks > INT_MAX) return (int)hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(tile->fn, dim3((unsigned)blocks), dim3(64 * tile->waves), 0, stream, a,
                           tiles_m, tiles_n);
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
    if (variant < SCONV_VARIANT_AUTO || variant > SCONV_VARIANT_TAP) return SGEMM_ERR_BAD_VARIANT;
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
    // Packed filters (ldw = K) assumed.
    const bool tile_ok = tile_fits(q, N, channels * kernel_h * kernel_w);
    const TileEntry *tile = !tile_ok                          ? nullptr
                            : variant == SCONV_VARIANT_TILE ? tile_forced(q, N, num_cus)
                            : variant == SCONV_VARIANT_AUTO ? tile_for(q, N, num_cus)
                                                            : nullptr;
    if (variant == SCONV_VARIANT_TILE && tile == nullptr) return SGEMM_ERR_VARIANT_SHAPE;
    // Packed filters (ldw = K) at a 16-byte aligned base assumed.
    const int K = channels * kernel_h * kernel_w;
    const bool w_aligned = K % 4 == 0;
    const DlEntry *tap = tap_for(q, N, w_aligned, K, num_cus);
    const DlEntry *dl = variant == SCONV_VARIANT_DIRECT ? dl_for(q, N, w_aligned, K, num_cus)
                        : variant == SCONV_VARIANT_TAP  ? tap
                        : (variant == SCONV_VARIANT_AUTO && tile != nullptr)
                            ? (tap != nullptr ? tap : dl_for(q, N, w_aligned, K, num_cus))
                            : nullptr;
    if ((variant == SCONV_VARIANT_DIRECT || variant == SCONV_VARIANT_TAP) && dl == nullptr)
        return SGEMM_ERR_VARIANT_SHAPE;
    const bool is_tap = dl != nullptr && dl == tap;
    char text[200];
    if (out_channels == 0 || N == 0) {
        std::snprintf(text, sizeof text, "none");
    } else if (variant == SCONV_VARIANT_AUTO && pointwise(q)) {
        std::snprintf(text, sizeof text, "gemm images=%d m=%d n=%d k=%d oh=%d ow=%d", batch,
                      out_channels, height * width, channels, OH, OW);
    } else if (stem != nullptr && (variant == SCONV_VARIANT_AUTO || variant == SCONV_VARIANT_STEM)) {
        const int spi = (int)ceil_div64((int64_t)OH * OW, kStemStrip);
        const int64_t total = (int64_t)spi * batch;
        const int64_t resident = (int64_t)num_cus * stem->wpe;
        std::snprintf(text, sizeof text,
                      "stem mb=%d k=%d window=%dx%dx%d strip=%d strips=%lld grid=%lld oh=%d ow=%d",
                      stem->mb, channels * kernel_h * kernel_w, channels, stem->rows, stem->wpitch,
                      kStemStrip, (long long)total, (long long)(total < resident ? total : resident),
                      OH, OW);
    } else if (dl != nullptr) {
        const int64_t tiles = ceil_div64(out_channels, dl->bm) * ceil_div64(N, dl->bn);
        std::snprintf(text, sizeof text, "%s bm=%d bn=%d waves=%d k=%d grid=%lld oh=%d ow=%d",
                      is_tap ? "tap" : "direct", dl->bm, dl->bn, dl->waves, K, (long long)tiles,
                      OH, OW);
    } else if (tile != nullptr) {
        const int64_t tiles = ceil_div64(out_channels, tile->bm) * ceil_div64(N, tile->bn);
        std::snprintf(text, sizeof text, "tile bm=%d bn=%d waves=%d k=%d grid=%lld oh=%d ow=%d",
                      tile->bm, tile->bn, tile->waves, channels * kernel_h * kernel_w,
                      (long long)tiles, OH, OW);
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
