// Convolution kernels (gfx950): the im2col producer and two implicit-GEMM
// forms of a 2-D convolution, Y <- alpha * W (*) X + beta * Y.
//
// The UNIVERSAL_SGEMM_CUDA README ("Results" section) times GEMM shapes of
// convolution layers lowered to products: C (M x N) = W (M x K) * B (K x N)
// with K = C*R*S filter taps and N = batch*OH*OW output positions, B being
// the im2col matrix of the input.  These kernels take the input itself:
//
//   X   packed NCHW: X[((b*C + c)*H + ih)*W + iw]
//   W   row m = filter m flattened, tap k = (c*R + r)*S + s at Wt[m*ldw + k]
//   Y   row m = output channel m, column n = (b*OH + oh)*OW + ow, Y[m*ldy + n]
//       (the layout the lowered product writes)
//   tap x(b, c, oh*sh - ph + r, ow*sw - pw + s), zero outside the image
//
// im2col_kernel writes B itself, for the lowered product.  conv_stem_kernel
// and conv_gemm_kernel never form B: they gather the taps of each output
// position from the input as they go.
#pragma once

#include "common.hpp"

namespace sgemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct ConvArgs {
    const float *X;
    const float *Wt;
    float *Y;
    int64_t ldw, ldy;
    int batch, C, H, W;  // input
    int M, R, S;         // output channels, filter rows and columns
    int sh, sw, ph, pw;  // strides and zero padding
    int OH, OW, K;       // output extent, taps per output (C*R*S)
    int64_t N;           // batch * OH * OW
    float alpha, beta;
};

typedef void (*ConvKernelFn)(ConvArgs, int, int);

// ---------------------------------------------------------------- im2col

// Each thread writes columns n0 .. n0+3 of rows k0 .. k0+3 of B (K x N, row
// pitch ldb), non-temporal (B is written once, for a later kernel): its 16
// input loads are all issued before its 4 stores, so each thread keeps 16
// loads in flight.  Rows k0 .. k0+3 are the same for the whole workgroup
// (blockIdx.y); consecutive workgroups write consecutive 4 KB pieces of
// those rows.  vec: B's base is 16-byte aligned and ldb % 4 == 0, so a
// group of four columns is one 128-bit store.
constexpr int kIm2colRows = 4;

__global__ void __launch_bounds__(256) im2col_kernel(ConvArgs a, float *__restrict__ B,
                                                     int64_t ldb, int, int vec)
{
    const float *__restrict__ X = a.X;
    const int64_t n0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (n0 >= a.N) return;
    const int k0 = blockIdx.y * kIm2colRows;
    const int ohw = a.OH * a.OW;
    int ihb[4], iwb[4];
    int64_t xb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int64_t n = n0 + q;
        if (n >= a.N) n = a.N - 1;
        const int b = (int)(n / ohw);
        const int p = (int)(n - (int64_t)b * ohw);
        const int oh = p / a.OW, ow = p - oh * a.OW;
        ihb[q] = oh * a.sh - a.ph;
        iwb[q] = ow * a.sw - a.pw;
        xb[q] = (int64_t)b * a.C * a.H * a.W;
    }
    f32x4 v[kIm2colRows];
#pragma unroll
    for (int kk = 0; kk < kIm2colRows; ++kk) {
        const int k = k0 + kk < a.K ? k0 + kk : a.K - 1;
        const int c = k / (a.R * a.S), r = (k / a.S) % a.R, s = k % a.S;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ih = ihb[q] + r, iw = iwb[q] + s;
            v[kk][q] = (ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
                           ? X[xb[q] + ((int64_t)c * a.H + ih) * a.W + iw]
                           : 0.f;
        }
    }
#pragma unroll
    for (int kk = 0; kk < kIm2colRows; ++kk) {
        if (k0 + kk >= a.K) break;
        float *dst = B + (int64_t)(k0 + kk) * ldb + n0;
        if (vec && n0 + 3 < a.N) {
            __builtin_nontemporal_store(v[kk], reinterpret_cast<f32x4 *>(dst));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (n0 + q < a.N) __builtin_nontemporal_store(v[kk][q], dst + q);
        }
    }
}

// ------------------------------------------------- implicit GEMM, any shape

// One 64 x 64 tile of Y per workgroup (4 waves, each a 32 x 32 block of
// v_mfma_f32_32x32x2_f32), K in slabs of 16 taps: every thread fetches 4
// weights and gathers 4 taps of its output column into registers, they go
// to LDS, and each wave runs 8 MFMAs.  Taps outside the image, rows past M,
// columns past N and taps past K are zeros.  This is the form for any
// geometry; the stem kernel below is the fast one.
//
// MFMA layout (v_mfma_f32_32x32x2_f32, lane l, h = l / 32): A operand
// A[l % 32][k = h], B operand B[k = h][l % 32],
// D[8 (i / 4) + 4 h + i % 4][l % 32] for accumulator element i.
constexpr int kConvTile = 64;

__global__ void __launch_bounds__(256) conv_gemm_kernel(ConvArgs a, int tiles_m, int)
{
    __shared__ float As[16][kConvTile + 4];  // [k][m]
    __shared__ float Bs[16][kConvTile + 4];  // [k][n]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, j = lane & 31;
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int m0 = tm * kConvTile;
    const int64_t n0 = (int64_t)tn * kConvTile;

    // This thread's output column for the B gather, fixed for the tile.
    const int bn = tid & 63, bk = tid >> 6;  // k rows bk, bk + 4, bk + 8, bk + 12
    const int64_t n = n0 + bn;
    const bool n_ok = n < a.N;
    const int ohw = a.OH * a.OW;
    int ih0 = 0, iw0 = 0;
    int64_t xb = 0;
    if (n_ok) {
        const int b = (int)(n / ohw);
        const int p = (int)(n - (int64_t)b * ohw);
        const int oh = p / a.OW, ow = p - oh * a.OW;
        ih0 = oh * a.sh - a.ph;
        iw0 = ow * a.sw - a.pw;
        xb = (int64_t)b * a.C * a.H * a.W;
    }
    // This thread's weights: row am, k columns ak .. ak + 3.
    const int am = tid >> 2, ak = 4 * (tid & 3);

    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;

    for (int k0 = 0; k0 < a.K; k0 += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = k0 + ak + q;
            av[q] = (m0 + am < a.M && k < a.K) ? a.Wt[(int64_t)(m0 + am) * a.ldw + k] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = k0 + bk + 4 * q;
            float v = 0.f;
            if (n_ok && k < a.K) {
                const int c = k / (a.R * a.S), r = (k / a.S) % a.R, s = k % a.S;
                const int ih = ih0 + r, iw = iw0 + s;
                if (ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
                    v = a.X[xb + ((int64_t)c * a.H + ih) * a.W + iw];
            }
            bv[q] = v;
        }
        __syncthreads();  // the previous slab's MFMAs have read the LDS
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            As[ak + q][am] = av[q];
            Bs[bk + 4 * q][bn] = bv[q];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 8; ++t)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[2 * t + h][wm * 32 + j],
                                                       Bs[2 * t + h][wn * 32 + j], acc, 0, 0, 0);
    }

    const int64_t col = n0 + wn * 32 + j;
    if (col >= a.N) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = m0 + wm * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (row >= a.M) continue;
        float *py = a.Y + (int64_t)row * a.ldy + col;
        float v = a.alpha * acc[i];
        if (a.beta != 0.f) v = fmaf(a.beta, *py, v);
        *py = v;
    }
}

// ------------------------------------------------------ stem fast path

// For the first layers of image networks: few input channels, a large
// image, M <= 32 MB output channels (the two stem readings of the skinny
// convolution-as-GEMM shapes: 3 channels, 7 x 7 stride 2 pad 3 or 3 x 3
// stride 2 pad 1, on 224 x 224 images).
//
// Output positions are cut into strips of 256 consecutive positions of one
// image.  Resident workgroups take contiguous ranges of strips.  For each
// strip the workgroup copies the input rows the strip touches -- every
// channel, ROWS rows, WPITCH columns with the image at column COL0 and
// zeros around it -- into an LDS window once; then each of its four waves
// computes M x 64 outputs (MB x 2 blocks of v_mfma_f32_32x32x2_f32), taking
// the B operand of every MFMA straight from the window.  The next strip's
// window is fetched into registers before the strip's MFMAs and written to
// LDS after them, so its latency is hidden behind the matrix work.
//
// Taps are paired: the MFMA's two k values are taps f = 2t and 2t + 1, one
// per half-wave.  In the window, tap f of output position q sits at
//   q's base + koff(f),   koff(f) = (c ROWS + r) WPITCH + s,
//   q's base = (oh - oh_lo) SH WPITCH + ow SW - pw + COL0,
// so with the geometry fixed at compile time koff(2t) is an immediate
// offset of the LDS read, and the upper half-wave's extra koff(2t+1) -
// koff(2t) is one of three constants (same row, next row, next channel),
// folded into per-lane base registers.  An odd last tap reads a zero slot.
// The loop over taps has no address arithmetic at all.
//
// The weights sit in LDS split by half-wave, As[h][row][t] = Wt[row][2t + h]
// (zero past M and K), row pitch TP (TP / 4 odd), so one 128-bit read feeds
// four tap pairs.
template <int CH, int R, int S, int WPITCH, int ROWS>
struct StemGeom {
    static constexpr int K = CH * R * S;
    static constexpr int KP = (K + 1) / 2;  // tap pairs
    static constexpr int WIN = CH * ROWS * WPITCH;
    static constexpr int ZERO = WIN;        // four zero floats after the window
    static constexpr int D_ROW = 1;
    static constexpr int D_NEXT_ROW = WPITCH - (S - 1);
    static constexpr int D_NEXT_CH = (ROWS - R + 1) * WPITCH - (S - 1);
    static constexpr int TP = ((KP + 3) / 4 * 4) / 4 % 2 == 1 ? (KP + 3) / 4 * 4
                                                              : (KP + 3) / 4 * 4 + 4;
    __host__ __device__ static constexpr int koff(int f)
    {
        return ((f / (R * S)) * ROWS + (f / S) % R) * WPITCH + f % S;
    }
    // 0: taps 2t and 2t+1 in one row; 1: 2t+1 starts the next row; 2: it
    // starts the next channel; 3: there is no tap 2t+1 (odd K).
    __host__ __device__ static constexpr int kind(int t)
    {
        return 2 * t + 1 >= K ? 3 : (2 * t + 1) % S != 0 ? 0 : (2 * t + 1) % (R * S) != 0 ? 1 : 2;
    }
};

constexpr int kStemStrip = 256;  // output positions per strip (4 waves x 64)
constexpr int kStemCol0 = 4;     // window column of input column 0 (>= pw)

template <int MB, int CH, int R, int S, int SH, int SW, int WPITCH, int ROWS, int WPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
conv_stem_kernel(ConvArgs a, int strips_per_image, int total_strips)
{
    using G = StemGeom<CH, R, S, WPITCH, ROWS>;
    constexpr int KP = G::KP, TP = G::TP;
    constexpr int G4 = WPITCH / 4;                          // 16-byte groups per window row
    constexpr int NST = (CH * ROWS * G4 + 255) / 256;       // groups staged per thread
    static_assert(WPITCH % 4 == 0, "window rows must be 16-byte multiples");
    static_assert(G::WIN * 4 + 16 < 65536, "LDS offsets must fit the immediate field");
    __shared__ __attribute__((aligned(16))) float As[2 * 32 * MB * TP];
    __shared__ __attribute__((aligned(16))) float win[G::WIN + 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, j = lane & 31;

    for (int e = tid; e < 2 * 32 * MB * TP; e += 256) {
        const int hh = e / (32 * MB * TP), rem = e % (32 * MB * TP);
        const int row = rem / TP, t = rem % TP, f = 2 * t + hh;
        As[e] = (row < a.M && f < G::K) ? a.Wt[(int64_t)row * a.ldw + f] : 0.f;
    }
    if (tid < 4) win[G::ZERO + tid] = 0.f;

    const int ohw = a.OH * a.OW;
    const bool vec_x = ((reinterpret_cast<uintptr_t>(a.X) & 15u) == 0) && (a.W % 4 == 0);
    // Two adjacent positions per lane can be one 64-bit store.
    const bool vec_y = ((reinterpret_cast<uintptr_t>(a.Y) & 7u) == 0) && (a.ldy % 2 == 0) &&
                       (ohw % 2 == 0);
    const int64_t s0 = (int64_t)blockIdx.x * total_strips / gridDim.x;
    const int64_t s1 = (int64_t)(blockIdx.x + 1) * total_strips / gridDim.x;
    const float *a_lane = As + (h * 32 * MB + j) * TP;

    // The window of strip st, fetched into registers: this thread's groups
    // e = tid + 256 i of the CH * ROWS rows of G4 16-byte groups.
    // Input loads and output stores address the kernel argument's base with
    // 32-bit byte offsets (the host takes this kernel only for inputs and
    // outputs below 4 GiB), which keeps 64-bit address arithmetic out of the
    // registers the tap loop needs.
    //
    // The window of strip st is fetched into registers (this thread's
    // 16-byte groups e = tid + 256 i of the CH * ROWS rows of G4 groups)
    // before the strip's MFMAs and written to LDS after them.  The loads
    // are unconditional, from a clamped address where the data lie outside
    // the image, and which of them hold data is kept as bits of one
    // register: a lane-dependent branch around a load would keep its
    // execution mask alive across the MFMA loop.
    const char *xbase = reinterpret_cast<const char *>(a.X);
    char *ybase = reinterpret_cast<char *>(a.Y);
    // A thread's groups keep their channel, window row and columns from strip
    // to strip: their byte offsets from the strip's first window row, and
    // which of their elements fall inside the image's columns, are worked
    // out once.
    uint32_t goff[NST];
    uint64_t col_ok = 0;  // bit 4 i + q: element q of group i is an image column
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int e = tid + 256 * i;
        const int rowid = e / G4, g = e - rowid * G4;
        const int c = rowid / ROWS, rr = rowid % ROWS;
        const int iw0 = 4 * g - kStemCol0;
        goff[i] = (uint32_t)((c * a.H + rr) * a.W + iw0) * 4u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = e < CH * ROWS * G4 && iw0 + q >= 0 && iw0 + q < a.W &&
                            (vec_x ? iw0 >= 0 && iw0 + 3 < a.W : true);
            col_ok |= (ok ? 1ull : 0ull) << (4 * i + q);
        }
    }
    f32x4 pre[NST];
    uint64_t valid = 0;  // col_ok and the group's row inside the image
    auto fetch = [&](int64_t st) {
        const int b = (int)(st / strips_per_image);
        const int p0 = (int)(st - (int64_t)b * strips_per_image) * kStemStrip;
        const int ih_lo = (p0 / a.OW) * SH - a.ph;
        // Byte offset of (image b, channel 0, row ih_lo, column 0); may
        // wrap when ih_lo < 0, where only rows inside the image are read.
        const uint32_t sbase = (uint32_t)((b * a.C * a.H + ih_lo) * a.W) * 4u;
        valid = 0;
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int rr = ((tid + 256 * i) / G4) % ROWS;
            const bool row_ok = (unsigned)(ih_lo + rr) < (unsigned)a.H;
            const uint64_t ok4 = row_ok ? (col_ok >> (4 * i)) & 15ull : 0ull;
            valid |= ok4 << (4 * i);
            if (vec_x) {
                pre[i] = *reinterpret_cast<const f32x4 *>(xbase + (ok4 ? sbase + goff[i] : 0u));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    pre[i][q] = *reinterpret_cast<const float *>(
                        xbase + ((ok4 >> q) & 1 ? sbase + goff[i] + 4u * q : 0u));
            }
        }
    };
    auto place = [&]() {
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int e = tid + 256 * i;
            if (e < CH * ROWS * G4) {
                f32x4 v;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[q] = (valid >> (4 * i + q)) & 1 ? pre[i][q] : 0.f;
                *reinterpret_cast<f32x4 *>(win + 4 * e) = v;
            }
        }
    };

    if (s0 < s1) {
        fetch(s0);
        place();
    }
    __syncthreads();  // the weights and the first window are in LDS
    for (int64_t st = s0; st < s1; ++st) {
        const int b = (int)(st / strips_per_image);
        const int p0 = (int)(st - (int64_t)b * strips_per_image) * kStemStrip;
        const int oh_lo = p0 / a.OW;
        // The next strip's window travels while this one is computed.
        if (st + 1 < s1) fetch(st + 1);

        // Per-lane window bases.  Lane j of a wave holds positions 2j and
        // 2j + 1 of the wave's 64 (column blocks cb = 0, 1 interleaved), so its
        // two outputs of a row are adjacent.  Positions past the image clamp
        // to its last one; their outputs are not stored.
        int base[2][4];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            int q = p0 + wave * 64 + 2 * j + cb;
            q = q < ohw ? q : ohw - 1;
            const int oh = q / a.OW, ow = q - oh * a.OW;
            const int pb = (oh - oh_lo) * SH * WPITCH + ow * SW - a.pw + kStemCol0;
            base[cb][0] = pb + h * G::D_ROW;
            base[cb][1] = pb + h * G::D_NEXT_ROW;
            base[cb][2] = pb + h * G::D_NEXT_CH;
            base[cb][3] = h ? G::ZERO - G::koff(2 * (KP - 1)) : pb;
        }

        f32x16 acc[MB][2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mb][cb][i] = 0.f;

        f32x4 a4[MB];
#pragma unroll
        for (int t = 0; t < KP; ++t) {
            if (t % 4 == 0) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    a4[mb] = *reinterpret_cast<const f32x4 *>(a_lane + mb * 32 * TP + t);
            }
            float bv[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) bv[cb] = win[base[cb][G::kind(t)] + G::koff(2 * t)];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[mb][t % 4], bv[cb],
                                                                       acc[mb][cb], 0, 0, 0);
        }

        // Epilogue: a half-wave writes 64 consecutive positions of a row of
        // Y, two per lane.
        const float alpha = a.alpha, beta = a.beta;
        const int q0 = p0 + wave * 64 + 2 * j;
        const uint32_t n0 = (uint32_t)(b * ohw + q0);
        const uint32_t ldy = (uint32_t)a.ldy;
        const bool both = q0 + 1 < ohw;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = mb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                if (row >= a.M || q0 >= ohw) continue;
                float *py = reinterpret_cast<float *>(ybase + ((uint32_t)row * ldy + n0) * 4u);
                float v0 = alpha * acc[mb][0][i], v1 = alpha * acc[mb][1][i];
                if (vec_y && both) {
                    f32x2 v = {v0, v1};
                    if (beta != 0.f) v += beta * *reinterpret_cast<const f32x2 *>(py);
                    __builtin_nontemporal_store(v, reinterpret_cast<f32x2 *>(py));
                } else {
                    if (beta != 0.f) v0 = fmaf(beta, py[0], v0);
                    __builtin_nontemporal_store(v0, py);
                    if (both) {
                        if (beta != 0.f) v1 = fmaf(beta, py[1], v1);
                        __builtin_nontemporal_store(v1, py + 1);
                    }
                }
            }

        __syncthreads();  // every wave is done with this window
        if (st + 1 < s1) place();
        __syncthreads();
    }
}

// Scale Y's M x N window by beta (alpha == 0): beta == 0 writes zeros.
__global__ void __launch_bounds__(256) conv_scale_kernel(float *Y, int64_t ldy, int M, int64_t N,
                                                         float beta)
{
    const int64_t total = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / N;
        float *p = Y + r * ldy + (idx - r * N);
        *p = (beta == 0.f) ? 0.f : beta * *p;
    }
}

}  // namespace sgemm
