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
#include "mfma_dl.hpp"

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

// ------------------------------------------------ implicit GEMM, MFMA tiles

// One BM x BN tile of Y per workgroup, for any filter, channel count,
// stride and padding: the shape of an image network's middle layers (many
// channels, small filters), where the contraction K = C R S is long and the
// work is dense.  The matrix-core pipeline is that of the GEMM tile kernel:
// slabs of 16 taps, v_mfma_f32_16x16x4_f32, a wave per (BM / WM) x (BN / WN)
// sub-tile, three LDS buffers per operand with the registers holding the
// slab after next's loads, one barrier per slab.
//
// The order of the contraction is changed (a sum may take its terms in any
// order): slab t covers filter tap (r, s) = rs(t) and channels
// 16 cb .. 16 cb + 15, with cb = t / RS, rs = t % RS (channels past C are
// zeros).  A slab's tap is then the same for every element of it, so:
//   - a tap of output position n in channel c is X at
//     base(n) + c H W + r W + s, base(n) the input offset of (b, 0, oh sh -
//     ph, ow sw - pw): a per-thread part (base(n) + r W + s, worked out once
//     per slab) plus a wave-uniform part (c H W), which is what a raw buffer
//     load takes as its vector and scalar offsets;
//   - a tap outside the image (or past N) gets a vector offset beyond the
//     buffer's size, for which the hardware returns zero: no select after
//     the load, so nothing waits for it before it is stored to LDS;
//   - the filter element (m, c, r, s) is Wt at m ldw + c RS + rs: a
//     per-thread offset (row and channel in the slab) plus a wave-uniform
//     one (16 cb RS + rs).
// Consecutive slabs walk the taps of one block of channels, so they read
// the same lines of X and Wt.  Rows past M, positions past N and channels
// past C are zeros; the epilogue writes alpha acc + beta Y (Y not read when
// beta == 0) inside the window.  X and Wt must each be under 2^31 bytes.
//
// Thread roles per slab: B element (kk, col) with col = tid % BN and
// kk = tid / BN + (NT / BN) i (kk, hence the channel, is the same for all
// lanes of a wave); A element (m, kk) with kk = tid % 16 and
// m = tid / 16 + (NT / 16) j.
//
// MFMA operand layout as in the GEMM tile kernel (lane l: A[l % 16][k],
// B[k][l % 16] with k = 4 (l / 16) + step; D[4 (l / 16) + i][l % 16]).
// LDS: A m-major with pitch 24 floats, B k-major with pitch BN + 4.
template <int BM, int BN, int WM, int WN>
struct ConvTile {
    static constexpr int NT = WM * WN * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int BK = 16;
    static constexpr int SA = BK + 8, SB = BN + 4;
    static constexpr int NA = BM * BK / NT;  // filter elements per thread per slab
    static constexpr int NB = BK * BN / NT;  // taps per thread per slab
    static constexpr int LDS_A = BM * SA, LDS_B = BK * SB;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BN % 64 == 0 && NT % BN == 0 && NB >= 1, "a wave's taps share one channel");
    static_assert(NT % BK == 0 && (BM * BK) % NT == 0, "filter slab splits evenly");
};

// Buffer descriptor word 3 for raw 32-bit loads (data format 32).
constexpr int kBufferWord3 = 0x00020000;
// A vector offset no buffer here reaches (buffers are under 2^31 bytes):
// loads through it return zero.
constexpr uint32_t kOffsetOut = 0x80000000u;

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff)
{
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

template <int BM, int BN, int WM, int WN, int WPE>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
conv_tile_kernel(ConvArgs a, int tiles_m, int tiles_n)
{
    using T = ConvTile<BM, BN, WM, WN>;
    constexpr int NT = T::NT, TM = T::TM, TN = T::TN, FM = T::FM, FN = T::FN;
    constexpr int BK = T::BK, SA = T::SA, SB = T::SB, NA = T::NA, NB = T::NB;
    __shared__ __attribute__((aligned(16))) float As[3 * T::LDS_A];
    __shared__ __attribute__((aligned(16))) float Bs[3 * T::LDS_B];

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tiles_m, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int M = a.M, N = (int)a.N, C = a.C, S = a.S;
    const int RS = a.R * a.S;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int wr = wave / WN, wc = wave % WN;
    const int lm = lane & 15, lg = lane >> 4;

    const uint32_t x_bytes = 4u * (uint32_t)a.batch * (uint32_t)C * (uint32_t)a.H * (uint32_t)a.W;
    const uint32_t w_bytes = 4u * ((uint32_t)(M - 1) * (uint32_t)a.ldw + (uint32_t)a.K);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.X), 0, (int)x_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wr_ =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.Wt), 0, (int)w_bytes, kBufferWord3);

    // Filter elements: channel akk of the slab, rows am0 + (NT / 16) j.
    const int akk = tid % BK, am0 = tid / BK;
    uint32_t a_off[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int m = m0 + am0 + (NT / BK) * j;
        a_off[j] = m < M ? 4u * ((uint32_t)m * (uint32_t)a.ldw + (uint32_t)akk * (uint32_t)RS)
                         : kOffsetOut;
    }

    // Taps: this thread's output position, fixed for the tile.
    const int col = tid % BN;
    const int krow = wave_s * 64 / BN;  // first slab row of this wave; then + NT / BN
    const int n = n0 + col;
    const bool n_ok = n < N;
    int ih0 = 0, iw0 = 0;
    uint32_t pbase = 0;  // element offset of (b, 0, ih0, iw0), modulo 2^32
    if (n_ok) {
        const int ohw = a.OH * a.OW;
        const int b = n / ohw;
        const int p = n - b * ohw;
        const int oh = p / a.OW, ow = p - oh * a.OW;
        ih0 = oh * a.sh - a.ph;
        iw0 = ow * a.sw - a.pw;
        pbase = ((uint32_t)(b * C * a.H) + (uint32_t)ih0) * (uint32_t)a.W + (uint32_t)iw0;
    }
    const uint32_t hw4 = 4u * (uint32_t)a.H * (uint32_t)a.W;

    float ra[NA], rb[NB];
    // Slab t: channel block cb, filter tap (r, s) (wave-uniform).
    auto fetch = [&](int cb, int r, int s) {
        const int rs = r * S + s;
        const int c0 = cb * BK;
        const uint32_t a_soff = 4u * ((uint32_t)c0 * (uint32_t)RS + (uint32_t)rs);
        const bool a_c_ok = c0 + akk < C;
#pragma unroll
        for (int j = 0; j < NA; ++j)
            ra[j] = buffer_load_f32(wr_, a_c_ok ? a_off[j] : kOffsetOut, a_soff);
        const bool tap_in = n_ok && (unsigned)(ih0 + r) < (unsigned)a.H &&
                            (unsigned)(iw0 + s) < (unsigned)a.W;
        const uint32_t b_voff =
            tap_in ? 4u * (pbase + (uint32_t)r * (uint32_t)a.W + (uint32_t)s) : kOffsetOut;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int c = c0 + krow + (NT / BN) * i;  // wave-uniform
            const bool c_ok = c < C;
            rb[i] = buffer_load_f32(xr, c_ok ? b_voff : kOffsetOut, c_ok ? (uint32_t)c * hw4 : 0u);
        }
    };
    auto stash = [&](int buf) {
        float *as = As + buf * T::LDS_A;
        float *bs = Bs + buf * T::LDS_B;
#pragma unroll
        for (int j = 0; j < NA; ++j) as[(am0 + (NT / BK) * j) * SA + akk] = ra[j];
#pragma unroll
        for (int i = 0; i < NB; ++i) bs[(krow + (NT / BN) * i) * SB + col] = rb[i];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int a_frag = (wr * TM + lm) * SA + 4 * lg;
    const int b_frag = (4 * lg) * SB + wc * TN + lm;
    // The slab's 4 k-steps; hook() runs before k-step 1 (the next slab's
    // registers go to LDS there, behind MFMAs in flight).
    auto compute = [&](int buf, auto hook) {
        const float *as = As + buf * T::LDS_A + a_frag;
        const float *bs = Bs + buf * T::LDS_B + b_frag;
        f32x4 af[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            af[fm] = *reinterpret_cast<const f32x4 *>(as + fm * 16 * SA);
        float bf[4][FN];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) bf[s][fn] = bs[s * SB + fn * 16];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s == 1) hook();
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[fm][s], bf[s][fn],
                                                                       acc[fm][fn], 0, 0, 0);
        }
    };

    // Slab t is read from buffer t % 3.  The registers hold slab t + 1
    // while slab t runs; they go to buffer (t + 1) % 3 inside slab t's MFMAs
    // and are refilled with slab t + 2.  That buffer was last read in slab
    // t - 2, which every wave left before the barrier that ended it.
    const int nslab = ((C + BK - 1) / BK) * RS;
    int f_cb = 0, f_r = 0, f_s = 0;  // the next slab to fetch
    auto advance = [&] {
        if (++f_s == S) {
            f_s = 0;
            if (++f_r == a.R) {
                f_r = 0;
                ++f_cb;
            }
        }
    };
    fetch(f_cb, f_r, f_s);
    advance();
    stash(0);
    if (nslab > 1) {
        fetch(f_cb, f_r, f_s);
        advance();
    }
    __syncthreads();
    int cur = 0;
    for (int t = 0; t < nslab; ++t) {
        const int nxt = cur == 2 ? 0 : cur + 1;
        const bool more = t + 1 < nslab;
        const bool more2 = t + 2 < nslab;
        compute(cur, [&] {
            if (more) {
                stash(nxt);
                if (more2) {
                    fetch(f_cb, f_r, f_s);
                    advance();
                }
            }
        });
        __syncthreads();
        cur = nxt;
    }

    const float alpha = a.alpha, beta = a.beta;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wr * TM + fm * 16 + 4 * lg + i;
            if (row >= M) continue;
            float *yrow = a.Y + (int64_t)row * a.ldy;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int c = n0 + wc * TN + fn * 16 + lm;
                if (c < N) {
                    float v = alpha * acc[fm][fn][i];
                    if (beta != 0.f) v = fmaf(beta, yrow[c], v);
                    yrow[c] = v;
                }
            }
        }
    }
}

// ------------------------------------ implicit GEMM, direct-to-LDS slabs

// The fast form of the tile kernel above for R x S filters it is built for
// (R and S compile-time), K = C R S a multiple of 16 and filter rows 16-byte
// aligned: no register holds slab data.  Both operands travel from memory
// straight into LDS with raw buffer loads in LDS mode (each lane's data lands
// at a wave-uniform LDS address + its lane offset), in the slab pipeline of
// the GEMM direct-load kernel: a ring of three buffers, the loads of slab
// t + 2 spread over k-steps 0-1 of slab t, one wait and barrier, then the
// next slab's operand reads spread over k-steps 2-3.  The contraction is in
// the natural order k = (c R + r) S + s.
//
//   filters: chunk cm of a slab (rows 16 cm .. 16 cm + 15) is one 16-byte
//     load per lane, lane l taking Wt[m0 + 16 cm + l % 16][k0 + 4 (l / 16)
//     .. + 3] to LDS slot l (the operand read of block cm is then slot l);
//     rows past M get an out-of-range offset, so they land as zeros.
//   taps: one load of a wave covers one slab row k (tap (c, r, s), the same
//     for the wave) and 64 consecutive output positions (the lane's
//     position fixed for the tile): vector offset base(n) + r W + s, or an
//     out-of-range offset for a tap outside the image (or past N), which
//     lands as zero; scalar offset c H W.  B is k-major in LDS with row
//     pitch BN + 4: a load writes 64 consecutive floats of one row, and the
//     operand reads (lane group g reading row 4 g + s) fall in distinct
//     banks.
template <int BM, int BN, int WM, int WN, int R, int S>
struct ConvDl {
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int CA = BM / 16;            // filter chunks per slab
    static constexpr int BH = BN / 64;            // 64-position pieces of a tap row
    static constexpr int SB = BN + 4;             // tap row pitch in LDS (floats)
    static constexpr int A_FLOATS = CA * 256;
    static constexpr int BUF = A_FLOATS + 16 * SB;  // floats per ring buffer
    static constexpr int NBUF = 3;
    static constexpr int LDS = NBUF * BUF;
    static constexpr int LA = CA / NW;            // filter loads per wave per slab,
    static constexpr int XA = CA % NW;            // and one more for waves 0 .. XA-1
    static constexpr int LB = 16 * BH / NW;       // tap loads per wave per slab
    static constexpr int L = LA + LB;
    static constexpr int LMAX = L + (XA > 0 ? 1 : 0);
    static constexpr int NREAD = FM + 2 * FN;     // operand reads per slab
    static constexpr int STRIDE = 2 * FM * FN / (LMAX + 1);
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BN % 64 == 0 && (16 * BH) % NW == 0 && NW % BH == 0,
                  "each wave loads whole tap rows of one 64-position piece");
    static_assert(STRIDE >= 1 && NREAD <= 2 * FM * FN, "too few MFMAs per slab");
    static_assert(LMAX * (NBUF - 1) <= 63, "loads in flight must fit the vmcnt field");
    static_assert(R * S <= 32, "tap mask is 32 bits");
};

template <int BM, int BN, int WM, int WN, int WPE, int R, int S>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
conv_dl_kernel(ConvArgs a, int tiles_m, int tiles_n)
{
    using D = ConvDl<BM, BN, WM, WN, R, S>;
    constexpr int NW = D::NW, TM = D::TM, TN = D::TN, FM = D::FM, FN = D::FN;
    constexpr int BH = D::BH, SB = D::SB, BUF = D::BUF, NBUF = D::NBUF;
    constexpr int LA = D::LA, XA = D::XA, LB = D::LB, L = D::L, LMAX = D::LMAX;
    constexpr int NREAD = D::NREAD, S1 = D::STRIDE;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS];

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tiles_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = a.M, N = (int)a.N;
    const int nslab = a.K / 16;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN, wc = wave % WN;
    const bool extra = XA > 0 && wave < XA;

    const uint32_t x_bytes = 4u * (uint32_t)a.batch * (uint32_t)a.C * (uint32_t)a.H * (uint32_t)a.W;
    const uint32_t w_bytes = 4u * ((uint32_t)(M - 1) * (uint32_t)a.ldw + (uint32_t)a.K);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.X), 0, (int)x_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.Wt), 0, (int)w_bytes, kBufferWord3);

    // Filter loads: load q (< LA, or LA for the extra waves) of this wave
    // fills chunk wave + q NW.
    uint32_t a_voff[LA + 1];
#pragma unroll
    for (int q = 0; q <= LA; ++q) {
        const int cm = wave + q * NW;
        const int row = m0 + 16 * cm + (lane & 15);
        a_voff[q] = row < M ? 4u * ((uint32_t)row * (uint32_t)a.ldw + 4u * (uint32_t)(lane >> 4))
                            : kOffsetOut;
    }
    // Tap loads: this wave's 64-position piece h (fixed) and, for load q,
    // slab row wave / BH + (NW / BH) q.
    const int h = wave % BH;
    const int n = n0 + 64 * h + lane;
    uint32_t pbase4 = 0, tap_ok = 0;
    if (n < N) {
        const int ohw = a.OH * a.OW;
        const int b = n / ohw;
        const int p = n - b * ohw;
        const int oh = p / a.OW, ow = p - oh * a.OW;
        const int ih0 = oh * a.sh - a.ph, iw0 = ow * a.sw - a.pw;
        pbase4 = 4u * (((uint32_t)(b * a.C * a.H) + (uint32_t)ih0) * (uint32_t)a.W + (uint32_t)iw0);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int s = 0; s < S; ++s)
                if ((unsigned)(ih0 + r) < (unsigned)a.H && (unsigned)(iw0 + s) < (unsigned)a.W)
                    tap_ok |= 1u << (r * S + s);
    }
    const uint32_t hw4 = 4u * (uint32_t)a.H * (uint32_t)a.W;
    const uint32_t w4 = 4u * (uint32_t)a.W;

    // Load q of slab ks (k0 = 16 ks) into ring buffer buf.
    auto load = [&](int q, int ks, int buf) {
        float *base = lds + buf * BUF;
        const int k0 = 16 * ks;
        if (q >= LA && q < L) {
            const int kk = wave / BH + (NW / BH) * (q - LA);
            const int k = k0 + kk;  // wave-uniform
            const int c = k / (R * S);
            const int rs = k - c * (R * S);
            const int r = rs / S, s = rs - r * S;
            const uint32_t voff = ((tap_ok >> rs) & 1u)
                                      ? pbase4 + (uint32_t)r * w4 + 4u * (uint32_t)s
                                      : kOffsetOut;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (lds_float *)(base + D::A_FLOATS + kk * SB + 64 * h), 4, (int)voff,
                (int)((uint32_t)c * hw4), 0, 0);
        } else {
            const int qa = q < LA ? q : LA;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wrs, (lds_float *)(base + (wave + qa * NW) * 256), 16, (int)a_voff[qa],
                4 * k0, 0, 0);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    f32x4 afs[2][FM];
    float bfs[2][4][FN];
    const int lg = lane >> 4, lm = lane & 15;
    const int b_lane = D::A_FLOATS + 4 * lg * SB + wc * TN + lm;
    // Operand read r (0 .. NREAD-1) of the slab in buffer buf, in order of
    // first use: filter blocks, then tap k-steps 0-1, then 2-3.
    auto read_op = [&](int r, int buf, f32x4 (&af)[FM], float (&bf)[4][FN]) {
        const float *base = lds + buf * BUF;
        if (r < FM) {
            af[r] = *reinterpret_cast<const f32x4 *>(base + (wr * FM + r) * 256 + 4 * lane);
        } else {
            const int hh = (r - FM) / FN, fn = (r - FM) % FN;
            const float *bs = base + b_lane + 2 * hh * SB + 16 * fn;
            bf[2 * hh][fn] = bs[0];
            bf[2 * hh + 1][fn] = bs[SB];
        }
    };
    auto ksteps = [&](int s0, int s1, const f32x4 (&af)[FM], const float (&bf)[4][FN],
                      auto hook) {
#pragma unroll
        for (int s = s0; s < s1; ++s)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    hook(((s - s0) * FM + fm) * FN + fn);
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[fm][s], bf[s][fn],
                                                                       acc[fm][fn], 0, 0, 0);
                }
    };

    // Slab t from buffer buf with operands in set P; slab t+1's operands go
    // to set P ^ 1.  After the last slab the reads fetch a stale buffer (in
    // bounds; the values go unused).
    auto slab = [&](auto P, int t, int buf) {
        constexpr int p = decltype(P)::value;
        // The loads of slab t + 2 go to the buffer slab t - 1 used (every
        // wave's reads of it had returned at barrier t - 1).
        const bool more = t >= 1 && t + NBUF - 1 < nslab;
        const int lb = buf == 0 ? NBUF - 1 : buf - 1;
        ksteps(0, 2, afs[p], bfs[p], [&](int i) {
            if (i > 0 && i % S1 == 0 && i / S1 <= LMAX) {
                if (more && (i / S1 <= L || extra)) load(i / S1 - 1, t + NBUF - 1, lb);
            }
        });
        __builtin_amdgcn_sched_barrier(0);
        if (extra)
            wait_slabs_barrier<LMAX, NBUF - 2>(nslab - 2 - t);
        else
            wait_slabs_barrier<L, NBUF - 2>(nslab - 2 - t);
        const int nb = buf + 1 == NBUF ? 0 : buf + 1;
        ksteps(2, 4, afs[p], bfs[p], [&](int i) {
            if (i < NREAD) {
                read_op(i, nb, afs[p ^ 1], bfs[p ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };

    // Prologue: slabs 0 .. NBUF-1 in flight, wait for slab 0.
#pragma unroll
    for (int b = 0; b < NBUF; ++b)
        if (b < nslab) {
#pragma unroll
            for (int q = 0; q < LMAX; ++q)
                if (q < L || extra) load(q, b, b);
        }
    if (extra)
        wait_slabs_barrier<LMAX, NBUF - 1>(nslab - 1);
    else
        wait_slabs_barrier<L, NBUF - 1>(nslab - 1);
#pragma unroll
    for (int r = 0; r < NREAD; ++r) read_op(r, 0, afs[0], bfs[0]);

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int buf = 0;
    for (int t = 0; t < nslab; t += 2) {
        slab(P0{}, t, buf);
        buf = buf + 1 == NBUF ? 0 : buf + 1;
        if (t + 1 < nslab) {
            slab(P1{}, t + 1, buf);
            buf = buf + 1 == NBUF ? 0 : buf + 1;
        }
    }

    const float alpha = a.alpha, beta = a.beta;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wr * TM + fm * 16 + 4 * lg + i;
            if (row >= M) continue;
            float *yrow = a.Y + (int64_t)row * a.ldy;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int c = n0 + wc * TN + fn * 16 + lm;
                if (c < N) {
                    float v = alpha * acc[fm][fn][i];
                    if (beta != 0.f) v = fmaf(beta, yrow[c], v);
                    yrow[c] = v;
                }
            }
        }
    }
}

// ------------------------------ implicit GEMM, one filter tap per k-step

// The direct-to-LDS form for R x S filters with the contraction ordered so
// that the tap arithmetic disappears from the loop.  A slab is 4 channels x
// RS taps (BK = 4 RS); in k-step st of a slab, lane group g (lanes 16 g ..
// 16 g + 15) of every MFMA takes channel c0 + g at tap st.  So:
//   - the filter slab of row m is Wt[m][BK t .. BK t + BK - 1], contiguous
//     (channels c0 .. c0 + 3, all taps), loaded 16 bytes per lane straight
//     into LDS (row pitch BK floats, no padding: lane (g, m) reads
//     m BK + g RS + st, which falls in 64 distinct banks for RS = 9);
//   - a tap load covers one (channel, tap) row of the slab and 64 output
//     positions: vector offset vtap[st] (worked out once per thread: the
//     input offset of its position at tap st, or an out-of-range offset
//     where the tap leaves the image), scalar offset c H W.  The tap index
//     is a compile-time constant in the unrolled loop, so a load is an M0
//     write, a scalar add and the load.  B rows have pitch P, chosen so that
//     RS P = 16 or 48 (mod 64): the four lane groups' rows then fall in
//     distinct banks.
// Operands are read from LDS one k-step ahead (two register sets); a slab's
// buffer is read during the whole slab.  With a ring of three buffers the
// loads of slab t + 2 are spread over slab t's MFMAs into the buffer slab
// t - 1 used, and at the end of slab t one wait (slab t + 1 landed) and one
// barrier (every wave done with buffer t) hand over to slab t + 1.  With two
// (half the LDS, so that two workgroups share a CU) the loads of slab t + 1
// go into that buffer over the first half of slab t's MFMAs, and the wait at
// its end takes them all.
// C must be a multiple of 4; filter rows 16-byte aligned.
template <int RS, int BN>
constexpr int conv_tap_pitch()
{
    for (int p = BN; p < BN + 64; ++p)
        if ((RS * p) % 64 == 16 || (RS * p) % 64 == 48) return p;
    return -1;
}

template <int BM, int BN, int WM, int WN, int R, int S, int NBUF_ = 3>
struct ConvTap {
    static constexpr int RS = R * S;
    static constexpr int BK = 4 * RS;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int BH = BN / 64;               // 64-position pieces of a tap row
    static constexpr int P = conv_tap_pitch<RS, BN>();
    static constexpr int AW = (BM * RS + 63) / 64;   // filter loads (64 16-byte slots) per slab
    static constexpr int A_FLOATS = AW * 256;        // BM * BK, padded to whole loads
    static constexpr int BUF = A_FLOATS + BK * P;
    static constexpr int NBUF = NBUF_;
    static constexpr int LDS = NBUF * BUF;
    static constexpr int LA = AW / NW, XA = AW % NW;
    static constexpr int G = 4 * BH / NW;            // channels whose taps a wave loads
    static constexpr int LB = G * RS;                // tap loads per wave per slab
    static constexpr int L = LA + LB;
    static constexpr int LMAX = L + (XA > 0 ? 1 : 0);
    static constexpr int MF = RS * FM * FN;          // MFMAs per wave per slab
    // Loads are spread over the whole slab with three buffers (they land a
    // slab later), over its first half with two (they land at its end).
    static constexpr int STRIDE = (NBUF == 2 ? MF / 2 : MF) / (LMAX + 1);
    static_assert(P > 0, "no conflict-free tap row pitch");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BN % 64 == 0 && (4 * BH) % NW == 0 && G >= 1 && NW % BH == 0,
                  "each wave loads the taps of whole channels for one 64-position piece");
    static_assert(STRIDE >= 1, "too few MFMAs per slab for the loads");
    static_assert(NBUF == 2 || NBUF == 3, "a ring of two or three slabs");
    static_assert(LMAX * (NBUF - 1) <= 63, "loads in flight must fit the vmcnt field");
};

template <int BM, int BN, int WM, int WN, int WPE, int R, int S, int NBUF_ = 3>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
conv_tap_kernel(ConvArgs a, int tiles_m, int tiles_n)
{
    using D = ConvTap<BM, BN, WM, WN, R, S, NBUF_>;
    constexpr int RS = D::RS, BK = D::BK, NW = D::NW, TM = D::TM, TN = D::TN;
    constexpr int FM = D::FM, FN = D::FN, BH = D::BH, P = D::P, BUF = D::BUF;
    constexpr int NBUF = D::NBUF;
    constexpr int LA = D::LA, XA = D::XA, G = D::G, LB = D::LB, L = D::L, LMAX = D::LMAX;
    constexpr int S1 = D::STRIDE;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS];

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tiles_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = a.M, N = (int)a.N;
    const int nslab = a.C / 4;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN, wc = wave % WN;
    const bool extra = XA > 0 && wave < XA;

    const uint32_t x_bytes = 4u * (uint32_t)a.batch * (uint32_t)a.C * (uint32_t)a.H * (uint32_t)a.W;
    const uint32_t w_bytes = 4u * ((uint32_t)(M - 1) * (uint32_t)a.ldw + (uint32_t)a.K);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.X), 0, (int)x_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.Wt), 0, (int)w_bytes, kBufferWord3);

    // Filter loads: load qa of this wave is slab load j = wave + qa NW, whose
    // lane l takes 16-byte slot 64 j + l: row (64 j + l) / RS, quad
    // (64 j + l) % RS of the row's BK floats.  Slots past the tile's BM
    // rows (the last load's padding) and rows past M land as zeros.
    uint32_t a_voff[LA + 1];
#pragma unroll
    for (int qa = 0; qa <= LA; ++qa) {
        const int j = wave + qa * NW;
        const int slot = 64 * j + lane;
        const int row = m0 + slot / RS;
        a_voff[qa] = (j < D::AW && slot < BM * RS && row < M)
                         ? 4u * ((uint32_t)row * (uint32_t)a.ldw + 4u * (uint32_t)(slot % RS))
                         : kOffsetOut;
    }
    // Tap loads: this wave's 64-position piece h and channels g0 .. g0 + G - 1
    // of each slab; vtap[st] is the lane's input offset at tap st.
    const int h = wave % BH;
    const int g0 = (wave / BH) * G;
    const int n = n0 + 64 * h + lane;
    uint32_t vtap[RS];
#pragma unroll
    for (int st = 0; st < RS; ++st) vtap[st] = kOffsetOut;
    if (n < N) {
        const int ohw = a.OH * a.OW;
        const int b = n / ohw;
        const int p = n - b * ohw;
        const int oh = p / a.OW, ow = p - oh * a.OW;
        const int ih0 = oh * a.sh - a.ph, iw0 = ow * a.sw - a.pw;
        const uint32_t pbase4 =
            4u * (((uint32_t)(b * a.C * a.H) + (uint32_t)ih0) * (uint32_t)a.W + (uint32_t)iw0);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int s = 0; s < S; ++s)
                if ((unsigned)(ih0 + r) < (unsigned)a.H && (unsigned)(iw0 + s) < (unsigned)a.W)
                    vtap[r * S + s] = pbase4 + 4u * ((uint32_t)r * (uint32_t)a.W + (uint32_t)s);
    }
    const uint32_t hw4 = 4u * (uint32_t)a.H * (uint32_t)a.W;

    // Load q of slab t into ring buffer buf: the tap loads, then the filter
    // loads (the extra waves' additional filter load last).
    auto load = [&](int q, int t, int buf) {
        float *base = lds + buf * BUF;
        if (q < LB) {
            const int g = g0 + q / RS, st = q % RS;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (lds_float *)(base + D::A_FLOATS + (g * RS + st) * P + 64 * h), 4,
                (int)vtap[st], (int)((uint32_t)(4 * t + g) * hw4), 0, 0);
        } else {
            const int qa = q - LB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wrs, (lds_float *)(base + (wave + qa * NW) * 256), 16, (int)a_voff[qa],
                4 * BK * t, 0, 0);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int lg = lane >> 4, lm = lane & 15;
    const int a_lane = (wr * TM + lm) * BK + lg * RS;
    const int b_lane = D::A_FLOATS + lg * RS * P + wc * TN + lm;
    float af[2][FM], bf[2][FN];
    // Operands of k-step st of the slab in buffer buf into set p.
    auto read = [&](int p, int buf, int st) {
        const float *base = lds + buf * BUF;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) af[p][fm] = base[a_lane + fm * 16 * BK + st];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) bf[p][fn] = base[b_lane + st * P + fn * 16];
    };

    // Slab t from buffer buf; its k-step st uses operand set (P0 + st) & 1.
    // It loads slab t + NBUF - 1 into the buffer slab t - 1 used (every
    // wave was done with it at the barrier that ended slab t - 1).
    auto slab = [&](auto P0, int t, int buf) {
        constexpr int p0 = decltype(P0)::value;
        const bool more = t + NBUF - 1 < nslab;
        const int lb = buf == 0 ? NBUF - 1 : buf - 1;  // the buffer of slab t - 1
#pragma unroll
        for (int st = 0; st < RS; ++st) {
            const int p = (p0 + st) & 1;
            if (st + 1 < RS) read(p ^ 1, buf, st + 1);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int i = (st * FM + fm) * FN + fn;
                    if (i > 0 && i % S1 == 0 && i / S1 <= LMAX) {
                        const int q = i / S1 - 1;
                        if (more && (q < L || extra)) load(q, t + NBUF - 1, lb);
                    }
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[p][fm], bf[p][fn],
                                                                       acc[fm][fn], 0, 0, 0);
                }
        }
        // Slab t + 1 has landed and every wave is done with buffer buf.
        if (extra)
            wait_slabs_barrier<LMAX, NBUF - 2>(nslab - 2 - t);
        else
            wait_slabs_barrier<L, NBUF - 2>(nslab - 2 - t);
        if (t + 1 < nslab) read((p0 + RS) & 1, buf == NBUF - 1 ? 0 : buf + 1, 0);
    };

    // Prologue: slabs 0 .. NBUF - 2 in flight, wait for slab 0.
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b)
        if (b < nslab) {
#pragma unroll
            for (int q = 0; q < LMAX; ++q)
                if (q < L || extra) load(q, b, b);
        }
    if (extra)
        wait_slabs_barrier<LMAX, NBUF - 2>(nslab - 1);
    else
        wait_slabs_barrier<L, NBUF - 2>(nslab - 1);
    read(0, 0, 0);

    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, RS & 1>;
    int buf = 0;
    for (int t = 0; t < nslab; t += 2) {
        slab(Q0{}, t, buf);
        buf = buf == NBUF - 1 ? 0 : buf + 1;
        if (t + 1 < nslab) {
            slab(Q1{}, t + 1, buf);
            buf = buf == NBUF - 1 ? 0 : buf + 1;
        }
    }

    const float alpha = a.alpha, beta = a.beta;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wr * TM + fm * 16 + 4 * lg + i;
            if (row >= M) continue;
            float *yrow = a.Y + (int64_t)row * a.ldy;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int c = n0 + wc * TN + fn * 16 + lm;
                if (c < N) {
                    float v = alpha * acc[fm][fn][i];
                    if (beta != 0.f) v = fmaf(beta, yrow[c], v);
                    yrow[c] = v;
                }
            }
        }
    }
}

// ------------------------------------------------------ stem fast path

// For the first layers of image networks: few input channels, a large
// image, M <= 32 MB output channels (the two stem readings of the skinny
// convolution-as-GEMM shapes: 3 channels, 7 x 7 stride 2 pad 3 or 3 x 3
// stride 2 pad 1, on 224 x 224 images).
//
// Output positions are cut into strips of 256 consecutive positions of one
// image, shared out over the resident workgroups (below).  For each
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
    const bool full_rows = a.M == 32 * MB;  // every row of the row blocks is an output
    // Strip order.  Workgroups are dealt to the eight XCDs in turn
    // (workgroup b runs on XCD b % 8), so the strips are cut into eight
    // contiguous regions, one per XCD, and an XCD's workgroups take its
    // region's strips round-robin.  The strips in flight on an XCD are then
    // neighbours: their windows share input rows in that XCD's L2, so each
    // input row crosses HBM once, and their output forms a few long runs
    // per row rather than one short piece per workgroup (stores alone, in
    // this stem's pattern: 5.1 TB/s with contiguous ranges per workgroup,
    // 5.6 TB/s dealt out).  A workgroup's strip count differs from the mean
    // of its XCD's workgroups by at most one.  Grids of fewer than eight
    // deal out all strips.
    const int NG = (int)gridDim.x;
    // Strip indices are below total_strips <= INT_MAX, and a step is at
    // most the grid size, so they and their sums fit 32 unsigned bits.
    uint32_t s0, s1, sstep;
    if (NG < 8) {
        s0 = blockIdx.x;
        s1 = total_strips;
        sstep = NG;
    } else {
        const int x = (int)blockIdx.x % 8;
        s0 = (uint32_t)((int64_t)x * total_strips / 8) + blockIdx.x / 8;
        s1 = (uint32_t)((int64_t)(x + 1) * total_strips / 8);
        sstep = (NG - 1 - x) / 8 + 1;  // the workgroups of XCD x
    }
    const float *a_lane = As + (h * 32 * MB + j) * TP;

    // Input loads and output stores address the kernel argument's base with
    // 32-bit byte offsets (the host takes this kernel only for inputs and
    // outputs below 4 GiB), which keeps 64-bit address arithmetic out of the
    // registers the tap loop needs.
    //
    // The window of strip st is fetched into registers (this thread's
    // 16-byte groups e = tid + 256 i of the CH * ROWS rows of G4 groups)
    // before the strip's MFMAs and written to LDS after them.  The loads
    // are unconditional: through a buffer resource with an out-of-range
    // offset where a group lies outside the image (below), else from a
    // clamped address, with which of them hold data kept as bits of one
    // register.  A lane-dependent branch around a load would keep its
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
    // With aligned rows, a 16-byte group lies wholly inside the image or
    // wholly outside it, and inputs under 2^31 bytes are read through a
    // buffer resource: a group outside gets an offset past the end, the
    // load returns zeros, and the window is written as loaded.  A group
    // whose columns are outside carries that offset (2^31) from the start
    // and adds it to the strip's base: a base at or past zero is below
    // 2^31, so the sum is at or past 2^31; a base that wrapped (first window
    // row above image 0, by at most pad_h rows) gives 2^31 - pad_h W 4,
    // which the condition below keeps past the input's end.
    const bool buf_x =
        vec_x && 4 * ((int64_t)a.batch * a.C * a.H * a.W + (int64_t)a.ph * a.W) <= (1ll << 31);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.X), 0,
        buf_x ? (int)(4 * (int64_t)a.batch * a.C * a.H * a.W) : 0, kBufferWord3);
    uint32_t gbuf[NST];  // goff, or kOffsetOut for a group outside the columns
    int grow[NST];       // the group's window row
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        gbuf[i] = (col_ok >> (4 * i)) & 15ull ? goff[i] : kOffsetOut;
        grow[i] = ((tid + 256 * i) / G4) % ROWS;
    }
    // The window of a strip of image b whose first output row is oh_lo.
    auto fetch = [&](int b, int oh_lo) {
        const int ih_lo = oh_lo * SH - a.ph;
        // Byte offset of (image b, channel 0, row ih_lo, column 0); may
        // wrap when ih_lo < 0, where only rows inside the image are read.
        const uint32_t sbase = (uint32_t)((b * a.C * a.H + ih_lo) * a.W) * 4u;
        if (buf_x) {
            // Strips away from the image's top and bottom edges test no rows.
            const bool rows_in = ih_lo >= 0 && ih_lo + ROWS <= a.H;
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                const bool ok = rows_in || (unsigned)(ih_lo + grow[i]) < (unsigned)a.H;
                pre[i] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               xr, (int)(ok ? sbase + gbuf[i] : kOffsetOut), 0, 0));
            }
            return;
        }
        valid = 0;
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const bool row_ok = (unsigned)(ih_lo + grow[i]) < (unsigned)a.H;
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
        if (buf_x) {
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                const int e = tid + 256 * i;
                if (e < CH * ROWS * G4) *reinterpret_cast<f32x4 *>(win + 4 * e) = pre[i];
            }
            return;
        }
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

    // Strip st is strip si of image b (st = b spi + si).  The loop carries
    // (b, si) and the strip's first output row from one strip to the next,
    // by additions: the step is qstep images and rstep strips.
    const int spi = strips_per_image;
    const int qstep = (int)(sstep / spi), rstep = (int)(sstep % spi);
    int cur_b = (int)(s0 / spi), cur_si = (int)(s0 % spi);
    int cur_oh = cur_si * kStemStrip / a.OW;
    if (s0 < s1) {
        fetch(cur_b, cur_oh);
        place();
    }
    __syncthreads();  // the weights and the first window are in LDS
    for (uint32_t st = s0; st < s1; st += sstep) {
        const int b = cur_b;
        const int p0 = cur_si * kStemStrip;
        const int oh_lo = cur_oh;
        int nxt_b = cur_b + qstep, nxt_si = cur_si + rstep;
        if (nxt_si >= spi) {
            nxt_si -= spi;
            ++nxt_b;
        }
        const int nxt_oh = nxt_si * kStemStrip / a.OW;
        // The next strip's window travels while this one is computed.
        if (st + sstep < s1) fetch(nxt_b, nxt_oh);
        cur_b = nxt_b;
        cur_si = nxt_si;
        cur_oh = nxt_oh;

        // Per-lane window bases.  Lane j of a wave holds positions 2j and
        // 2j + 1 of the wave's 64 (column blocks cb = 0, 1 interleaved), so its
        // two outputs of a row are adjacent.  Positions past the image clamp
        // to its last one; their outputs are not stored.  A position's
        // offset from the strip's first output row is below OW + 255, so
        // its output row is at most (ROWS - R) / SH rows on (what the host
        // checks when it picks this kernel): a few compare-and-subtract
        // steps find it, with no division.
        int base[2][4];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            int q = p0 + wave * 64 + 2 * j + cb;
            q = q < ohw ? q : ohw - 1;
            int ow = q - oh_lo * a.OW, dr = 0;
#pragma unroll
            for (int u = 0; u < (ROWS - R) / SH; ++u)
                if (ow >= a.OW) {
                    ow -= a.OW;
                    ++dr;
                }
            const int pb = dr * SH * WPITCH + ow * SW - a.pw + kStemCol0;
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
        if (full_rows && vec_y && p0 + wave * 64 + 64 <= ohw) {
            // Every lane stores both positions of every row: the address is
            // a wave-uniform row base plus this lane's fixed offset.
            const uint32_t wbase = (uint32_t)(b * ohw + p0 + wave * 64) * 4u;
            const uint32_t lane_off = (4u * (uint32_t)h * ldy + 2u * (uint32_t)j) * 4u;
            // The row stride, opaque here so that the 16 MB row bases are
            // formed store by store (a few scalar instructions each) rather
            // than hoisted out of the strip loop into scalar registers.
            uint32_t ldy4 = ldy * 4u;
            asm volatile("" : "+s"(ldy4));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row0 = mb * 32 + 8 * (i >> 2) + (i & 3);  // half-wave 0's row
                    char *rb = ybase + (wbase + (uint32_t)row0 * ldy4);
                    f32x2 *py = reinterpret_cast<f32x2 *>(rb + lane_off);
                    f32x2 v = {alpha * acc[mb][0][i], alpha * acc[mb][1][i]};
                    if (beta != 0.f) v += beta * *py;
                    __builtin_nontemporal_store(v, py);
                }
        } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = mb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (row >= a.M || q0 >= ohw) continue;
                    float *py =
                        reinterpret_cast<float *>(ybase + ((uint32_t)row * ldy + n0) * 4u);
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
        }

        __syncthreads();  // every wave is done with this window
        if (st + sstep < s1) place();
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
