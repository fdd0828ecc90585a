// Vector-FMA register-tile kernel (the comparison path to the MFMA kernel).
//
// This is the design the pages build up step by step for SIMT cores: the
// 2-D thread tile with register-cached operand fragments, 128-bit loads,
// an A slab stored transposed (k-major) so that a thread's A fragment is one
// 128-bit LDS read, and double-buffered slabs with one barrier per slab
// (NVIDIA_SGEMM_PRACTICE README, kernels 4-7; cnblogs matmul_opt.cu,
// "Advanced" kernel: BM = BN = 128, BK = 8, 8 x 8 outputs per thread).
//
// Changes for gfx950:
//   * 256 threads = four 64-lane waves.  Thread (ty, tx) = (tid/16, tid%16)
//     owns rows {4ty..4ty+3, 64+4ty..64+4ty+3} and columns
//     {4tx..4tx+3, 64+4tx..64+4tx+3} of the 128 x 128 tile.  Splitting each
//     8-wide fragment into two 4-wide halves 64 apart makes the 16 lanes
//     of a row read 64 consecutive floats of the B slab (all banks, no
//     conflict) and lets a whole wave share 4 distinct A addresses
//     (broadcast).
//   * Fragments are 128-bit LDS reads; 64 scalar FMAs per k per thread.
//   * A 160 x 160 form (10 x 10 per thread: a third, 2-wide band of rows
//     and columns from 128) for shapes where it fills whole rounds.
//   * Edges: loads outside the matrix are zero-filled, stores are masked,
//     so any M, N, K and any leading dimension work.
#pragma once

#include "common.hpp"
#include "mfma_tile.hpp"  // load4_masked

namespace sgemm {

// Row (or column) of the tile that fragment element i of thread index t
// (ty or tx) covers: 4-wide bands 64 apart, then, for the 160 tile, a
// 2-wide band from 128.
template <int TT>
__device__ __forceinline__ int valu_band(int i, int t)
{
    return i < 4 ? 4 * t + i : (i < 8 ? 64 + 4 * t + i - 4 : 128 + 2 * t + i - 8);
}

// BT x BT tile (BT = 128 or 160), BK = 8, 256 threads, (BT / 16)^2 outputs
// per thread.  The 160 tile fills whole rounds where the 128 one leaves a
// part-empty last round (5120^3: 1024 tiles over 512 resident workgroups
// against 1600).
template <bool AVEC, bool BVEC, int BT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
valu_tile_kernel(GemmArgs g)
{
    static_assert(BT == 128 || BT == 160, "tile is 128 or 160");
    constexpr int BM = BT, BN = BT, BK = 8;
    constexpr int TT = BT / 16;   // outputs per thread along each axis
    constexpr int PA = BM + 4;    // pitch of the transposed A slab (k-major)
    constexpr int PB = BN + 4;    // pitch of the B slab (k-major)
    constexpr int NL = (2 * BT + 255) / 256;  // float4 loads per operand per thread
    constexpr int B4 = BN / 4;    // float4 per B slab row

    __shared__ __attribute__((aligned(16))) float As[2][BK * PA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * PB];

    int tm, tn;
    tile_of_block(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;
    const int tid = threadIdx.x;
    const int ty = tid >> 4;
    const int tx = tid & 15;

    // Slab float4 number i = tid + 256 l (l < NL, i < 2 BT): of A, row i/2,
    // k 4 (i%2); of B, k i / B4, columns 4 (i % B4).
    int a_r[NL], a_c[NL], b_r[NL], b_c[NL];
    bool a_ok[NL], live[NL];
    const float *a_src[NL];
    const float *b_src[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const int i = tid + 256 * l;
        live[l] = i < 2 * BT;
        a_r[l] = i >> 1;
        a_c[l] = (i & 1) * 4;
        a_ok[l] = live[l] && m0 + a_r[l] < M;
        a_src[l] = g.A + (int64_t)(m0 + a_r[l]) * g.lda + a_c[l];
        b_r[l] = i / B4;
        b_c[l] = (i % B4) * 4;
        b_src[l] = g.B + (int64_t)b_r[l] * g.ldb + n0 + b_c[l];
    }

    f32x4 ra[NL], rb[NL];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            if (!live[l]) continue;
            ra[l] = load4_masked<AVEC>(a_src[l] + k0, a_ok[l], k0 + a_c[l], K);
            rb[l] = load4_masked<BVEC>(b_src[l] + (int64_t)k0 * g.ldb, k0 + b_r[l] < K,
                                       n0 + b_c[l], N);
        }
    };
    auto stash = [&](int buf) {
        float *as = &As[buf][0];
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            if (!live[l]) continue;
            as[(a_c[l] + 0) * PA + a_r[l]] = ra[l].x;
            as[(a_c[l] + 1) * PA + a_r[l]] = ra[l].y;
            as[(a_c[l] + 2) * PA + a_r[l]] = ra[l].z;
            as[(a_c[l] + 3) * PA + a_r[l]] = ra[l].w;
            *reinterpret_cast<f32x4 *>(&Bs[buf][b_r[l] * PB + b_c[l]]) = rb[l];
        }
    };

    float acc[TT][TT];
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TT; ++j)
            acc[i][j] = 0.f;

    // Unrolled over all of BK, the compiler hoists every step's fragments;
    // for the 160 tile (100 accumulators) that overflows two waves' registers.
    constexpr int KU = TT == 10 ? 2 : BK;
    auto compute = [&](int buf) {
        const float *as = &As[buf][0];
        const float *bs = &Bs[buf][0];
#pragma unroll KU
        for (int k = 0; k < BK; ++k) {
            float af[TT], bf[TT];
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(as + k * PA + 4 * ty);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(as + k * PA + 64 + 4 * ty);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bs + k * PB + 4 * tx);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bs + k * PB + 64 + 4 * tx);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                af[q] = a0[q];
                af[4 + q] = a1[q];
                bf[q] = b0[q];
                bf[4 + q] = b1[q];
            }
            if constexpr (TT == 10) {
                const f32x2 a2 = *reinterpret_cast<const f32x2 *>(as + k * PA + 128 + 2 * ty);
                const f32x2 b2 = *reinterpret_cast<const f32x2 *>(bs + k * PB + 128 + 2 * tx);
                af[8] = a2.x;
                af[9] = a2.y;
                bf[8] = b2.x;
                bf[9] = b2.y;
            }
#pragma unroll
            for (int i = 0; i < TT; ++i)
#pragma unroll
                for (int j = 0; j < TT; ++j)
                    acc[i][j] = fmaf(af[i], bf[j], acc[i][j]);
        }
    };

    const int nslab = (K + BK - 1) / BK;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int t = 0; t < nslab; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < nslab;
        if (more) fetch((t + 1) * BK);
        compute(cur);
        if (more) stash(cur ^ 1);
        __syncthreads();
    }

    const float alpha = g.alpha, beta = g.beta;
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int row = m0 + valu_band<TT>(i, ty);
        if (row >= M) continue;
        float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
        for (int j = 0; j < TT; ++j) {
            const int col = n0 + valu_band<TT>(j, tx);
            if (col < N) {
                float v = alpha * acc[i][j];
                if (beta != 0.f) v = fmaf(beta, crow[col], v);
                crow[col] = v;
            }
        }
    }
}

// C <- beta * C over the M x N window (beta == 0 writes zeros without
// reading C).  Used when K == 0 or alpha == 0.
__global__ void __launch_bounds__(256)
scale_kernel(float *C, int64_t ldc, int M, int N, float beta)
{
    const int64_t total = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / N;
        const int64_t c = idx - r * N;
        float *p = C + r * ldc + c;
        *p = (beta == 0.f) ? 0.f : beta * *p;
    }
}

}  // namespace sgemm
