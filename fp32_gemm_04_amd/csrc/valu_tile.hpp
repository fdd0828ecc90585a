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
//   * Edges: loads outside the matrix are zero-filled, stores are masked,
//     so any M, N, K and any leading dimension work.
#pragma once

#include "common.hpp"
#include "mfma_tile.hpp"  // load4_masked

namespace sgemm {

template <bool AVEC, bool BVEC>
__global__ void __launch_bounds__(256)
valu_tile_kernel(GemmArgs g)
{
    constexpr int BM = 128, BN = 128, BK = 8;
    constexpr int PA = BM + 4;  // pitch of the transposed A slab (k-major)
    constexpr int PB = BN + 4;  // pitch of the B slab (k-major)

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

    // One float4 of A (row tid/2, k 4*(tid%2)) and one of B (k tid/32,
    // columns 4*(tid%32)) per thread per slab.
    const int a_r = tid >> 1;
    const int a_c = (tid & 1) * 4;
    const bool a_ok = m0 + a_r < M;
    const float *a_src = g.A + (int64_t)(m0 + a_r) * g.lda + a_c;
    const int b_r = tid >> 5;
    const int b_c = (tid & 31) * 4;
    const float *b_src = g.B + (int64_t)b_r * g.ldb + n0 + b_c;

    f32x4 ra, rb;
    auto fetch = [&](int k0) {
        ra = load4_masked<AVEC>(a_src + k0, a_ok, k0 + a_c, K);
        rb = load4_masked<BVEC>(b_src + (int64_t)k0 * g.ldb, k0 + b_r < K, n0 + b_c, N);
    };
    auto stash = [&](int buf) {
        float *as = &As[buf][0];
        as[(a_c + 0) * PA + a_r] = ra.x;
        as[(a_c + 1) * PA + a_r] = ra.y;
        as[(a_c + 2) * PA + a_r] = ra.z;
        as[(a_c + 3) * PA + a_r] = ra.w;
        *reinterpret_cast<f32x4 *>(&Bs[buf][b_r * PB + b_c]) = rb;
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = 0.f;

    auto compute = [&](int buf) {
        const float *as = &As[buf][4 * ty];
        const float *bs = &Bs[buf][4 * tx];
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(as + k * PA);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(as + k * PA + 64);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bs + k * PB);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bs + k * PB + 64);
            const float af[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float bf[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
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
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4);
        if (row >= M) continue;
        float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = n0 + (j < 4 ? 4 * tx + j : 64 + 4 * tx + j - 4);
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
