// The pages' optimisation ladder for SIMT cores, rebuilt on gfx950 as
// separate kernels, one per rung, for measurement beside the pages' own
// tables.  None of them is picked by the shape-driven selector; they run only
// when forced through sgemm_f32_variant.  The last rung, double-buffered
// slabs, is valu_tile_kernel.
//
// Every rung handles any M, N, K, leading dimension and alignment: loads
// outside the matrices read zero (cnblogs matmul_opt.cu, "Optimized" kernel)
// and stores are masked, which the NVIDIA_SGEMM_PRACTICE kernels leave out.
// Every rung ends with the same epilogue, C = alpha * acc + beta * C
// (NVIDIA_SGEMM_PRACTICE README, kernel 1), with C not read when beta == 0.
//
// Rungs (workgroup tile, threads, what changes from the previous one):
//   0 naive        16 x 16, 256: one thread per element of C, its dot
//                  product read from global memory; consecutive lanes take
//                  consecutive rows (NVIDIA_SGEMM_PRACTICE kernel 1;
//                  UNIVERSAL_SGEMM_CUDA README "naive").
//   1 coalesced     4 x 64, 256: consecutive lanes take consecutive columns,
//                  so a 64-lane wave reads one 256-byte run of a B row and
//                  writes one of C, and shares its A element
//                  (UNIVERSAL_SGEMM_CUDA "global memory coalescing").
//   2 lds          32 x 32, 1024: A and B in 32 x 32 LDS tiles, rows padded
//                  by one float (NVIDIA_SGEMM_PRACTICE kernel 2; matmul_opt.cu
//                  "Optimized"; UNIVERSAL_SGEMM_CUDA "shared memory cache
//                  blocking").
//   3 tile1d       64 x 64, 512, BK = 8: each thread computes 8 rows of one
//                  column, its B value held in a register (kernel 3;
//                  "blocktiling 1d").
//   4 tile2d      128 x 128, 256, BK = 8: each thread computes an 8 x 8 block
//                  of C, operands read from LDS in the product loop (kernel
//                  4; "blocktiling 2d").
//   5 regcache    as 4, with the thread's 8 A and 8 B values per k copied to
//                  registers first and multiplied as an outer product
//                  (kernel 5).
//   6 vec4        as 5, with 128-bit global loads where rows are aligned and
//                  the A slab stored transposed (k-major), so that fragments
//                  are 128-bit LDS reads (kernel 6).
//   7 dbuf        valu_tile_kernel: as 6 with two slab buffers, the next slab
//                  loaded while the current one is multiplied, one barrier per
//                  slab (kernel 7; matmul_opt.cu "Advanced").
#pragma once

#include "common.hpp"
#include "mfma_tile.hpp"  // load4_masked

namespace sgemm {

constexpr int kLadderRungs = 8;

// C(m, n) = alpha * acc + beta * C(m, n); C is not read when beta == 0.
__device__ __forceinline__ void ladder_store(const GemmArgs &g, int m, int n, float acc)
{
    float *p = g.C + (int64_t)m * g.ldc + n;
    float v = g.alpha * acc;
    if (g.beta != 0.f) v = fmaf(g.beta, *p, v);
    *p = v;
}

// Output tile of this workgroup, row-major over tiles_m x tiles_n.
__device__ __forceinline__ void ladder_tile(const GemmArgs &g, int &tm, int &tn)
{
    tm = blockIdx.x / g.tiles_n;
    tn = blockIdx.x - tm * g.tiles_n;
}

// Rung 0.
__global__ void __launch_bounds__(256) ladder_naive_kernel(GemmArgs g)
{
    int tm, tn;
    ladder_tile(g, tm, tn);
    const int m = tm * 16 + (threadIdx.x & 15);
    const int n = tn * 16 + (threadIdx.x >> 4);
    if (m >= g.M || n >= g.N) return;
    const float *a = g.A + (int64_t)m * g.lda;
    const float *b = g.B + n;
    float acc = 0.f;
    for (int k = 0; k < g.K; ++k) acc = fmaf(a[k], b[(int64_t)k * g.ldb], acc);
    ladder_store(g, m, n, acc);
}

// Rung 1.
__global__ void __launch_bounds__(256) ladder_coalesced_kernel(GemmArgs g)
{
    int tm, tn;
    ladder_tile(g, tm, tn);
    const int m = tm * 4 + (threadIdx.x >> 6);
    const int n = tn * 64 + (threadIdx.x & 63);
    if (m >= g.M || n >= g.N) return;
    const float *a = g.A + (int64_t)m * g.lda;
    const float *b = g.B + n;
    float acc = 0.f;
    for (int k = 0; k < g.K; ++k) acc = fmaf(a[k], b[(int64_t)k * g.ldb], acc);
    ladder_store(g, m, n, acc);
}

// Rung 2.
__global__ void __launch_bounds__(1024) ladder_lds_kernel(GemmArgs g)
{
    constexpr int T = 32;
    __shared__ float As[T][T + 1];
    __shared__ float Bs[T][T + 1];
    int tm, tn;
    ladder_tile(g, tm, tn);
    const int ty = threadIdx.x / T, tx = threadIdx.x % T;
    const int m = tm * T + ty, n = tn * T + tx;
    float acc = 0.f;
    for (int k0 = 0; k0 < g.K; k0 += T) {
        As[ty][tx] = (m < g.M && k0 + tx < g.K) ? g.A[(int64_t)m * g.lda + k0 + tx] : 0.f;
        Bs[ty][tx] = (k0 + ty < g.K && n < g.N) ? g.B[(int64_t)(k0 + ty) * g.ldb + n] : 0.f;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < T; ++kk) acc = fmaf(As[ty][kk], Bs[kk][tx], acc);
        __syncthreads();
    }
    if (m < g.M && n < g.N) ladder_store(g, m, n, acc);
}

// Rung 3.
__global__ void __launch_bounds__(512) ladder_tile1d_kernel(GemmArgs g)
{
    constexpr int BM = 64, BN = 64, BK = 8, TM = 8;
    __shared__ float As[BM][BK];
    __shared__ float Bs[BK][BN];
    int tm, tn;
    ladder_tile(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int col = tid % BN, row0 = (tid / BN) * TM;
    // One element of each slab per thread.
    const int ar = tid / BK, ac = tid % BK;
    const int br = tid / BN, bc = tid % BN;
    float acc[TM] = {};
    for (int k0 = 0; k0 < g.K; k0 += BK) {
        As[ar][ac] = (m0 + ar < g.M && k0 + ac < g.K)
                         ? g.A[(int64_t)(m0 + ar) * g.lda + k0 + ac] : 0.f;
        Bs[br][bc] = (k0 + br < g.K && n0 + bc < g.N)
                         ? g.B[(int64_t)(k0 + br) * g.ldb + n0 + bc] : 0.f;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const float b = Bs[k][col];
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i] = fmaf(As[row0 + i][k], b, acc[i]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = m0 + row0 + i, n = n0 + col;
        if (m < g.M && n < g.N) ladder_store(g, m, n, acc[i]);
    }
}

// Rungs 4 (REGCACHE false) and 5 (true): 128 x 128 x 8 tile, 8 x 8 outputs
// per thread at rows 8 ty .. 8 ty + 7, columns 8 tx .. 8 tx + 7.
template <bool REGCACHE>
__global__ void __launch_bounds__(256) ladder_tile2d_kernel(GemmArgs g)
{
    constexpr int BM = 128, BN = 128, BK = 8, TM = 8, TN = 8;
    __shared__ float As[BM][BK];
    __shared__ float Bs[BK][BN];
    int tm, tn;
    ladder_tile(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int ty = tid / 16, tx = tid % 16;
    float acc[TM][TN] = {};
    for (int k0 = 0; k0 < g.K; k0 += BK) {
        // Four elements of each slab per thread.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = tid + 256 * u;
            const int ar = e / BK, ac = e % BK;
            As[ar][ac] = (m0 + ar < g.M && k0 + ac < g.K)
                             ? g.A[(int64_t)(m0 + ar) * g.lda + k0 + ac] : 0.f;
            const int br = e / BN, bc = e % BN;
            Bs[br][bc] = (k0 + br < g.K && n0 + bc < g.N)
                             ? g.B[(int64_t)(k0 + br) * g.ldb + n0 + bc] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            if constexpr (REGCACHE) {
                float af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) af[i] = As[TM * ty + i][k];
#pragma unroll
                for (int j = 0; j < TN; ++j) bf[j] = Bs[k][TN * tx + j];
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(af[i], bf[j], acc[i][j]);
            } else {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = fmaf(As[TM * ty + i][k], Bs[k][TN * tx + j], acc[i][j]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int m = m0 + TM * ty + i, n = n0 + TN * tx + j;
            if (m < g.M && n < g.N) ladder_store(g, m, n, acc[i][j]);
        }
}

// Rung 6: as rung 5 with 128-bit global loads (AVEC / BVEC: the rows of A /
// B are 16-byte aligned, else the same loads run element-wise) and the A slab
// stored k-major, so both fragments are two 128-bit LDS reads.
template <bool AVEC, bool BVEC>
__global__ void __launch_bounds__(256) ladder_vec4_kernel(GemmArgs g)
{
    constexpr int BM = 128, BN = 128, BK = 8, TM = 8, TN = 8;
    __shared__ __attribute__((aligned(16))) float As[BK][BM];  // transposed
    __shared__ __attribute__((aligned(16))) float Bs[BK][BN];
    int tm, tn;
    ladder_tile(g, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int ty = tid / 16, tx = tid % 16;
    // One float4 of A (row tid / 2, k 4 (tid % 2)) and one of B (k tid / 32,
    // columns 4 (tid % 32)) per thread per slab.
    const int ar = tid / 2, ac = (tid % 2) * 4;
    const int br = tid / 32, bc = (tid % 32) * 4;
    const float *a_src = g.A + (int64_t)(m0 + ar) * g.lda + ac;
    float acc[TM][TN] = {};
    for (int k0 = 0; k0 < g.K; k0 += BK) {
        const f32x4 a = load4_masked<AVEC>(a_src + k0, m0 + ar < g.M, k0 + ac, g.K);
        const f32x4 b = load4_masked<BVEC>(g.B + (int64_t)(k0 + br) * g.ldb + n0 + bc,
                                           k0 + br < g.K, n0 + bc, g.N);
        As[ac + 0][ar] = a.x;
        As[ac + 1][ar] = a.y;
        As[ac + 2][ar] = a.z;
        As[ac + 3][ar] = a.w;
        *reinterpret_cast<f32x4 *>(&Bs[br][bc]) = b;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&As[k][TM * ty]);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&As[k][TM * ty + 4]);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&Bs[k][TN * tx]);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&Bs[k][TN * tx + 4]);
            const float af[TM] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float bf[TN] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(af[i], bf[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int m = m0 + TM * ty + i, n = n0 + TN * tx + j;
            if (m < g.M && n < g.N) ladder_store(g, m, n, acc[i][j]);
        }
}

}  // namespace sgemm
