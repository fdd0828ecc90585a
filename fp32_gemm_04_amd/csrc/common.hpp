// Shared device-side pieces of the SGEMM kernels: argument block, vector
// type, and the workgroup -> output-tile mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Everything a tile kernel needs.  Leading dimensions are 64-bit so that
// row*ld never overflows, whatever the matrix size.
struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;  // output tiles along M and N
    int group_m;           // tile rows per raster group (L2 reuse)
};

// Host-side handle of a tile kernel: all of them take the argument block.
typedef void (*KernelFn)(GemmArgs);

// Direct-load MFMA kernel for a tile shape and waves-per-SIMD target, or
// null if none is built for it (defined in mfma_dl.hip).
KernelFn direct_kernel(int bm, int bn, int wm, int wn, int wpe);

// Number of XCDs (accelerator complex dies) on MI355X.  The hardware hands
// consecutive workgroup ids to the XCDs in turn, and each XCD has its own L2.
constexpr int kNumXcd = 8;

// Map a workgroup id to the output tile (tm, tn) it computes.
//
// Step 1 (XCD-aware): workgroups b, b+8, b+16, ... all run on one XCD, so
// they are given one contiguous range of logical tile numbers; tiles that
// share rows of A and columns of B then meet in the same L2.  The mapping
// is a bijection on [0, nblocks) for any nblocks.
// Step 2 (grouped raster): logical tiles walk down `group_m` tile rows before
// moving one tile column right, so the tiles resident at one time form a
// compact rectangle rather than a long strip.
__device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n,
                                              int group_m, int &tm, int &tn)
{
    const int nblocks = tiles_m * tiles_n;
    const int q = nblocks / kNumXcd;
    const int r = nblocks % kNumXcd;
    const int x = bid % kNumXcd;
    const int i = bid / kNumXcd;
    const int logical = x * q + (x < r ? x : r) + i;

    const int per_group = group_m * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * group_m;
    const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in_group = logical - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// Balancing a kernel's work per SIMD, for kernels that run one workgroup
// per CU whose 4 WPE waves fill it: each SIMD has its own matrix core, and
// how the hardware places a workgroup's waves on the SIMDs is not fixed.  A
// wave reads the SIMD it runs on (HW_ID) and takes a rank among that SIMD's
// waves with an LDS counter; simd_share then numbers the waves SIMD by SIMD,
// so waves on one SIMD hold adjacent shares of the workgroup's work.  The
// numbering is a permutation of 0 .. waves-1 for any placement.
struct SimdRank {
    int simd, rank;
};

// counts: 4 ints of LDS.  Contains a barrier; the counts are final after the
// caller's next barrier.
__device__ __forceinline__ SimdRank simd_rank_begin(int *counts)
{
    if (threadIdx.x < 4) counts[threadIdx.x] = 0;
    __syncthreads();
    SimdRank r;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID, 4, 2)" : "=s"(r.simd));
    int v = 0;
    if ((threadIdx.x & 63) == 0) v = atomicAdd(&counts[r.simd], 1);
    r.rank = __shfl(v, 0);
    return r;
}

__device__ __forceinline__ int simd_share(const int *counts, SimdRank r)
{
    int before = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (q < r.simd) before += counts[q];
    return before + r.rank;
}

}  // namespace sgemm
