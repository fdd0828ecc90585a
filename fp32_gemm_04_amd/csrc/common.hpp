// Shared device-side pieces of the SGEMM kernels: argument block, vector
// type, and the workgroup -> output-tile mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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

// Stream-K.  When the output tiles do not fill whole rounds of resident
// workgroups, the work is cut finer: a unit is one BK-deep k-iteration of one
// tile, units are numbered tile by tile, and `workers` resident workgroups
// take equal contiguous ranges of them, [w U / W, (w+1) U / W).  A worker's
// range covers whole tiles, written to C as usual, plus at most a partial
// tile at each end.  A partial tile's raw sum goes to the workspace, slot
// 2 w for the worker's first segment and 2 w + 1 for its last; a second
// kernel (the fixup) then adds a split tile's partials in worker order and
// applies alpha and beta.  The result does not depend on timing, and no
// workgroup waits for another.
// Stream-K with whole rounds first: the tiles that fill whole rounds of the
// resident workgroups (dp_tiles, a multiple of workers) run one tile per
// workgroup, round-robin; only the tiles of the last, part-full round are
// cut into (tile, k-iteration) units and shared out, so only they leave
// partial sums for the fixup.
struct SkArgs {
    float *ws;       // 2 * sk_workers slots of BM * BN floats
    int64_t units;   // (tiles - dp_tiles) * iters: the shared units
    int iters;       // k-iterations per tile
    int bk;          // k per iteration
    int workers;     // resident workgroups (the grid)
    int dp_tiles;    // tiles run whole: tile r * workers + w for each round r
    int sk_workers;  // workers sharing the units (<= workers, <= units; 0 if none)
};

__host__ __device__ inline int64_t sk_begin(int64_t w, int64_t units, int workers)
{
    return w * units / workers;
}

// The worker whose range holds unit u.
__host__ __device__ inline int sk_worker_of(int64_t u, int64_t units, int workers)
{
    return (int)(((u + 1) * workers - 1) / units);
}

// Logical worker of workgroup bid: workgroups bid, bid + 8, ... run on one
// XCD and take adjacent ranges, so the tiles they share meet in its L2.
__device__ __forceinline__ int sk_logical_worker(int bid, int workers)
{
    const int q = workers / kNumXcd, r = workers % kNumXcd;
    const int x = bid % kNumXcd, i = bid / kNumXcd;
    return x * q + (x < r ? x : r) + i;
}

// Tile t of the grouped raster (group_m tile rows at a time).
__host__ __device__ inline void sk_tile(int t, int tiles_m, int tiles_n, int group_m, int &tm,
                                        int &tn)
{
    const int per_group = group_m * tiles_n;
    const int group = t / per_group;
    const int first_m = group * group_m;
    const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in_group = t - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// Runs this workgroup's share: its whole tiles, then its stream-K range,
// body(args, m0, n0) once per tile segment, with args narrowed to the
// segment's k-range and, for a partial tile, pointed at the workspace slot
// (row pitch BN, alpha 1, beta 0).
template <int BM, int BN, typename Body>
__device__ __forceinline__ void sk_run(const GemmArgs &g, const SkArgs &s, Body body)
{
    const int w = sk_logical_worker(blockIdx.x, s.workers);
    // Whole tiles: in round r the workgroups take tiles r W .. r W + W - 1,
    // so those one XCD runs at once are adjacent.
    for (int t = w; t < s.dp_tiles; t += s.workers) {
        int tm, tn;
        sk_tile(t, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
        body(g, tm * BM, tn * BN);
        __syncthreads();  // the next tile reuses the LDS buffers
    }
    if (w >= s.sk_workers) return;
    int64_t u = sk_begin(w, s.units, s.sk_workers);
    const int64_t u1 = sk_begin(w + 1, s.units, s.sk_workers);
    bool first = true;
    while (u < u1) {
        const int t = s.dp_tiles + (int)(u / s.iters);
        const int it0 = (int)(u - (int64_t)(t - s.dp_tiles) * s.iters);
        const int64_t left = u1 - u;
        const int it1 = left < (int64_t)(s.iters - it0) ? it0 + (int)left : s.iters;
        int tm, tn;
        sk_tile(t, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int k0 = it0 * s.bk;
        const int k1 = it1 * s.bk < g.K ? it1 * s.bk : g.K;
        GemmArgs a = g;
        a.A = g.A + k0;
        a.B = g.B + (int64_t)k0 * g.ldb;
        a.K = k1 - k0;
        if (it0 != 0 || it1 != s.iters) {
            // Element (m0 + r, n0 + c) of the tile lands at slot[r * BN + c].
            // Formed in integers: the shifted base itself lies outside the slot.
            const float *slot = s.ws + (int64_t)(2 * w + (first ? 0 : 1)) * (BM * BN);
            a.C = reinterpret_cast<float *>(reinterpret_cast<uintptr_t>(slot) -
                                            (uintptr_t)((int64_t)m0 * BN + n0) * sizeof(float));
            a.ldc = BN;
            a.alpha = 1.f;
            a.beta = 0.f;
        }
        body(a, m0, n0);
        __syncthreads();  // the next segment reuses the LDS buffers
        u += it1 - it0;
        first = false;
    }
}

// Host-side handles of the tile kernels: one output tile per workgroup, or a
// stream-K range per workgroup.
typedef void (*SkKernelFn)(GemmArgs, SkArgs);

// Direct-load MFMA kernel for a tile shape and waves-per-SIMD target, or
// null if none is built for it (defined in mfma_dl.hip); the stream-K form.
// shifted: the form for B rows that need not be 16-byte aligned (or null).
KernelFn direct_kernel(int bm, int bn, int wm, int wn, int wpe, bool shifted);
SkKernelFn direct_sk_kernel(int bm, int bn, int wm, int wn, int wpe, bool shifted);

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
