// libsgemm host side: argument checks, the shape-driven tile selector and
// kernel launches behind the C ABI declared in include/sgemm.h.
//
// Every kernel lives in the headers included below; this file only decides
// which one runs and with what grid.  sgemm_f32 and sgemm_f32_variant
// allocate, free, copy and synchronise nothing: work is queued on the
// caller's stream, and stream-K partial tiles go to a static device array
// (`scratch`).  Only sgemm_tune allocates (a scratch C) and synchronises.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/sgemm.h"
#include "common.hpp"
#include "mfma_tile.hpp"
#include "skinny.hpp"
#include "stream16.hpp"
#include "valu_tile.hpp"
#include "ladder.hpp"

namespace sgemm {

__device__ float g_stream_zero16[4] = {0.f, 0.f, 0.f, 0.f};

// Stream-K fixup.  Workgroup (x, y) handles elements [1024 y, 1024 (y+1))
// of output tile dp_tiles + x (the shared tiles only), four adjacent ones
// per thread (BN is a multiple of 4, so they share a row).  A tile whose
// units all fall to one worker was written in full and is skipped.  Otherwise its partial sums are added in worker
// order, from the slot each worker used (2 w if the tile was its first
// segment, 2 w + 1 if its last), and C is written as alpha * sum + beta * C
// (C not read when beta == 0).  The slot list (one 64-bit division per
// worker) is worked out once per workgroup, into LDS.
constexpr int kSkMaxWorkers = 1024;  // 256 CUs x 4 workgroups
constexpr int kSkFixupElems = 1024;  // elements per fixup workgroup

__global__ void __launch_bounds__(256) sk_fixup_kernel(GemmArgs g, SkArgs s, int bm, int bn)
{
    __shared__ int slot_of[kSkMaxWorkers];
    const int t = s.dp_tiles + blockIdx.x;
    const int e = (blockIdx.y * 256 + threadIdx.x) * 4;
    const int64_t ua = (int64_t)blockIdx.x * s.iters;
    const int wa = sk_worker_of(ua, s.units, s.sk_workers);
    const int wb = sk_worker_of(ua + s.iters - 1, s.units, s.sk_workers);
    if (wa == wb) return;
    const int nw = wb - wa + 1;
    for (int i = threadIdx.x; i < nw; i += blockDim.x) {
        const int w = wa + i;
        const int64_t b = sk_begin(w, s.units, s.sk_workers);
        slot_of[i] = 2 * w + (b >= ua ? 0 : 1);
    }
    __syncthreads();
    if (e >= bm * bn) return;
    int tm, tn;
    sk_tile(t, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    const int r = e / bn, c = e - r * bn;
    const int row = tm * bm + r, col = tn * bn + c;
    if (row >= g.M || col >= g.N) return;
    const int64_t slot_floats = (int64_t)bm * bn;
    float *pc = g.C + (int64_t)row * g.ldc + col;
    // C as one 128-bit access where the four columns exist and are aligned;
    // it is read (beta != 0) before the partials, so the two latencies overlap.
    const bool vec = col + 3 < g.N && (reinterpret_cast<uintptr_t>(pc) & 15u) == 0;
    f32x4 c_old = {0.f, 0.f, 0.f, 0.f};
    if (g.beta != 0.f) {
        if (vec) {
            c_old = *reinterpret_cast<const f32x4 *>(pc);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (col + q < g.N) c_old[q] = pc[q];
        }
    }
    // The partial sums, added in worker order; loaded four at a time, so
    // that a thread waits for one memory latency per four partials, not one
    // per partial (nw is the same for the whole workgroup).
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < nw; i += 4) {
        f32x4 part[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i + j < nw)
                part[j] = *reinterpret_cast<const f32x4 *>(s.ws + slot_of[i + j] * slot_floats + e);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i + j < nw) sum += part[j];
    }
    f32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[q] = g.alpha * sum[q];
        if (g.beta != 0.f) v[q] = fmaf(g.beta, c_old[q], v[q]);
    }
    if (vec) {
        *reinterpret_cast<f32x4 *>(pc) = v;
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (col + q < g.N) pc[q] = v[q];
    }
}

namespace {

// One entry of the tile table.
struct TileConfig {
    const char *family;  // "mfma" or "valu"
    int bm, bn, bk;      // workgroup tile and K slab
    int wm, wn;          // wave grid inside the workgroup
    int threads;         // workgroup size the kernel is compiled for
    int occupancy;       // workgroups that fit on one CU (LDS/registers)
    double efficiency;   // fraction of the CU's fp32 peak, register-staged path
    KernelFn fn[2][2];   // [A 128-bit loads][B 128-bit loads]
    KernelFn dl;         // direct-to-LDS variant (A rows 16-byte aligned, B rows too) or null
    double dl_efficiency;  // ... when the direct-load variant runs
    SkKernelFn sk_fn[2][2];  // stream-K forms of fn and dl
    SkKernelFn sk_dl;
    double one_efficiency;   // measured with one workgroup per CU (0: 0.85 x efficiency)
    KernelFn dls;            // direct-load forms for B rows of any alignment (or null)
    SkKernelFn sk_dls;
};

// How the operands allow slabs to be loaded straight into LDS: not at all
// (A rows not 16-byte aligned), with B rows 16-byte aligned, or with B rows
// at any 4-byte alignment (the shifted form).
enum DirectMode { kDirectNone = 0, kDirectAligned = 1, kDirectShifted = 2 };

KernelFn dl_of(const TileConfig &c, int dmode)
{
    return dmode == kDirectAligned ? c.dl : dmode == kDirectShifted ? c.dls : nullptr;
}

SkKernelFn sk_dl_of(const TileConfig &c, int dmode)
{
    return dmode == kDirectAligned ? c.sk_dl : dmode == kDirectShifted ? c.sk_dls : nullptr;
}

// The direct-load stream-K kernels take K a multiple of 16 only.
int sk_dmode(int dmode, int K) { return K % 16 == 0 ? dmode : kDirectNone; }

// WPE (waves per SIMD) = OCC workgroups per CU x waves per workgroup / 4 SIMDs.
#define SGEMM_MFMA_WPE(WM, WN, OCC) ((OCC) * (WM) * (WN) / 4)
#define SGEMM_MFMA_KERNEL(BM, BN, BK, WM, WN, OCC, ST, AV, BV) \
    mfma_tile_kernel<BM, BN, BK, WM, WN, SGEMM_MFMA_WPE(WM, WN, OCC), ST, AV, BV>
#define SGEMM_MFMA_SK_KERNEL(BM, BN, BK, WM, WN, OCC, ST, AV, BV) \
    mfma_tile_sk_kernel<BM, BN, BK, WM, WN, SGEMM_MFMA_WPE(WM, WN, OCC), ST, AV, BV>
// ROCC: the occupancy the register-staged kernels are compiled for (the
// entry's own OCC unless its direct-load kernel holds more LDS).
#define SGEMM_MFMA_ENTRY_R(BM, BN, BK, WM, WN, OCC, ROCC, ST, EFF, DL, DLEFF, SKDL, ONE) \
    {"mfma", BM, BN, BK, WM, WN, WM * WN * 64, OCC, EFF,                                 \
     {{SGEMM_MFMA_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, false, false),                    \
       SGEMM_MFMA_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, false, true)},                    \
      {SGEMM_MFMA_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, true, false),                     \
       SGEMM_MFMA_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, true, true)}},                    \
     DL, DLEFF,                                                                          \
     {{SGEMM_MFMA_SK_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, false, false),                 \
       SGEMM_MFMA_SK_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, false, true)},                 \
      {SGEMM_MFMA_SK_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, true, false),                  \
       SGEMM_MFMA_SK_KERNEL(BM, BN, BK, WM, WN, ROCC, ST, true, true)}},                 \
     SKDL, ONE,                                                                          \
     direct_kernel(BM, BN, WM, WN, SGEMM_MFMA_WPE(WM, WN, OCC), true),                   \
     direct_sk_kernel(BM, BN, WM, WN, SGEMM_MFMA_WPE(WM, WN, OCC), true)}
#define SGEMM_MFMA_ENTRY(BM, BN, BK, WM, WN, OCC, ST, EFF, DL, DLEFF, SKDL, ONE) \
    SGEMM_MFMA_ENTRY_R(BM, BN, BK, WM, WN, OCC, OCC, ST, EFF, DL, DLEFF, SKDL, ONE)
#define SGEMM_DL_KERNEL(BM, BN, WM, WN, OCC) \
    direct_kernel(BM, BN, WM, WN, SGEMM_MFMA_WPE(WM, WN, OCC), false)
#define SGEMM_DL_SK_KERNEL(BM, BN, WM, WN, OCC) \
    direct_sk_kernel(BM, BN, WM, WN, SGEMM_MFMA_WPE(WM, WN, OCC), false)

// The MFMA tile table.  Occupancy (workgroups per CU) is what LDS and the
// register budget allow.  Efficiencies are the fractions of the CU's fp32
// peak measured with every CU holding `occupancy` workgroups (5120^3,
// 4096^3, 2048^3, the im2col mid shapes): register-staged path, then
// direct-load path.  The last column is the efficiency measured when each CU
// holds a single tile (2560^3, 2048^3, 1024^3): small tiles lose most there,
// with little work per tile to hide load latency behind.
// The 64 x 64 tile with a three-stage pipeline at two workgroups per CU is
// faster than the four-per-CU entry when a CU has one tile (1024^3: 27.6
// against 31.1 us), slower when it has several, which its lower efficiency
// encodes.  The entry after it is the 64 x 64 direct-load tile with a four-slab
// ring (one workgroup per CU; twelve slabs measured 6% slower, 1024^3: 24.3
// against 22.8 us) and with one tile per CU (1024^3: 22.8 against 27.6 us; 768^3: 18.1
// against 22.5).  Its register-staged kernels (the two-per-CU build) are
// only run when forced: its efficiency of 0 keeps the selector off them.
// The 128 x 128 direct-load tile with eight waves (two per SIMD, 64 x 32
// each) at one workgroup per CU serves a CU that holds a single tile or a
// stream-K share (2048^3: 133.5 against 138.7 us for the four-wave tile;
// stream-K at 1280^3: 49.4 against 52.1); with several tiles per CU it is
// slower (2304^3: 293 against 202 us), since no second workgroup overlaps a
// tile's fill and epilogue.  Its register-staged kernels are forced-only.
// The 192 x 128 direct-load tile (eight waves of 48 x 64, one workgroup per
// CU) is for M = 384-like shapes whose 128 x 128 tiles would leave a
// part-full round: (384,14161,1152) is 222 of them, one per CU, 111.8 us
// against 117.4 for the stream-K 128 x 128 plan (ldb 14164: 109.0 against
// 112.2); the 96 x 224 tile below now takes that shape.  Its
// register-staged kernels are forced-only too.
// The 96 x 96 direct-load tile (four waves of 48 x 48, two workgroups per
// CU) cuts 1536^3 into 256 tiles, one per CU, with no partial tiles to add
// up: 66.7 against 71.9 us for the stream-K 128 x 128 plan.  It also takes
// shapes whose 128 x 128 or 64 x 64 tiles fill the CUs worse: 3000^3 420.6
// against 502.6 us, (1536, 1536, 768) 39.4 against 49.0, 1600^3 82.3
// against 86.8.  Its efficiencies: 0.69 with one tile per CU (1536^3),
// 0.82-0.84 with two or three (2048^3 to 2560^3), entered as 0.80.  Its
// register-staged kernels are forced-only.
// The 64 x 32 tile (four waves of 32 x 16, two workgroups per CU) is for
// problems too small to fill the CUs with 64 x 64 tiles: twice the tiles,
// each half the work, 24-31% faster from 128^3 to 640^3 (512^3: 9.7 against
// 13.1 us; (333, 517, 259) on the register-staged path 11.6 against 16.9;
// (500, 501, 500) shifted 13.0 against 18.9).  Its efficiencies (0.355 with
// one tile per CU, 0.45 register-staged and 0.50 direct-load with more) keep
// it off 768^3 and up, where it is slower (1024^3: 23.8 against 22.9 us).
// The 96 x 224 direct-load tile (four waves of 48 x 112, one workgroup per
// CU) cuts (384, 14161, 1152) into 4 x 64 = 256 tiles, one per CU, where
// 192 x 128 makes 222 and leaves the busiest CU 15% above the mean: 101.4
// against 112.8 us with operands rotating through HBM, 118.0 against
// 121.3 back to back on one operand set.  Its one-tile efficiency is
// entered as 0.74 (scaled to the 192 x 128 entry's 0.82, which that shape
// measures at 0.755); 0.60 with more tiles per CU keeps it to the
// one-tile case.
// The 128 x 176 direct-load tile (four waves of 32 x 176, two workgroups per
// CU) gives (256, 43264, 1152) 492 tiles, at most two per CU, where 128 x
// 128 makes 676 and puts three on the busiest CU: 191.8 against 207.7 us.
// 176 = 11 x 16 allows no other wave split; at two waves per SIMD the
// kernel spills 36 bytes (four values reloaded once per loop trip).  At
// 3328^3 it lost to the stream-K plan (560 against 550 us): its efficiency
// of 0.83 is the lowest that still takes the first shape.
const TileConfig kMfmaTiles[] = {
    SGEMM_MFMA_ENTRY(160, 160, 16, 2, 2, 2, 3, 0.77, SGEMM_DL_KERNEL(160, 160, 2, 2, 2), 0.88,
                     SGEMM_DL_SK_KERNEL(160, 160, 2, 2, 2), 0.82),
    SGEMM_MFMA_ENTRY(128, 128, 16, 2, 2, 2, 3, 0.82, SGEMM_DL_KERNEL(128, 128, 2, 2, 2), 0.90,
                     SGEMM_DL_SK_KERNEL(128, 128, 2, 2, 2), 0.79),
    SGEMM_MFMA_ENTRY(64, 64, 32, 2, 2, 4, 2, 0.70, nullptr, 0.0, nullptr, 0.44),
    SGEMM_MFMA_ENTRY(32, 256, 32, 1, 4, 2, 2, 0.50, nullptr, 0.0, nullptr, 0.0),
    SGEMM_MFMA_ENTRY(64, 256, 16, 1, 4, 2, 3, 0.60, SGEMM_DL_KERNEL(64, 256, 1, 4, 2), 0.90,
                     SGEMM_DL_SK_KERNEL(64, 256, 1, 4, 2), 0.0),
    SGEMM_MFMA_ENTRY(64, 64, 32, 2, 2, 2, 3, 0.55, nullptr, 0.0, nullptr, 0.495),
    SGEMM_MFMA_ENTRY_R(64, 64, 32, 2, 2, 1, 2, 3, 0.0, SGEMM_DL_KERNEL(64, 64, 2, 2, 1), 0.60,
                       SGEMM_DL_SK_KERNEL(64, 64, 2, 2, 1), 0.56),
    SGEMM_MFMA_ENTRY_R(128, 128, 16, 2, 4, 1, 1, 3, 0.0, SGEMM_DL_KERNEL(128, 128, 2, 4, 1), 0.80,
                       SGEMM_DL_SK_KERNEL(128, 128, 2, 4, 1), 0.82),
    SGEMM_MFMA_ENTRY_R(192, 128, 16, 4, 2, 1, 1, 3, 0.0, SGEMM_DL_KERNEL(192, 128, 4, 2, 1), 0.80,
                       SGEMM_DL_SK_KERNEL(192, 128, 4, 2, 1), 0.82),
    SGEMM_MFMA_ENTRY(96, 96, 16, 2, 2, 2, 3, 0.0, SGEMM_DL_KERNEL(96, 96, 2, 2, 2), 0.80,
                     SGEMM_DL_SK_KERNEL(96, 96, 2, 2, 2), 0.69),
    SGEMM_MFMA_ENTRY(64, 32, 16, 2, 2, 2, 3, 0.45, SGEMM_DL_KERNEL(64, 32, 2, 2, 2), 0.50,
                     nullptr, 0.355),
    SGEMM_MFMA_ENTRY_R(96, 224, 16, 2, 2, 1, 1, 3, 0.0, SGEMM_DL_KERNEL(96, 224, 2, 2, 1), 0.60,
                       nullptr, 0.74),
    SGEMM_MFMA_ENTRY(128, 176, 16, 4, 1, 2, 3, 0.0, SGEMM_DL_KERNEL(128, 176, 4, 1, 2), 0.83,
                     nullptr, 0.0),
};

// The vector-FMA kernel's two tiles (both two workgroups per CU).
#define SGEMM_VALU_ENTRY(BT)                                                        \
    {"valu", BT, BT, 8, 2, 2, 256, 2, 0.45,                                         \
     {{valu_tile_kernel<false, false, BT>, valu_tile_kernel<false, true, BT>},      \
      {valu_tile_kernel<true, false, BT>, valu_tile_kernel<true, true, BT>}},       \
     nullptr, 0.0, {{nullptr, nullptr}, {nullptr, nullptr}}, nullptr, 0.0, nullptr, nullptr}
const TileConfig kValuTiles[] = {SGEMM_VALU_ENTRY(128), SGEMM_VALU_ENTRY(160)};

// The VALU tile that leaves the least work per resident workgroup: the 160
// tile where the 128 one would leave a part-empty last round (5120^3).
const TileConfig *valu_tile(int M, int N, int num_cus)
{
    const TileConfig *best = nullptr;
    double best_work = 0.0;
    for (const TileConfig &c : kValuTiles) {
        const int64_t tiles = ((int64_t)M + c.bm - 1) / c.bm * (((int64_t)N + c.bn - 1) / c.bn);
        const int64_t slots = (int64_t)num_cus * c.occupancy;
        const double work = (double)((tiles + slots - 1) / slots) * c.bm * c.bn;
        if (best == nullptr || work < best_work) {
            best = &c;
            best_work = work;
        }
    }
    return best;
}

constexpr double kHbmBytesPerCuCycle = 8.0e12 / (256 * 2.4e9);  // MI355X HBM share
constexpr double kFlopsPerCuCycle = 256.0;                      // fp32 MFMA per CU
// The shifted direct-load form against the aligned one, both run stream-K
// ((256,43265,1152) against (256,43264,1152): 212.5 against 201.2 us;
// (384,14161,1152) with ldb 14161 against 14164: 115.0 against 109.8 us).
constexpr double kShiftedEfficiency = 0.95;

double dl_efficiency(const TileConfig &c, int dmode)
{
    return c.dl_efficiency * (dmode == kDirectShifted ? kShiftedEfficiency : 1.0);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Rough time (in CU cycles) of running the problem with tile config c: the
// work of the most loaded CU (ceil(tiles / CUs) tiles; a partial tile costs
// a whole one) at the entry's efficiency (that of the register-staged path
// when partial tiles exist), lowered when a CU holds fewer
// workgroups than its occupancy (fewer waves to hide latency); never less
// than the time to move the operands through HBM once.  `dmode`: how the
// operands allow the direct-load path (DirectMode).
double estimate_cycles(const TileConfig &c, int M, int N, int K, int num_cus, int dmode)
{
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    const int64_t per_cu = ceil_div(tiles, num_cus);
    const bool dl = dl_of(c, dmode) != nullptr;
    const int bk = dl ? 16 : c.bk;
    // Partial tiles at the right or bottom edge cost a whole tile: the
    // direct-load kernels run them through the same body, the register-staged
    // ones through a masked copy of theirs.
    double eff = dl ? dl_efficiency(c, dmode) : c.efficiency;
    if (eff <= 0.0) return HUGE_VAL;  // only run when forced
    if (per_cu == 1 && c.one_efficiency > 0.0)
        eff = c.one_efficiency * (dl && dmode == kDirectShifted ? kShiftedEfficiency : 1.0);
    else if (per_cu < c.occupancy)
        eff *= 0.85;
    const double kpad = (double)ceil_div(K, bk) * bk;
    const double compute = (double)per_cu * 2.0 * c.bm * c.bn * kpad / (kFlopsPerCuCycle * eff);
    const double bytes = 4.0 * ((double)M * K + (double)K * N + (double)M * N);
    const double memory = bytes / (kHbmBytesPerCuCycle * num_cus);
    return compute > memory ? compute : memory;
}

// Tile rows per raster group: enough rows that the tiles one XCD holds at
// once (its 32 CUs times occupancy) form a roughly square patch.
int group_rows(const TileConfig &c, int tiles_m, int tiles_n, int num_cus)
{
    const int resident = (num_cus / kNumXcd > 0 ? num_cus / kNumXcd : 1) * c.occupancy;
    int gm = 1;
    while (gm * gm < resident) ++gm;
    if (gm > tiles_m) gm = tiles_m;
    (void)tiles_n;
    return gm > 0 ? gm : 1;
}

// Stream-K plan for tile config c (see common.hpp), with its estimated time.
struct SkPlan {
    bool use;
    SkArgs args;        // ws filled in at launch
    int split_tiles;    // tiles whose units span more than one worker
    int partials;       // partial tile segments written to the workspace
    size_t ws_bytes;    // 2 * workers * BM * BN floats
    double cycles;      // estimate, CU cycles
};

// Measured on MI355X (mid im2col shapes, 1024^3 to 4608^3): each worker
// pays about 4.5 units' time on top of its units (the pipeline fill and the
// partial-tile store of its segments: 6% at (256,43264,1152), 95 units per
// worker; 1% at 3840^3, 422), and the fixup pass moves its bytes at about
// 5.3 TB/s, plus a launch.  Stream-K is taken only when its estimate is 5%
// below the best one-tile-per-workgroup estimate.
constexpr double kSkWorkerOverheadUnits = 4.5;
constexpr double kSkFixupBytesPerCycle = 5.3e12 / 2.4e9;
constexpr double kSkFixupLaunchCycles = 7200.0;
constexpr double kSkMargin = 0.95;
// Below this (one tile per workgroup, estimated) the fixup launch costs more
// than stream-K saves (512^3 and 768^3 measured 9-25% slower with it).
constexpr double kSkMinCycles = 60000.0;

SkPlan plan_streamk(const TileConfig &c, int M, int N, int K, int num_cus, int dmode)
{
    SkPlan p = {};
    if (c.sk_fn[0][0] == nullptr || K <= 0 || M <= 0 || N <= 0) return p;
    dmode = sk_dmode(dmode, K);
    const bool dl = sk_dl_of(c, dmode) != nullptr;
    const int bk = dl ? 16 : c.bk;
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    const int iters = (int)ceil_div(K, bk);
    const int64_t all_units = tiles * iters;
    if (tiles > 0x7fffffff || all_units <= 0) return p;
    const int64_t slots = (int64_t)num_cus * c.occupancy;
    const int64_t cap = slots < kSkMaxWorkers ? slots : kSkMaxWorkers;
    const int workers = (int)(all_units < cap ? all_units : cap);
    // Whole rounds run one tile per workgroup; the rest is shared out.
    const int64_t dp_tiles = tiles / workers * workers;
    const int64_t units = (tiles - dp_tiles) * iters;
    const int sk_workers = (int)(units < workers ? units : workers);
    // Partial segments: a worker's first shared segment unless it starts a
    // tile and covers all of it; its last (if another) unless it ends a tile.
    // Split tiles: tiles holding a worker boundary.
    int partials = 0, split = 0;
    int64_t last_split = -1;
    for (int w = 0; w < sk_workers; ++w) {
        const int64_t b = sk_begin(w, units, sk_workers), e = sk_begin(w + 1, units, sk_workers);
        const int64_t first_end = (b / iters + 1) * iters;
        if (b % iters != 0 || e < first_end) ++partials;
        if (e > first_end && e % iters != 0) ++partials;
        if (w > 0 && b % iters != 0 && b / iters != last_split) {
            ++split;
            last_split = b / iters;
        }
    }
    p.args.ws = nullptr;
    p.args.units = units;
    p.args.iters = iters;
    p.args.bk = bk;
    p.args.workers = workers;
    p.args.dp_tiles = (int)dp_tiles;
    p.args.sk_workers = sk_workers;
    p.split_tiles = split;
    p.partials = partials;
    p.ws_bytes = (size_t)2 * sk_workers * c.bm * c.bn * sizeof(float);

    const double eff = dl ? dl_efficiency(c, dmode) : c.efficiency;
    if (eff <= 0.0) {  // only run when forced
        p.cycles = HUGE_VAL;
        return p;
    }
    const double unit_cycles = 2.0 * c.bm * c.bn * bk / (kFlopsPerCuCycle * eff);
    const double per_worker = (double)all_units / workers;
    const double compute =
        (double)all_units / num_cus * unit_cycles * (1.0 + kSkWorkerOverheadUnits / per_worker);
    const double bytes = 4.0 * ((double)M * K + (double)K * N + (double)M * N);
    const double memory = bytes / (kHbmBytesPerCuCycle * num_cus);
    // The fixup reads every partial and reads and writes C of the split tiles.
    const double fix_bytes = ((double)partials + 2.0 * split) * c.bm * c.bn * 4.0;
    const double fixup = split > 0 ? fix_bytes / kSkFixupBytesPerCycle + kSkFixupLaunchCycles : 0;
    p.cycles = (compute > memory ? compute : memory) + fixup;
    return p;
}

// Bytes of one stream-K workspace slot (see `scratch` below).
constexpr size_t kSkSlotBytes = (size_t)2 * 512 * 128 * 128 * sizeof(float);  // 64 MiB

// The kernel a call runs: a tile config, one tile per workgroup or stream-K.
struct Choice {
    const TileConfig *c;
    SkPlan sk;
};

// allow_sk false: no stream-K (a forced stream-K variant runs its tile one
// tile per workgroup).  The selector never takes a stream-K plan whose
// partial tiles would not fit a workspace slot.
Choice choose(int variant, int M, int N, int K, int num_cus, int dmode, bool allow_sk = true)
{
    Choice ch = {nullptr, {}};
    if (variant == SGEMM_VARIANT_VALU) {
        ch.c = valu_tile(M, N, num_cus);
        return ch;
    }
    if (variant >= SGEMM_VARIANT_STREAMK_TILE) {
        ch.c = &kMfmaTiles[variant - SGEMM_VARIANT_STREAMK_TILE];
        if (!allow_sk) return ch;
        ch.sk = plan_streamk(*ch.c, M, N, K, num_cus, dmode);
        ch.sk.use = ch.sk.args.workers > 0;
        return ch;
    }
    if (variant >= SGEMM_VARIANT_MFMA_TILE) {
        ch.c = &kMfmaTiles[variant - SGEMM_VARIANT_MFMA_TILE];
        return ch;
    }
    double best = 0.0;
    for (const TileConfig &c : kMfmaTiles) {
        const double dp = estimate_cycles(c, M, N, K, num_cus, dmode);
        if (ch.c == nullptr || dp < best) {
            ch = {&c, {}};
            best = dp;
        }
    }
    // Automatic stream-K only on the direct-load path: with unaligned
    // operands the register-staged segments run below the efficiency the
    // estimate assumes ((384, 14161, 1152) measured 4.5% slower with it).
    if (!allow_sk || sk_dmode(dmode, K) == kDirectNone || best < kSkMinCycles) return ch;
    for (const TileConfig &c : kMfmaTiles) {
        if (sk_dl_of(c, dmode) == nullptr) continue;
        SkPlan sp = plan_streamk(c, M, N, K, num_cus, dmode);
        if (sp.args.workers > 0 && sp.ws_bytes <= kSkSlotBytes && sp.cycles / kSkMargin < best) {
            sp.use = true;
            ch = {&c, sp};
            best = sp.cycles / kSkMargin;
        }
    }
    return ch;
}

// Stream-K partial tiles live in `scratch`, a device array that the HIP
// runtime places when it loads this code object and keeps until the process
// ends, one copy per device.  No call allocates, frees or synchronises for
// it.  The array is split into kSkSlots slots, each large enough for every
// stream-K plan the tile table makes on 256 CUs (2 x 512 workers x 128 x 128
// floats).  A slot belongs to one stream at a time: calls on that stream use
// it in stream order, and each use sets the slot's event to the completion
// of its last kernel.  A call on another stream may take a slot over only once that
// event has completed (hipEventQuery: no wait), so no queued or running work
// still reads it.  When every slot is busy on other streams, or the stream
// is being captured into a graph (a replay could run anywhere, at any time),
// the selector's choice runs without stream-K and a forced stream-K variant
// returns an error.  Nothing in a slot needs clearing: the fixup reads only
// partials that the same call's first kernel wrote.
constexpr int kSkSlots = 4;
constexpr int64_t kSkSlotFloats = (int64_t)(kSkSlotBytes / sizeof(float));
static __device__ __align__(256) float scratch[kSkSlots * kSkSlotFloats];

constexpr int kMaxDevices = 64;

struct SkSlot {
    bool owned;          // owner holds a stream
    hipStream_t owner;
    hipEvent_t done;     // recorded on owner after each use
};
struct SkPool {
    bool ready;          // set-up ran (successfully or not)
    hipError_t error;    // set-up status; slots are unusable unless hipSuccess
    float *base;         // this device's address of `scratch`
    SkSlot slot[kSkSlots];
};
std::mutex g_pool_mutex;
SkPool g_pool[kMaxDevices];

// Once per device, with that device current, under g_pool_mutex: find this
// device's copy of `scratch` and create the slots' events.  In host code the
// name `scratch` is only a stand-in for the symbol; kernels get `base`.
hipError_t pool_setup(int dev)
{
    SkPool &p = g_pool[dev];
    if (p.ready) return p.error;
    p.ready = true;
    p.base = nullptr;
    hipError_t e = hipGetSymbolAddress((void **)&p.base, HIP_SYMBOL(scratch));
    for (int i = 0; i < kSkSlots && e == hipSuccess; ++i) {
        p.slot[i].owned = false;
        e = hipEventCreateWithFlags(&p.slot[i].done, hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        p.base = nullptr;
    }
    p.error = e;
    return e;
}

// Whether work queued on `stream` is being captured into a graph.  A failed
// query counts as capturing.
bool stream_capturing(hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

// A slot for a stream-K call of `bytes` on `stream` (device dev), with
// g_pool_mutex held by the caller: the stream's own slot, else one whose
// last use has completed.  Returns 0 with *slot set, or the reason there is
// none (an SGEMM_ERR_* value).
int sk_slot(int dev, hipStream_t stream, size_t bytes, int *slot)
{
    if (bytes > kSkSlotBytes) return SGEMM_ERR_WORKSPACE;
    if (dev < 0 || dev >= kMaxDevices || pool_setup(dev) != hipSuccess) return SGEMM_ERR_NO_SLOT;
    if (stream_capturing(stream)) return SGEMM_ERR_CAPTURING;
    SkPool &p = g_pool[dev];
    for (int i = 0; i < kSkSlots; ++i)
        if (p.slot[i].owned && p.slot[i].owner == stream) {
            *slot = i;
            return 0;
        }
    for (int i = 0; i < kSkSlots; ++i) {
        bool idle = !p.slot[i].owned;
        if (!idle) {
            const hipError_t q = hipEventQuery(p.slot[i].done);
            if (q != hipSuccess && q != hipErrorNotReady) (void)hipGetLastError();
            idle = q == hipSuccess;
        }
        if (idle) {
            p.slot[i].owned = true;
            p.slot[i].owner = stream;
            *slot = i;
            return 0;
        }
    }
    return SGEMM_ERR_NO_SLOT;
}

// Argument checks of the C ABI (no HIP call).  Returns 0 or -p.
int check_args(int M, int N, int K, float alpha, const void *A, int lda, const void *B,
               int ldb, const void *C, int ldc, bool check_pointers)
{
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const bool reads_ab = alpha != 0.0f && K > 0 && M > 0 && N > 0;
    if (check_pointers && reads_ab && (A == nullptr || ((uintptr_t)A & 3u) != 0)) return -5;
    if (lda < (K > 1 ? K : 1)) return -6;
    if (check_pointers && reads_ab && (B == nullptr || ((uintptr_t)B & 3u) != 0)) return -7;
    if (ldb < (N > 1 ? N : 1)) return -8;
    if (check_pointers && M > 0 && N > 0 && (C == nullptr || ((uintptr_t)C & 3u) != 0))
        return -10;
    if (ldc < (N > 1 ? N : 1)) return -11;
    return 0;
}

constexpr int kNumMfmaTiles = (int)(sizeof(kMfmaTiles) / sizeof(kMfmaTiles[0]));
// The forced-tile variants must stay below the ladder's and the stream-K
// ones inside the values the variant field reserves for them.
static_assert(SGEMM_VARIANT_MFMA_TILE + kNumMfmaTiles <= SGEMM_VARIANT_LADDER,
              "MFMA tile variants would reach the ladder's values");
static_assert(SGEMM_VARIANT_LADDER + SGEMM_LADDER_RUNGS <= SGEMM_VARIANT_STREAMK_TILE,
              "ladder variants would reach the stream-K tile values");

bool is_ladder(int v)
{
    return v >= SGEMM_VARIANT_LADDER && v < SGEMM_VARIANT_LADDER + kLadderRungs;
}

bool valid_variant(int v)
{
    return v == SGEMM_VARIANT_AUTO || v == SGEMM_VARIANT_MFMA || v == SGEMM_VARIANT_VALU ||
           v == SGEMM_VARIANT_SKINNY ||
           (v >= SGEMM_VARIANT_MFMA_TILE && v < SGEMM_VARIANT_MFMA_TILE + kNumMfmaTiles) ||
           (v >= SGEMM_VARIANT_STREAMK_TILE && v < SGEMM_VARIANT_STREAMK_TILE + kNumMfmaTiles) ||
           is_ladder(v);
}

// The ladder rungs of ladder.hpp: name, output tile, threads per workgroup.
// Rung 7 is the VALU register-tile kernel.
struct LadderRung {
    const char *name;
    int tile_m, tile_n, threads;
};
const LadderRung kLadder[kLadderRungs] = {
    {"naive", 16, 16, 256},     {"coalesced", 4, 64, 256}, {"lds", 32, 32, 1024},
    {"tile1d", 64, 64, 512},    {"tile2d", 128, 128, 256}, {"regcache", 128, 128, 256},
    {"vec4", 128, 128, 256},    {"dbuf", 128, 128, 256},
};

// Launch rungs 0-6 (rung 7 goes through the VALU tile path).
int launch_ladder(int rung, GemmArgs g, bool avec, bool bvec, hipStream_t stream)
{
    const LadderRung &r = kLadder[rung];
    g.tiles_m = (int)ceil_div(g.M, r.tile_m);
    g.tiles_n = (int)ceil_div(g.N, r.tile_n);
    g.group_m = 1;
    const int64_t blocks = (int64_t)g.tiles_m * g.tiles_n;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
    KernelFn fn = nullptr;
    switch (rung) {
    case 0: fn = ladder_naive_kernel; break;
    case 1: fn = ladder_coalesced_kernel; break;
    case 2: fn = ladder_lds_kernel; break;
    case 3: fn = ladder_tile1d_kernel; break;
    case 4: fn = ladder_tile2d_kernel<false>; break;
    case 5: fn = ladder_tile2d_kernel<true>; break;
    default:
        fn = avec ? (bvec ? ladder_vec4_kernel<true, true> : ladder_vec4_kernel<true, false>)
                  : (bvec ? ladder_vec4_kernel<false, true> : ladder_vec4_kernel<false, false>);
        break;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(r.threads), 0, stream, g);
    return (int)hipGetLastError();
}

// Per-device compute-unit count, queried once per device.
std::atomic<int> g_num_cus[kMaxDevices];

hipError_t device_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_num_cus[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *cus = cached;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    if (dev >= 0 && dev < kMaxDevices) {
        // First call on this device: set up its stream-K workspace slots too
        // (a failure only keeps stream-K off on this device).
        {
            std::lock_guard<std::mutex> lock(g_pool_mutex);
            (void)pool_setup(dev);
        }
        g_num_cus[dev].store(n, std::memory_order_relaxed);
    }
    *cus = n;
    return hipSuccess;
}

bool is_vec_ok(const void *p, int ld) { return ((uintptr_t)p & 15u) == 0 && (ld & 3) == 0; }

// The skinny streaming kernel: waves per workgroup; per column-block count
// Q, waves per SIMD and k steps per chunk (a step is Q registers of B per
// lane; one chunk of loads is in flight while the previous chunk's MFMAs
// run).  A wave holds MB x Q = 4 accumulators of 32 x 32 whatever M is:
// Q = 4 (128-column strips) for M <= 32, Q = 2 (64-column strips) for
// M <= 64.  The pairs below were the fastest of a measured grid
// (2 or 3 waves per SIMD x 8 to 32 steps): the Q = 4 kernel spills at 3.
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyWpe4 = 2, kSkinnyKc4 = 8;
constexpr int kSkinnyWpe2 = 3, kSkinnyKc2 = 8;

int skinny_q(int M) { return M <= 32 ? 4 : 2; }
int skinny_kc(int M) { return M <= 32 ? kSkinnyKc4 : kSkinnyKc2; }

bool skinny_fits(int M, int K) { return M <= 64 && K <= kSkinnyMaxK; }

// The fast skinny kernel addresses B and C by 32-bit byte offsets from the
// matrix base and moves 128 bits at a time.
bool skinny_fast_ok(int M, int N, int K, const void *B, int ldb, const void *C, int ldc)
{
    const int q = skinny_q(M);
    const int64_t b_bytes = ((int64_t)K * ldb + N) * 4;
    const int64_t c_bytes = ((int64_t)M * ldc + N) * 4;
    const bool aligned = ((uintptr_t)B % (4 * q)) == 0 && ((uintptr_t)C % (4 * q)) == 0 &&
                         ldb % q == 0 && ldc % q == 0;
    return aligned && b_bytes < (1ll << 32) && c_bytes < (1ll << 32);
}

// Shape-driven choice: the streaming kernel when A is small and there are
// enough 128-column strips to give every wave of the chip several.
bool use_skinny(int variant, int M, int N, int K, int num_cus)
{
    if (variant == SGEMM_VARIANT_SKINNY) return true;
    if (variant != SGEMM_VARIANT_AUTO) return false;
    const int64_t strips = ((int64_t)N + 32 * skinny_q(M) - 1) / (32 * skinny_q(M));
    return skinny_fits(M, K) && strips >= (int64_t)num_cus * 8;
}

// The 16x16x4 streaming kernel takes the HBM-bound skinny shapes (M <= 32)
// whose B and C rows are 16-byte aligned and whose N is a multiple of its
// 64-column strip; the other skinny shapes run skinny_kernel.
constexpr int kStreamWpe = 2;  // waves per SIMD (four-wave workgroups)

bool stream16_ok(int M, int N, int K, const void *B, int ldb, const void *C, int ldc)
{
    return M <= 32 && K <= kSkinnyMaxK && N % 64 == 0 && is_vec_ok(B, ldb) &&
           is_vec_ok(C, ldc);
}

int stream16_grid(int N, int num_cus)
{
    const int nstrip = N / 64;
    const int slots = num_cus * kStreamWpe;
    return nstrip < slots ? nstrip : slots;
}

template <int FM>
int launch_stream16(const GemmArgs &g, int num_cus, hipStream_t stream)
{
    const size_t lds = (size_t)16 * FM * stream_pitch(g.K) * sizeof(float);
    hipLaunchKernelGGL((stream16_kernel<FM, 8, 4, kStreamWpe>), dim3(stream16_grid(g.N, num_cus)),
                       dim3(256), lds, stream, g, 0, g.N / 64);
    return (int)hipGetLastError();
}

struct SkinnyLaunch {
    int begin, end, blocks;
};

struct SkinnyPlan {
    int mb, q, kh, pitch, lds_bytes;
    SkinnyLaunch fast, masked;  // strips for each kernel (empty if begin == end)
};

// Strips [begin, end) over a grid that stays resident: at most as many
// workgroups as fit on the chip at once (wpe waves per SIMD), so the copy of
// A into LDS is paid once per workgroup; the kernel gives each wave a
// contiguous share.
SkinnyLaunch skinny_split(int begin, int end, int wpe, int num_cus)
{
    SkinnyLaunch l;
    l.begin = begin;
    l.end = end;
    const int64_t strips = end - begin;
    const int64_t resident_blocks = (int64_t)num_cus * 4 * wpe / kSkinnyWaves;
    int64_t blocks = (strips + kSkinnyWaves - 1) / kSkinnyWaves;
    if (blocks > resident_blocks) blocks = resident_blocks;
    l.blocks = (int)(blocks > 0 ? blocks : 1);
    return l;
}

SkinnyPlan plan_skinny(int M, int N, int K, bool fast, int num_cus)
{
    SkinnyPlan p;
    p.mb = M <= 32 ? 1 : 2;
    p.q = skinny_q(M);
    p.kh = (K + 1) / 2;
    p.pitch = skinny_pitch(p.kh, skinny_kc(M));
    p.lds_bytes = 2 * p.mb * 32 * p.pitch * (int)sizeof(float);
    const int strip = 32 * p.q;
    const int nstrips = (int)(((int64_t)N + strip - 1) / strip);
    const int nfull = fast ? N / strip : 0;
    const int wpe = p.q == 4 ? kSkinnyWpe4 : kSkinnyWpe2;
    // The fast kernel: one workgroup of 4 wpe waves per CU.
    p.fast.begin = 0;
    p.fast.end = nfull;
    p.fast.blocks = nfull < num_cus ? (nfull > 0 ? nfull : 1) : num_cus;
    p.masked = skinny_split(nfull, nstrips, wpe, num_cus);
    return p;
}

template <int MB, int Q, int WPE, int KC>
int launch_skinny(const GemmArgs &g, const SkinnyPlan &p, hipStream_t stream)
{
    const dim3 block(kSkinnyWaves * 64);
    if (p.fast.end > p.fast.begin)
        hipLaunchKernelGGL((skinny_kernel<MB, Q, 4 * WPE, WPE, KC, true>), dim3(p.fast.blocks),
                           dim3(4 * WPE * 64), p.lds_bytes, stream, g, p.kh, p.pitch,
                           p.fast.begin, p.fast.end);
    if (p.masked.end > p.masked.begin)
        hipLaunchKernelGGL((skinny_kernel<MB, Q, kSkinnyWaves, WPE, KC, false>),
                           dim3(p.masked.blocks), block, p.lds_bytes, stream, g, p.kh, p.pitch,
                           p.masked.begin, p.masked.end);
    return (int)hipGetLastError();
}



// Tuned choices (sgemm_tune): the variant measured fastest for a problem
// key.  Looked up by AUTO calls while the table is not empty.
struct TuneKey {
    int device, M, N, K, lda, ldb, ldc, vec;  // vec: bit 0 A, bit 1 B, bit 2 C 128-bit paths
    bool operator==(const TuneKey &o) const
    {
        return device == o.device && M == o.M && N == o.N && K == o.K && lda == o.lda &&
               ldb == o.ldb && ldc == o.ldc && vec == o.vec;
    }
};
struct TuneEntry {
    TuneKey key;
    int variant;
};
std::mutex g_tune_mutex;
std::vector<TuneEntry> g_tuned;
std::atomic<int> g_tuned_count{0};

TuneKey tune_key(int device, int M, int N, int K, int lda, int ldb, int ldc, bool avec,
                 bool bvec, bool cvec)
{
    return {device, M, N, K, lda, ldb, ldc, (avec ? 1 : 0) | (bvec ? 2 : 0) | (cvec ? 4 : 0)};
}

// The tuned variant for key, or SGEMM_VARIANT_AUTO.
int tuned_variant(const TuneKey &key)
{
    if (g_tuned_count.load(std::memory_order_acquire) == 0) return SGEMM_VARIANT_AUTO;
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    for (const TuneEntry &e : g_tuned)
        if (e.key == key) return e.variant;
    return SGEMM_VARIANT_AUTO;
}

void record_tuned(const TuneKey &key, int variant)
{
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    for (TuneEntry &e : g_tuned)
        if (e.key == key) {
            e.variant = variant;
            return;
        }
    g_tuned.push_back({key, variant});
    g_tuned_count.store((int)g_tuned.size(), std::memory_order_release);
}

// The stream-K kernel and, when tiles are split, the fixup, on `stream`;
// partial tiles go to slot `slot` of `pool` (none when no units are shared),
// whose event then marks the completion of the last of them.  The caller
// holds g_pool_mutex when a slot is passed.
int launch_streamk(const Choice &ch, GemmArgs g, int cus, int dmode, bool avec, bool bvec,
                   hipStream_t stream, SkPool *pool, int slot)
{
    const TileConfig *c = ch.c;
    g.tiles_m = (int)ceil_div(g.M, c->bm);
    g.tiles_n = (int)ceil_div(g.N, c->bn);
    g.group_m = group_rows(*c, g.tiles_m, g.tiles_n, cus);
    const int64_t blocks = (int64_t)g.tiles_m * g.tiles_n;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
    SkArgs sa = ch.sk.args;
    sa.ws = pool != nullptr ? pool->base + (int64_t)slot * kSkSlotFloats : nullptr;
    const SkKernelFn dfn = sk_dl_of(*c, sk_dmode(dmode, g.K));
    const SkKernelFn fn = dfn ? dfn : c->sk_fn[avec][bvec];
    // The slot's event is the completion event of the call's last kernel,
    // attached to that kernel's dispatch: a separate event record costs a
    // queue entry of its own (measured: 3 us more per call at 1280^3-1792^3,
    // against 1-2 us for the attached form).
    // (A plan without a slot, which may run under graph capture, uses plain
    // launches.)
    hipEvent_t done = pool != nullptr ? pool->slot[slot].done : nullptr;
    const bool fixup = ch.sk.split_tiles > 0;
    const dim3 main_grid((unsigned)sa.workers), main_block(c->threads);
    if (done != nullptr && !fixup)
        hipExtLaunchKernelGGL(fn, main_grid, main_block, 0, stream, nullptr, done, 0, g, sa);
    else
        hipLaunchKernelGGL(fn, main_grid, main_block, 0, stream, g, sa);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && fixup) {
        const dim3 fix_grid((unsigned)(blocks - sa.dp_tiles),
                            (unsigned)ceil_div(c->bm * c->bn, kSkFixupElems));
        if (done != nullptr)
            hipExtLaunchKernelGGL(sk_fixup_kernel, fix_grid, dim3(256), 0, stream, nullptr, done,
                                  0, g, sa, c->bm, c->bn);
        else
            hipLaunchKernelGGL(sk_fixup_kernel, fix_grid, dim3(256), 0, stream, g, sa, c->bm,
                               c->bn);
        e = hipGetLastError();
        // The first kernel is queued: the slot's event must follow it.
        if (e != hipSuccess && done != nullptr) (void)hipEventRecord(done, stream);
    }
    return (int)e;
}

// use_tuned: an AUTO call takes the tuned variant of its key if there is one.
int launch(int variant, int M, int N, int K, float alpha, const float *A, int lda,
           const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream,
           bool use_tuned = true)
{
    if (!valid_variant(variant)) return SGEMM_ERR_BAD_VARIANT;
    const int bad = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc, true);
    if (bad != 0) return bad;
    if (M == 0 || N == 0) return 0;
    bool from_tuned = false;
    if (use_tuned && variant == SGEMM_VARIANT_AUTO &&
        g_tuned_count.load(std::memory_order_acquire) > 0 && K > 0 && alpha != 0.0f) {
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess)
            variant = tuned_variant(tune_key(dev, M, N, K, lda, ldb, ldc, is_vec_ok(A, lda),
                                             is_vec_ok(B, ldb), is_vec_ok(C, ldc)));
        from_tuned = variant != SGEMM_VARIANT_AUTO;
    }

    if (K == 0 || alpha == 0.0f) {
        const int64_t total = (int64_t)M * N;
        int64_t blocks = ceil_div(total, 256);
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(scale_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C,
                           (int64_t)ldc, M, N, beta);
        return (int)hipGetLastError();
    }

    if (variant == SGEMM_VARIANT_SKINNY && !skinny_fits(M, K)) return SGEMM_ERR_VARIANT_SHAPE;

    int cus = 0;
    const hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return (int)e;

    GemmArgs g;
    g.A = A;
    g.B = B;
    g.C = C;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = ldc;
    g.M = M;
    g.N = N;
    g.K = K;
    g.alpha = alpha;
    g.beta = beta;

    if (use_skinny(variant, M, N, K, cus) && stream16_ok(M, N, K, B, ldb, C, ldc)) {
        g.tiles_m = g.tiles_n = g.group_m = 1;
        return M <= 16 ? launch_stream16<1>(g, cus, stream) : launch_stream16<2>(g, cus, stream);
    }

    if (use_skinny(variant, M, N, K, cus)) {
        const bool fast = skinny_fast_ok(M, N, K, B, ldb, C, ldc);
        const SkinnyPlan p = plan_skinny(M, N, K, fast, cus);
        g.tiles_m = g.tiles_n = g.group_m = 1;
        return p.mb == 1 ? launch_skinny<1, 4, kSkinnyWpe4, kSkinnyKc4>(g, p, stream)
                         : launch_skinny<2, 2, kSkinnyWpe2, kSkinnyKc2>(g, p, stream);
    }

    const bool avec = is_vec_ok(A, lda), bvec = is_vec_ok(B, ldb);
    if (is_ladder(variant)) {
        const int rung = variant - SGEMM_VARIANT_LADDER;
        if (rung < kLadderRungs - 1) return launch_ladder(rung, g, avec, bvec, stream);
        variant = SGEMM_VARIANT_VALU;
    }
    const int dmode = avec ? (bvec ? kDirectAligned : kDirectShifted) : kDirectNone;
    // A forced stream-K variant reports why it cannot have a workspace slot;
    // the selector's choice (or a tuned one) then runs without stream-K.
    const bool force_sk = variant >= SGEMM_VARIANT_STREAMK_TILE && !from_tuned;
    Choice ch = choose(variant, M, N, K, cus, dmode);
    if (ch.sk.use) {
        std::unique_lock<std::mutex> lock(g_pool_mutex, std::defer_lock);
        int slot = -1, why = 0;
        int dev = 0;
        if (ch.sk.ws_bytes > 0) {  // no shared units (whole rounds only): no workspace
            lock.lock();
            const hipError_t de = hipGetDevice(&dev);
            if (de != hipSuccess) return (int)de;
            why = sk_slot(dev, stream, ch.sk.ws_bytes, &slot);
        }
        if (why == 0)
            return launch_streamk(ch, g, cus, dmode, avec, bvec, stream,
                                  slot >= 0 ? &g_pool[dev] : nullptr, slot);
        if (force_sk) return why;
        lock.unlock();
        ch = choose(variant, M, N, K, cus, dmode, false);
    }
    const TileConfig *c = ch.c;
    g.tiles_m = (int)ceil_div(M, c->bm);
    g.tiles_n = (int)ceil_div(N, c->bn);
    g.group_m = group_rows(*c, g.tiles_m, g.tiles_n, cus);
    const int64_t blocks = (int64_t)g.tiles_m * g.tiles_n;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
    const KernelFn dfn = dl_of(*c, dmode);
    const KernelFn fn = dfn ? dfn : c->fn[avec][bvec];
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(c->threads), 0, stream, g);
    return (int)hipGetLastError();
}

// Mean time per launch (us) of `reps` launches of variant, after one
// untimed launch; the launches write C (a scratch copy).  A variant that
// cannot run the problem returns its status and no time.
int time_variant(int variant, int M, int N, int K, float alpha, const float *A, int lda,
                 const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream,
                 int reps, hipEvent_t e0, hipEvent_t e1, float *us)
{
    int rc = launch(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, false);
    if (rc != 0) return rc;
    hipError_t e = hipEventRecord(e0, stream);
    for (int r = 0; r < reps && e == hipSuccess && rc == 0; ++r)
        rc = launch(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, false);
    if (rc != 0) return rc;
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e != hipSuccess) return (int)e;
    *us = ms * 1000.f / (float)reps;
    return 0;
}

int tune(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
         float beta, float *C, int ldc, hipStream_t stream, int reps, int *chosen, float *us)
{
    const int bad = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc, true);
    if (bad != 0) return bad;
    if (reps < 1) return -13;
    if (chosen) *chosen = SGEMM_VARIANT_AUTO;
    if (us) *us = 0.f;
    if (M == 0 || N == 0 || K == 0 || alpha == 0.0f)  // nothing to choose
        return launch(SGEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    // Scratch C with the same offset from a 16-byte boundary as C, so each
    // candidate takes the load and store paths it takes on C.
    const size_t c_floats = (size_t)(M - 1) * ldc + N;
    const size_t shift = ((uintptr_t)C & 15u);
    char *raw = nullptr;
    e = hipMalloc((void **)&raw, c_floats * sizeof(float) + 16);
    if (e != hipSuccess) return (int)e;
    float *scratch = reinterpret_cast<float *>(raw + shift);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    e = hipMemsetAsync(raw, 0, c_floats * sizeof(float) + 16, stream);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);

    int best = SGEMM_VARIANT_AUTO, first_error = 0;
    float best_us = 0.f;
    bool have = false;
    std::vector<int> candidates = {SGEMM_VARIANT_AUTO};
    if (skinny_fits(M, K)) candidates.push_back(SGEMM_VARIANT_SKINNY);
    for (int i = 0; i < kNumMfmaTiles; ++i) candidates.push_back(SGEMM_VARIANT_MFMA_TILE + i);
    for (int i = 0; i < kNumMfmaTiles; ++i) candidates.push_back(SGEMM_VARIANT_STREAMK_TILE + i);
    for (size_t i = 0; i < candidates.size() && e == hipSuccess; ++i) {
        float t = 0.f;
        const int rc = time_variant(candidates[i], M, N, K, alpha, A, lda, B, ldb, beta, scratch,
                                    ldc, stream, reps, e0, e1, &t);
        if (rc > 0) (void)hipGetLastError();  // a launch the device refused
        if (rc != 0) {
            if (first_error == 0) first_error = rc;
            continue;
        }
        if (!have || t < best_us) {
            best = candidates[i];
            best_us = t;
            have = true;
        }
    }
    const hipError_t se = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = se;
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    const hipError_t fe = hipFree(raw);
    if (e == hipSuccess) e = fe;
    if (e != hipSuccess) return (int)e;
    if (!have) return first_error;

    record_tuned(tune_key(dev, M, N, K, lda, ldb, ldc, is_vec_ok(A, lda), is_vec_ok(B, ldb),
                          is_vec_ok(C, ldc)),
                 best);
    if (chosen) *chosen = best;
    if (us) *us = best_us;
    return launch(best, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, false);
}

}  // namespace
}  // namespace sgemm

extern "C" int sgemm_f32(int M, int N, int K, float alpha, const float *A, int lda,
                         const float *B, int ldb, float beta, float *C, int ldc,
                         hipStream_t stream)
{
    return sgemm::launch(SGEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream);
}

extern "C" int sgemm_f32_variant(int variant, int M, int N, int K, float alpha,
                                 const float *A, int lda, const float *B, int ldb,
                                 float beta, float *C, int ldc, hipStream_t stream)
{
    return sgemm::launch(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

extern "C" int sgemm_plan(int variant, int M, int N, int K, int lda, int ldb, int ldc,
                          float alpha, int num_cus, char *buf, int buflen)
{
    using namespace sgemm;
    if (!valid_variant(variant)) return SGEMM_ERR_BAD_VARIANT;
    const int bad = check_args(M, N, K, alpha, nullptr, lda, nullptr, ldb, nullptr, ldc, false);
    if (bad != 0) return bad;
    if (num_cus < 1 || (buf == nullptr && buflen > 0) || buflen < 0) return -12;
    // A tuned choice for this problem on the current device (bases assumed
    // 16-byte aligned); the table is empty unless sgemm_tune ran, and only
    // then is the HIP runtime asked for the device.
    int tuned = SGEMM_VARIANT_AUTO;
    if (variant == SGEMM_VARIANT_AUTO && g_tuned_count.load(std::memory_order_acquire) > 0 &&
        M > 0 && N > 0 && K > 0 && alpha != 0.0f) {
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess)
            tuned = tuned_variant(tune_key(dev, M, N, K, lda, ldb, ldc, (lda & 3) == 0,
                                           (ldb & 3) == 0, (ldc & 3) == 0));
        variant = tuned;
    }
    char text[160];
    if (M == 0 || N == 0) {
        std::snprintf(text, sizeof text, "none");
    } else if (K == 0 || alpha == 0.0f) {
        std::snprintf(text, sizeof text, "scale m=%d n=%d", M, N);
    } else if (variant == SGEMM_VARIANT_SKINNY && !skinny_fits(M, K)) {
        return SGEMM_ERR_VARIANT_SHAPE;
    } else if (use_skinny(variant, M, N, K, num_cus) &&
               stream16_ok(M, N, K, nullptr, ldb, nullptr, ldc)) {
        // Plans assume 16-byte aligned bases, as the description says.
        std::snprintf(text, sizeof text, "stream16 fm=%d strip=64 kc=8 strips=%d grid=%d",
                      M <= 16 ? 1 : 2, N / 64, stream16_grid(N, num_cus));
    } else if (use_skinny(variant, M, N, K, num_cus)) {
        // Plans assume 16-byte aligned bases, as the description says.
        const bool fast = skinny_fast_ok(M, N, K, nullptr, ldb, nullptr, ldc);
        const SkinnyPlan p = plan_skinny(M, N, K, fast, num_cus);
        std::snprintf(text, sizeof text,
                      "skinny mb=%d q=%d kc=%d kh=%d pitch=%d fast=%dx%d+%d masked=%dx%d+%d "
                      "lds=%d",
                      p.mb, p.q, skinny_kc(M), p.kh, p.pitch,
                      p.fast.blocks * (p.fast.end > p.fast.begin),
                      4 * (p.q == 4 ? kSkinnyWpe4 : kSkinnyWpe2), p.fast.end - p.fast.begin,
                      p.masked.blocks * (p.masked.end > p.masked.begin), kSkinnyWaves,
                      p.masked.end - p.masked.begin, p.lds_bytes);
    } else if (is_ladder(variant)) {
        const LadderRung &r = kLadder[variant - SGEMM_VARIANT_LADDER];
        std::snprintf(text, sizeof text, "ladder rung=%d name=%s tile=%dx%d threads=%d grid=%lld",
                      variant - SGEMM_VARIANT_LADDER, r.name, r.tile_m, r.tile_n, r.threads,
                      (long long)ceil_div(M, r.tile_m) * ceil_div(N, r.tile_n));
    } else {
        const int dmode = (lda & 3) == 0 ? ((ldb & 3) == 0 ? kDirectAligned : kDirectShifted)
                                         : kDirectNone;
        const Choice ch = choose(variant, M, N, K, num_cus, dmode);
        const TileConfig *c = ch.c;
        const int tiles_m = (int)ceil_div(M, c->bm);
        const int tiles_n = (int)ceil_div(N, c->bn);
        const SkPlan &sp = ch.sk;
        const bool dl = sp.use ? sk_dl_of(*c, sk_dmode(dmode, K)) != nullptr
                               : dl_of(*c, dmode) != nullptr;
        std::snprintf(text, sizeof text,
                      "%s bm=%d bn=%d bk=%d waves=%dx%d occ=%d vecA=%d vecB=%d grid=%lld "
                      "group=%d load=%s streamk=%d dp=%d split=%d ws=%zu",
                      c->family, c->bm, c->bn, dl ? 16 : c->bk, c->wm, c->wn, c->occupancy,
                      (lda & 3) == 0,
                      (ldb & 3) == 0, (long long)tiles_m * tiles_n,
                      group_rows(*c, tiles_m, tiles_n, num_cus),
                      !dl ? "regs" : dmode == kDirectShifted ? "shifted" : "direct",
                      sp.use ? sp.args.workers : 0, sp.use ? sp.args.dp_tiles : 0,
                      sp.use ? sp.split_tiles : 0, sp.use ? sp.ws_bytes : (size_t)0);
    }
    if (tuned != SGEMM_VARIANT_AUTO) {
        const size_t n = std::strlen(text);
        std::snprintf(text + n, sizeof text - n, " tuned=%d", tuned);
    }
    if (buflen > 0) {
        std::strncpy(buf, text, (size_t)buflen - 1);
        buf[buflen - 1] = '\0';
    }
    return 0;
}

extern "C" int sgemm_tune(int M, int N, int K, float alpha, const float *A, int lda,
                          const float *B, int ldb, float beta, float *C, int ldc,
                          hipStream_t stream, int reps, int *chosen, float *us)
{
    return sgemm::tune(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, reps, chosen, us);
}

extern "C" void sgemm_tune_reset(void)
{
    std::lock_guard<std::mutex> lock(sgemm::g_tune_mutex);
    sgemm::g_tuned.clear();
    sgemm::g_tuned_count.store(0, std::memory_order_release);
}

extern "C" int sgemm_num_mfma_tiles(void) { return sgemm::kNumMfmaTiles; }

extern "C" const char *sgemm_status_string(int status)
{
    switch (status) {
    case 0: return "success";
    case -1: return "invalid M (negative)";
    case -2: return "invalid N (negative)";
    case -3: return "invalid K (negative)";
    case -5: return "invalid A (NULL or not 4-byte aligned)";
    case -6: return "invalid lda (< max(1, K))";
    case -7: return "invalid B (NULL or not 4-byte aligned)";
    case -8: return "invalid ldb (< max(1, N))";
    case -10: return "invalid C (NULL or not 4-byte aligned)";
    case -11: return "invalid ldc (< max(1, N))";
    case -12: return "invalid plan arguments (num_cus < 1 or no buffer)";
    case -13: return "invalid reps (< 1)";
    case SGEMM_ERR_BAD_VARIANT: return "unknown kernel variant";
    case SGEMM_ERR_VARIANT_SHAPE: return "the forced kernel variant cannot run this shape";
    case SGEMM_ERR_WORKSPACE:
        return "stream-K partial tiles would not fit a workspace slot of the library";
    case SGEMM_ERR_NO_SLOT:
        return "every stream-K workspace slot of the device is busy with other streams' work";
    case SGEMM_ERR_CAPTURING: return "stream-K is not run on a stream being captured into a graph";
    default: break;
    }
    if (status > 0) return hipGetErrorString((hipError_t)status);
    return "unknown status";
}
