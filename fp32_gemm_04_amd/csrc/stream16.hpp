// Streaming kernel for short, wide products on v_mfma_f32_16x16x4_f32:
// M <= 16 FM rows, K <= 240, many columns (the im2col shapes of the
// UNIVERSAL_SGEMM_CUDA README, "Results" section).  All of A is a few tens
// of KB and stays in LDS; B and C cross HBM once, B straight into the
// registers that feed the matrix cores.  Used for M <= 32, where the
// product is bound by HBM (for 32 < M <= 64, which sits at the ridge
// between HBM and the matrix cores, skinny.hpp measured faster).
//
// Layout.  A wave owns strips of 64 columns and computes all M rows of a
// strip.  k is walked in steps of 4; at step t lane l (j = l % 16,
// g = l / 16) contributes k = 4t + g, so each lane loads one 16-byte
// B[4t + g][n0 + 4j .. n0 + 4j + 3] per step, and those four values are
// the B operands of four 16-column blocks: block f of the strip holds the
// columns n0 + 4j + f.  A K that is not a multiple of 16 costs at most one
// partial step, not a partial 16-wide chunk.
// The A operand of step t is A[16 fm + j][4t + g]; A is stored in LDS as
// As[row][16c + 4g + s] = A[row][16c + 4s + g] (c = t / 4, s = t % 4), so
// one 128-bit LDS read gives a lane its A values for four steps.  The row
// pitch is 8 mod 16 floats, which makes that read conflict-free.
// C: lane l holds rows 16 fm + 4g + i of column j in each block f, i.e. four
// adjacent columns n0 + 4j .. n0 + 4j + 3 per row: one 16-byte store each.
//
// Pipeline.  Steps are fetched in groups of KC into a ring of three register
// sets (set indices are compile-time constants: the loop is unrolled by
// three groups); while group q's MFMAs run, groups q+1 and q+2 are in
// flight, and the stream of groups runs on across strips.  Rows of B at or
// past K load from a 16-byte block of zeros, so no load needs a mask.
// The B loads are issued by inline assembly and waited for explicitly
// (s_waitcnt vmcnt(n) that leaves the younger groups in flight, written as
// an instruction that redefines the loaded registers, so no MFMA can be
// scheduled above it).  Left to the compiler, the C stores at the end of a
// strip, pending together with loads, would force it to wait for every
// outstanding load, the prefetch included: on gfx9 loads and stores share
// one counter and the compiler assumes they may complete out of order.
// Loads the compiler does not know about only make its own waits (for C
// reads when beta != 0) stricter.
// The grid stays resident; wave w of W takes the contiguous strip range
// [w S / W, (w+1) S / W).  Requires B and C rows 16-byte aligned and
// N % 64 == 0 (the host sends other shapes to skinny.hpp).
#pragma once

#include "common.hpp"

namespace sgemm {

// 16 bytes of zeros that loads of B rows past K read.
extern __device__ float g_stream_zero16[4];

// 16 bytes at p (16-byte aligned, global), non-temporal; not tracked by the
// compiler's wait counting: see stream_wait.
__device__ __forceinline__ f32x4 stream_load(const float *p)
{
    f32x4 v;
    asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(v) : "v"(p) : "memory");
    return v;
}

// Wait until at most N vector memory operations of this wave are in flight;
// the KC registers of b count as written here.
template <int N, int KC>
__device__ __forceinline__ void stream_wait(f32x4 (&b)[KC])
{
    static_assert(KC == 8, "written for groups of 8 steps");
    asm volatile("s_waitcnt vmcnt(%8)"
                 : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]),
                   "+v"(b[6]), "+v"(b[7])
                 : "n"(N)
                 : "memory");
}

// Row pitch (floats) of the LDS copy of A for K.
__host__ __device__ inline int stream_pitch(int K) { return (K + 15) / 16 * 16 + 8; }

template <int FM, int KC, int WAVES, int WPE>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
stream16_kernel(GemmArgs g, int strip_begin, int strip_end)
{
    static_assert(KC % 4 == 0, "a group covers whole 16-wide chunks of k");
    extern __shared__ __attribute__((aligned(16))) float As[];
    constexpr int ROWS = 16 * FM;
    const int M = g.M, K = g.K;
    const int pitch = stream_pitch(K);
    const int kpad = pitch - 8;  // K rounded up to 16

    // 1. A -> LDS in the step order above; zero outside A.  Batches of
    // independent loads per thread, so the copy costs a few L2 round trips.
    {
        constexpr int NT = WAVES * 64, BATCH = 8;
        const int total = ROWS * kpad;
        for (int base = threadIdx.x; base < total; base += NT * BATCH) {
            float v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int idx = base + u * NT;
                const int row = idx / kpad, kk = idx - row * kpad;
                const int k = (kk & ~15) + 4 * (kk & 3) + ((kk >> 2) & 3);
                v[u] = (idx < total && row < M && k < K) ? g.A[(int64_t)row * g.lda + k] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int idx = base + u * NT;
                if (idx < total) {
                    const int row = idx / kpad;
                    As[row * pitch + idx - row * kpad] = v[u];
                }
            }
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const float *a_lane = As + j * pitch + 4 * gq;
    const int T = (K + 3) / 4;            // k-steps per strip
    const int G = (T + KC - 1) / KC;      // groups per strip

    const int64_t nwaves = (int64_t)gridDim.x * WAVES;
    const int64_t w = (int64_t)blockIdx.x * WAVES + wave;
    const int64_t nstrip = strip_end - strip_begin;
    const int s_first = strip_begin + (int)(w * nstrip / nwaves);
    const int s_last = strip_begin + (int)((w + 1) * nstrip / nwaves);
    const int ngroup = (s_last - s_first) * G;
    if (ngroup == 0) return;

    // Load cursor: the next group to fetch is group gl of strip sl.
    int sl = s_first, gl = 0;
    const int64_t ldb = g.ldb;
    f32x4 bq[3][KC];
    auto fetch = [&](f32x4 (&b)[KC]) {
        const float *col = g.B + (int64_t)sl * 64 + 4 * j;
#pragma unroll
        for (int s = 0; s < KC; ++s) {
            const int row = 4 * (gl * KC + s) + gq;
            b[s] = stream_load(row < K ? col + row * ldb : g_stream_zero16);
        }
        if (++gl == G) {
            gl = 0;
            ++sl;
        }
    };

    f32x4 acc[FM][4];
    auto clear = [&]() {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[fm][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    clear();

    // MFMAs of group gc (steps gc*KC ...), operands in b; steps past T are
    // skipped in blocks of four (wave-uniform).
    auto compute = [&](const f32x4 (&b)[KC], int gc) {
#pragma unroll
        for (int q = 0; q < KC / 4; ++q) {
            const int t0 = gc * KC + 4 * q;
            if (t0 < T) {
                f32x4 af[FM];
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    af[fm] = *reinterpret_cast<const f32x4 *>(a_lane + fm * 16 * pitch + 4 * t0);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                        for (int f = 0; f < 4; ++f)
                            acc[fm][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                af[fm][s], b[4 * q + s][f], acc[fm][f], 0, 0, 0);
            }
        }
    };
    const float alpha = g.alpha, beta = g.beta;
    auto store = [&](int strip) {
        float *col = g.C + (int64_t)strip * 64 + 4 * j;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * fm + 4 * gq + i;
                if (row < M) {
                    f32x4 *p = reinterpret_cast<f32x4 *>(col + (int64_t)row * g.ldc);
                    f32x4 v = {alpha * acc[fm][0][i], alpha * acc[fm][1][i],
                               alpha * acc[fm][2][i], alpha * acc[fm][3][i]};
                    if (beta != 0.f) {
                        const f32x4 c = *p;
                        v.x = fmaf(beta, c.x, v.x);
                        v.y = fmaf(beta, c.y, v.y);
                        v.z = fmaf(beta, c.z, v.z);
                        v.w = fmaf(beta, c.w, v.w);
                    }
                    // Non-temporal: C is written once and not read back
                    // here.  Plain stores leave up to the memory-side
                    // cache's size of dirty C behind when the kernel ends,
                    // which the next launch pays for: back to back on
                    // (32, 1605632, 27) plain stores took 81.1 us a launch,
                    // these 79.5.
                    __builtin_nontemporal_store(v, p);
                }
            }
    };

    // Compute cursor: group gc of strip sc.  A finished strip's C is written
    // at the start of the next group, after that group's wait and before the
    // next fetch: the stores then sit between the group waited for and the
    // younger group in issue order, and a wait that counts loads only never
    // has to drain the prefetch (it may wait for the stores, which were
    // issued a whole group earlier).
    int sc = s_first, gc = 0;
    bool pending = false;
    auto flush = [&]() {
        if (pending) {
            store(sc - 1);
            clear();
            pending = false;
        }
    };
    // Group n: wait for its loads (the one group after it stays in flight),
    // write a finished strip, issue group n+2 into the set group n-1 used,
    // compute.
    auto run = [&](f32x4 (&cur)[KC], f32x4 (&after_next)[KC], int n) {
        if (n + 1 < ngroup)
            stream_wait<KC>(cur);
        else
            stream_wait<0>(cur);
        flush();
        if (n + 2 < ngroup) fetch(after_next);
        compute(cur, gc);
        if (++gc == G) {
            gc = 0;
            ++sc;
            pending = true;
        }
    };
    fetch(bq[0]);
    if (ngroup > 1) fetch(bq[1]);
    for (int n = 0; n < ngroup; n += 3) {
        run(bq[0], bq[2], n);
        if (n + 1 < ngroup) run(bq[1], bq[0], n + 1);
        if (n + 2 < ngroup) run(bq[2], bq[1], n + 2);
    }
    flush();
}

}  // namespace sgemm
