// Streaming kernel for skinny products: M <= 64 rows, small K (<= 240),
// very many columns N -- the im2col convolution shapes of the
// UNIVERSAL_SGEMM_CUDA README ("Results" section: (32, 1605632, 27),
// (64, 1605632, 147), (64, 559104, 147)).  There the whole of A is a few
// tens of KB while B and C are hundreds of MB, so the product is bound by
// HBM (or sits at the ridge between HBM and the matrix cores), and the
// kernel is built to move every byte of B and C through HBM exactly once,
// with wide accesses and many of them in flight:
//
//   * A is copied once per workgroup into LDS and stays there.
//   * Each wave owns strips of 32*Q columns of C and computes all M rows of
//     a strip with v_mfma_f32_32x32x2_f32: MB 32-row blocks times Q column
//     blocks, one 16-float accumulator each per lane (MB*Q = 4 keeps the
//     accumulators at 64 registers: Q = 4 for M <= 32, Q = 2 for M <= 64).
//   * Column block q of a strip holds the columns n0 + Q*j + q
//     (j = 0..31): with that interleaving one Q-wide load of B[k][n0+Q*j ..]
//     by lane j gives the B operand of all Q column blocks, so B comes
//     straight from HBM into registers in 32*Q*4-byte row segments per
//     half-wave, with no LDS round trip and no barrier in the loop; and the
//     Q accumulators of a lane hold Q adjacent columns, so C is written with
//     Q-wide stores.  B is read with non-temporal loads (each element is
//     used by one wave only), which measured faster than caching it, and C
//     is written with non-temporal stores: plain ones leave dirty C in the
//     memory-side cache for the next launch to write back (back to back on
//     (64, 1605632, 147): 315.5 against 308.0 us a launch).
//   * The k index is split between the half-waves: lane group h = l/32
//     takes k = h*kh + s at step s (kh = ceil(K/2)).  The contraction is
//     order-free, and this makes a lane's A values for consecutive steps
//     contiguous in LDS, so one 128-bit LDS read feeds four steps.
//   * B is fetched in chunks of KC steps, the next chunk's loads issued
//     before the current chunk's MFMAs (register double buffer).
//
// MFMA layout (v_mfma_f32_32x32x2_f32, lane l): A operand A[l%32][k = l/32],
// B operand B[k = l/32][l%32], D[8*(r/4) + 4*(l/32) + r%4][l%32], r = 0..15.
//
// LDS layout of A (floats): As[h][row][s] = A[row][h*kh + s] (0 outside A),
// row pitch SAK (kh rounded up to the chunk size, SAK/4 odd so that 16
// consecutive rows fall on distinct bank groups for 128-bit reads).
#pragma once

#include "common.hpp"

namespace sgemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSkinnyMaxK = 240;  // keeps the A copy within 64 KB of LDS

// Row pitch (floats) of the LDS copy of A for a given kh = ceil(K/2) and
// chunk size kc.
__host__ __device__ inline int skinny_pitch(int kh, int kc)
{
    int p = (kh + kc - 1) / kc * kc;
    if ((p / 4) % 2 == 0) p += 4;
    return p;
}

// acc += A(:, steps c .. c+STEPS) x b, for the MB row blocks and Q column
// blocks (STEPS <= KC, a multiple of 4).  Steps past the end of K carry
// zeros in both A (LDS padding) and b, so a last chunk may run whole.
template <int MB, int Q, int KC, int STEPS, typename VQ>
__device__ __forceinline__ void skinny_mma(f32x16 (&acc)[MB][Q], const VQ (&b)[KC],
                                           const float *a_lane, int sak, int c)
{
    static_assert(STEPS % 4 == 0 && STEPS <= KC, "bad step count");
    // A for 4 steps per row block is one 128-bit LDS read; the next group's
    // reads are issued before the current group's MFMAs.
    f32x4 a4[2][MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        a4[0][mb] = *reinterpret_cast<const f32x4 *>(a_lane + mb * 32 * sak + c);
#pragma unroll
    for (int i = 0; i < STEPS / 4; ++i) {
        if (i + 1 < STEPS / 4) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                a4[(i + 1) & 1][mb] =
                    *reinterpret_cast<const f32x4 *>(a_lane + mb * 32 * sak + c + 4 * (i + 1));
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    acc[mb][q] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        a4[i & 1][mb][s], b[4 * i + s][q], acc[mb][q], 0, 0, 0);
    }
}

// As skinny_mma for the last chunk, which holds cnt <= KC valid steps: the
// A operands are read in groups of 4 steps and the MFMAs of steps at or past
// cnt are skipped (cnt is the same for the whole wave, so these are
// branches, not masks; with K = 147 the last chunk holds 2 of its 8 steps).
template <int MB, int Q, int KC, typename VQ>
__device__ __forceinline__ void skinny_mma_tail(f32x16 (&acc)[MB][Q], const VQ (&b)[KC],
                                                const float *a_lane, int sak, int c, int cnt)
{
#pragma unroll
    for (int i = 0; i < KC / 4; ++i) {
        if (4 * i < cnt) {
            f32x4 a4[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                a4[mb] = *reinterpret_cast<const f32x4 *>(a_lane + mb * 32 * sak + c + 4 * i);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (4 * i + s < cnt) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int q = 0; q < Q; ++q)
                            acc[mb][q] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                a4[mb][s], b[4 * i + s][q], acc[mb][q], 0, 0, 0);
                }
        }
    }
}

// Q floats of B at byte offset off from base (both 4Q-byte aligned),
// non-temporal, issued by inline assembly so that the compiler does not
// count it: the FAST path waits for its loads itself (skinny_wait).
template <int Q, typename VQ>
__device__ __forceinline__ VQ skinny_load(const char *base, uint32_t off)
{
    VQ v;
    if constexpr (Q == 4)
        asm volatile("global_load_dwordx4 %0, %1, %2 nt" : "=v"(v) : "v"(off), "s"(base) : "memory");
    else
        asm volatile("global_load_dwordx2 %0, %1, %2 nt" : "=v"(v) : "v"(off), "s"(base) : "memory");
    return v;
}

// Wait until at most N vector memory operations of this wave are in
// flight; the registers of b count as written here, so nothing that reads
// them can be scheduled above the wait.
template <int N, typename VQ>
__device__ __forceinline__ void skinny_wait(VQ (&b)[8])
{
    asm volatile("s_waitcnt vmcnt(%8)"
                 : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]),
                   "+v"(b[6]), "+v"(b[7])
                 : "n"(N)
                 : "memory");
}

// MB: 32-row blocks of A (1 or 2); Q: column blocks per strip (strip width
// 32*Q).  WAVES per workgroup, WPE waves per SIMD the register budget must
// allow, KC k-steps per chunk (multiple of 4).  The grid is sized to stay
// resident (the A copy is paid once per workgroup) and covers strips
// [strip_begin, strip_end); each wave takes a contiguous range of them.
// FAST: every strip lies inside B and C, whose rows are aligned to the
// access width, and the byte offsets of B and C fit in 32 bits: all
// accesses are Q-wide, addressed from the (wave-uniform) matrix base.  It
// runs one workgroup of WAVES = 4 WPE waves per CU, the ranges balanced per
// SIMD.  Otherwise (the ragged last strip, unaligned operands) every access
// is masked, and wave w of W takes [w S / W, (w+1) S / W).
template <int MB, int Q, int WAVES, int WPE, int KC, bool FAST>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
skinny_kernel(GemmArgs g, int kh, int sak, int strip_begin, int strip_end)
{
    static_assert(KC % 4 == 0, "chunk must be a multiple of 4 steps");
    typedef float VQ __attribute__((ext_vector_type(Q)));
    extern __shared__ __attribute__((aligned(16))) float As[];
    constexpr int ROWS = MB * 32;
    constexpr int STRIP = 32 * Q;
    const int M = g.M, N = g.N, K = g.K;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    // FAST runs one workgroup per CU, WAVES = 4 WPE waves, with the strips
    // balanced per SIMD (simd_rank_begin).
    __shared__ int simd_waves[4];
    SimdRank sr = {0, 0};
    if constexpr (FAST) sr = simd_rank_begin(simd_waves);

    // 1. A -> LDS, split by k half; zero outside A and past kh.  Loads are
    // issued in batches of 16 independent ones per thread, so the copy costs
    // a few L2 round trips rather than one per element.
    {
        constexpr int NT = WAVES * 64;
        constexpr int BATCH = 16;
        const int total = 2 * ROWS * sak;
        for (int base = threadIdx.x; base < total; base += NT * BATCH) {
            float v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int idx = base + u * NT;
                const int r = idx / sak;
                const int s = idx - r * sak;
                const int h = r / ROWS;
                const int m = r - h * ROWS;
                const int k = h * kh + s;
                v[u] = (idx < total && m < M && s < kh && k < K) ? g.A[(int64_t)m * g.lda + k]
                                                                 : 0.f;
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u)
                if (base + u * NT < total) As[base + u * NT] = v[u];
        }
    }
    __syncthreads();

    const int j = lane & 31;    // column group of the strip / row of the A operand
    const int h = lane >> 5;    // which half of K this lane feeds
    const int k_lane = h * kh;  // first k of this lane's half
    const float *a_lane = As + (h * ROWS + j) * sak;
    // Chunks whose steps are all valid for both halves come first; the
    // last chunk (steps [kh_full, kh) and zero padding) is masked.
    const int kh_full = (kh - 1) / KC * KC;
    const int64_t ldb = g.ldb;
    const uint32_t ldb4 = (uint32_t)(ldb * 4);
    const char *bbase = reinterpret_cast<const char *>(g.B);
    const float alpha = g.alpha, beta = g.beta;

    const int64_t nstrip = strip_end - strip_begin;
    int s_first, s_last;
    if constexpr (FAST) {
        // Workgroup b takes strips [b S / G, (b+1) S / G), cut into WAVES
        // equal shares; with WPE waves on each SIMD holding adjacent shares,
        // each SIMD gets a quarter of the workgroup's strips (+-1).
        const int64_t t = simd_share(simd_waves, sr);
        const int64_t b0 = (int64_t)blockIdx.x * nstrip / gridDim.x;
        const int64_t nb = ((int64_t)blockIdx.x + 1) * nstrip / gridDim.x - b0;
        s_first = strip_begin + (int)(b0 + t * nb / WAVES);
        s_last = strip_begin + (int)(b0 + (t + 1) * nb / WAVES);
    } else {
        const int64_t nwaves = (int64_t)gridDim.x * WAVES;
        const int64_t w = (int64_t)blockIdx.x * WAVES + wave;
        s_first = strip_begin + (int)(w * nstrip / nwaves);
        s_last = strip_begin + (int)((w + 1) * nstrip / nwaves);
    }

    if constexpr (FAST) {
        // The wave's strips as one stream of K chunks (nck per strip; the
        // last chunk of a strip may hold steps past kh or rows past K: those
        // read a clamped row and are zeroed once loaded).  Chunks rotate
        // through three register sets, the loop unrolled by three so each set
        // is a compile-time choice: while chunk i is multiplied, chunks i+1
        // and i+2 are in flight, across strip boundaries too.  Chunk i:
        //   wait for its loads (chunk i+1 stays in flight), write the C of a
        //   strip finished by chunk i-1, issue chunk i+2, multiply.
        // The C stores then sit between chunk i+1's loads and chunk i+2's,
        // so the wait before chunk i+1 can leave chunk i+2 in flight (it may
        // also wait for those stores, issued a whole chunk earlier).  The
        // lambdas are forced inline: called with different register sets,
        // an out-of-line copy would put the sets in scratch memory.
        static_assert(KC == 8, "the explicit waits are written for chunks of 8 steps");
        const int nck = (kh + KC - 1) / KC;
        const int total = (s_last - s_first) * nck;
        if (total == 0) return;
        // The base of B in scalar registers (the loads' saddr operand).
        const uint64_t bb = (uint64_t)(uintptr_t)bbase;
        const char *bsc = reinterpret_cast<const char *>(
            ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bb >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bb));
        int sl = s_first, cl = 0;  // next chunk to load
        auto fetch = [&](VQ(&b)[KC]) __attribute__((always_inline)) {
            const uint32_t col = (uint32_t)(sl * STRIP + Q * j);
#pragma unroll
            for (int s = 0; s < KC; ++s) {
                int row = k_lane + cl * KC + s;
                row = row < K ? row : K - 1;
                b[s] = skinny_load<Q, VQ>(bsc, (uint32_t)row * ldb4 + col * 4u);
            }
            if (++cl == nck) {
                cl = 0;
                ++sl;
            }
        };
        f32x16 acc[MB][Q];
        auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mb][q][r] = 0.f;
        };
        clear();
        // C as a wave-uniform base plus 32-bit offsets: a lane's offset for
        // row block mb, accumulator register r is lane_off + rr * ldc4 with
        // rr = 32 mb + 8 (r / 4) + r % 4 a constant, so each store costs one
        // add and nothing per row is kept live across the loop (kept live,
        // those values are spilled, and reloading a spill waits for every
        // outstanding load, the prefetched chunks included).
        // (Global address space spelled out: a generic pointer would make
        // these flat stores, which also count against the LDS reads' waits.)
        typedef __attribute__((address_space(1))) char gchar;
        typedef __attribute__((address_space(1))) VQ gVQ;
        const uint64_t cb = (uint64_t)(uintptr_t)g.C;
        gchar *csc = (gchar *)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(cb >> 32))
                                << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)cb));
        const uint32_t ldc4 = (uint32_t)g.ldc * 4u;
        // Every row of the row blocks exists and C is not read: no masks.
        const bool plain = M == ROWS && beta == 0.f;
        auto store = [&](int strip) __attribute__((always_inline)) {
            const uint32_t lane_off =
                (uint32_t)(strip * STRIP + Q * j) * 4u + (uint32_t)(4 * h) * ldc4;
            if (plain) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const uint32_t rr = mb * 32 + 8 * (r / 4) + (r % 4);
                        VQ v;
#pragma unroll
                        for (int q = 0; q < Q; ++q) v[q] = alpha * acc[mb][q][r];
                        __builtin_nontemporal_store(v, (gVQ *)(csc + (lane_off + rr * ldc4)));
                    }
                return;
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = mb * 32 + 8 * (r / 4) + (r % 4);
                    if (rr + 4 * h >= M) continue;
                    VQ v;
#pragma unroll
                    for (int q = 0; q < Q; ++q) v[q] = alpha * acc[mb][q][r];
                    gVQ *pc = (gVQ *)(csc + (lane_off + (uint32_t)rr * ldc4));
                    if (beta != 0.f) {
                        const VQ old = *pc;
#pragma unroll
                        for (int q = 0; q < Q; ++q) v[q] = fmaf(beta, old[q], v[q]);
                    }
                    __builtin_nontemporal_store(v, pc);
                }
        };
        int sc = s_first, cc = 0;  // chunk being multiplied
        bool pending = false;
        auto run = [&](VQ(&cur)[KC], VQ(&after_next)[KC], int i) __attribute__((always_inline)) {
            if (i + 1 < total)
                skinny_wait<KC>(cur);
            else
                skinny_wait<0>(cur);
            if (pending) {
                store(sc - 1);
                clear();
                pending = false;
            }
            if (i + 2 < total) fetch(after_next);
            if (cc + 1 < nck) {
                skinny_mma<MB, Q, KC, KC>(acc, cur, a_lane, sak, cc * KC);
            } else {
                // Last chunk of the strip: zero the steps past kh or K.
#pragma unroll
                for (int s = 0; s < KC; ++s) {
                    const int step = cc * KC + s;
                    if (!(step < kh && k_lane + step < K)) {
#pragma unroll
                        for (int q = 0; q < Q; ++q) cur[s][q] = 0.f;
                    }
                }
                skinny_mma_tail<MB, Q, KC>(acc, cur, a_lane, sak, cc * KC, kh - cc * KC);
            }
            if (++cc == nck) {
                cc = 0;
                ++sc;
                pending = true;
            }
        };
        VQ b0[KC], b1[KC], b2[KC];
        fetch(b0);
        if (total > 1) fetch(b1);
        for (int i = 0; i < total; i += 3) {
            run(b0, b2, i);
            if (i + 1 < total) run(b1, b0, i + 1);
            if (i + 2 < total) run(b2, b1, i + 2);
        }
        if (pending) store(sc - 1);
        return;
    }

    for (int strip = s_first; strip < s_last; ++strip) {
        const int n = strip * STRIP + Q * j;  // this lane's first column

        // b[s] = B[k_lane + c + s][n .. n+Q-1], zero outside B; `masked`:
        // the steps may lie past kh or K.
        // FAST loads are never behind a branch: a step past kh or K reads a
        // clamped, valid row of B and is then replaced by zero, so the
        // compiler can count outstanding loads exactly.
        auto fill = [&](VQ(&b)[KC], int c, bool masked) {
#pragma unroll
            for (int s = 0; s < KC; ++s) {
                const bool k_ok = !masked || (c + s < kh && k_lane + c + s < K);
                VQ v;
#pragma unroll
                for (int q = 0; q < Q; ++q) v[q] = 0.f;
                if (FAST) {
                    int row = k_lane + c + s;
                    if (masked) row = row < K ? row : K - 1;
                    v = __builtin_nontemporal_load(reinterpret_cast<const VQ *>(
                        bbase + (uint32_t)(((int64_t)row * ldb + n) * 4)));
                    if (masked && !k_ok) {
#pragma unroll
                        for (int q = 0; q < Q; ++q) v[q] = 0.f;
                    }
                } else if (k_ok) {
                    const float *p = g.B + (int64_t)(k_lane + c + s) * ldb + n;
#pragma unroll
                    for (int q = 0; q < Q; ++q)
                        if (n + q < N) v[q] = p[q];
                }
                b[s] = v;
            }
        };

        f32x16 acc[MB][Q];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mb][q][r] = 0.f;

        // The loads of chunk c + KC are issued before the MFMAs of chunk c.
        // Inside the loop every load is unmasked, so no load sits behind a
        // branch and the wait before the MFMAs of chunk c covers only the
        // loads of chunk c.
        VQ bc[KC], bn[KC];
        if (kh_full > 0) {
            fill(bc, 0, false);
            int c = 0;
            for (; c + KC < kh_full; c += KC) {
                fill(bn, c + KC, false);
                // Keep the prefetch at the top of the loop body: without
                // this the scheduler sinks the loads next to their use in
                // the following iteration and nothing overlaps.
                __builtin_amdgcn_sched_barrier(0);
                skinny_mma<MB, Q, KC, KC>(acc, bc, a_lane, sak, c);
#pragma unroll
                for (int s = 0; s < KC; ++s) bc[s] = bn[s];
            }
            fill(bn, kh_full, true);
            __builtin_amdgcn_sched_barrier(0);
            skinny_mma<MB, Q, KC, KC>(acc, bc, a_lane, sak, c);
            skinny_mma_tail<MB, Q, KC>(acc, bn, a_lane, sak, kh_full, kh - kh_full);
        } else {
            fill(bc, 0, true);
            skinny_mma_tail<MB, Q, KC>(acc, bc, a_lane, sak, 0, kh);
        }

        // Epilogue: row r of block mb, columns n .. n+Q-1.
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = mb * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                if (row >= M) continue;
                VQ v;
#pragma unroll
                for (int q = 0; q < Q; ++q) v[q] = alpha * acc[mb][q][r];
                if (FAST) {
                    VQ *pc = reinterpret_cast<VQ *>(reinterpret_cast<char *>(g.C) +
                                                    (uint32_t)(((int64_t)row * g.ldc + n) * 4));
                    if (beta != 0.f) {
                        const VQ old = *pc;
#pragma unroll
                        for (int q = 0; q < Q; ++q) v[q] = fmaf(beta, old[q], v[q]);
                    }
                    __builtin_nontemporal_store(v, pc);
                } else {
                    float *pc = g.C + (int64_t)row * g.ldc + n;
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        if (n + q < N) {
                            float o = v[q];
                            if (beta != 0.f) o = fmaf(beta, pc[q], o);
                            pc[q] = o;
                        }
                    }
                }
            }
        }
    }
}

}  // namespace sgemm
