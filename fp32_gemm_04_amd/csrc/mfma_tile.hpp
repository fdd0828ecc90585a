// fp32 matrix-core (MFMA) tile kernel for gfx950.
//
// Prior art: the block-tiled kernels of the NVIDIA_SGEMM_PRACTICE README
// (kernels 2-7: shared-memory slabs, 2-D tiles per thread, 128-bit loads,
// double-buffered prefetch) and the "Advanced" kernel of the cnblogs
// matmul_opt.cu post (BM x BN x BK slabs, double buffer, one barrier per
// slab, zero-filled masked edge loads).  Those were written for NVIDIA SIMT
// cores; here the inner product runs on the CDNA matrix cores with
// v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate, no down-conversion) and
// each 64-lane wave owns a (BM/WM) x (BN/WN) sub-tile of the output.
//
// One workgroup computes one BM x BN tile of C:
//   1. K is walked in slabs of BK.  The A slab (BM x BK) and B slab
//      (BK x BN) are fetched from HBM with 128-bit loads (32-bit ones only
//      where a row ends inside the quad), zero-filled outside the matrix,
//      and kept in registers until the current slab's math is done
//      (prefetch).
//   2. They are written to one of two LDS buffers (ping-pong), so one
//      barrier per slab suffices: the buffer being written was last read
//      before the previous barrier.  The write is issued inside the slab's
//      MFMA sequence (after its first k-step), not after it.
//   3. Each wave reads its MFMA operands from LDS and issues FM x FN
//      independent 16x16x4 MFMAs per k-step into FM x FN accumulators.
//   4. Epilogue: C = alpha*acc + beta*C, with C not read when beta == 0,
//      stores masked to the M x N window.
// Workgroups whose tile lies wholly inside C take an unmasked copy of the
// loop (only a ragged last K slab is masked), with 128-bit loads even when
// rows are only 4-byte aligned; edge tiles take the fully masked copy.
//
// MFMA operand layout (v_mfma_f32_16x16x4_f32, 64 lanes, lane l):
//   A operand: one float, A[row = l%16][k = l/16]
//   B operand: one float, B[k = l/16][col = l%16]
//   D (4 floats): D[row = 4*(l/16) + i][col = l%16], i = 0..3
// The contraction index may be permuted freely as long as A and B agree, so
// within a 16-wide k chunk lane group g = l/16 takes k = 4g + s at step s.
// That makes a lane's four A values for steps s = 0..3 contiguous in an
// m-major LDS row: one 128-bit LDS read feeds four MFMAs.
//
// LDS layout (floats):
//   A slab: m-major, row pitch SA = BK + 4.  A 128-bit read by 16 lanes of
//           consecutive m starts at m*SA; SA = 4*odd spreads the 16 rows
//           over all 64 banks, so the read is conflict-free.
//   B slab: k-major, row pitch SB = BN + 4.  Lanes of group g read row
//           4g + s; the +4 shifts each group to its own 16 banks.
#pragma once

#include "common.hpp"

namespace sgemm {

// Four consecutive floats p[0..3] of one matrix row, zero where the row is
// out of range or a column is >= limit.  With VEC the caller guarantees that
// p is 16-byte aligned whenever col is a multiple of 4.
template <bool VEC>
__device__ __forceinline__ f32x4 load4_masked(const float *__restrict__ p, bool row_ok,
                                              int col, int limit)
{
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row_ok) {
        if (VEC && col + 3 < limit) {
            v = *reinterpret_cast<const f32x4 *>(p);
        } else {
            if (col < limit) v.x = p[0];
            if (col + 1 < limit) v.y = p[1];
            if (col + 2 < limit) v.z = p[2];
            if (col + 3 < limit) v.w = p[3];
        }
    }
    return v;
}

// Four consecutive floats p[0..3].  ALIGNED: p is 16-byte aligned.
// Otherwise p need only be 4-byte aligned: the copy still compiles to one
// 128-bit global load, which gfx950 serves at any dword alignment.
template <bool ALIGNED>
__device__ __forceinline__ f32x4 load4(const float *__restrict__ p)
{
    if (ALIGNED) return *reinterpret_cast<const f32x4 *>(p);
    f32x4 v;
    __builtin_memcpy(&v, p, sizeof v);
    return v;
}

template <int BM, int BN, int BK, int WM, int WN>
struct MfmaTile {
    static constexpr int NT = WM * WN * 64;  // threads per workgroup
    static constexpr int TM = BM / WM;       // wave sub-tile rows
    static constexpr int TN = BN / WN;       // wave sub-tile columns
    static constexpr int FM = TM / 16;       // 16x16 MFMA blocks per wave, along M
    static constexpr int FN = TN / 16;       // ... along N
    static constexpr int SA = BK + 8;        // LDS pitch of an A slab row (m-major)
    static constexpr int SB = BN + 4;        // LDS pitch of a B slab row (k-major)
    static constexpr int AQ = BK / 4;        // float4 per A slab row
    static constexpr int BQ = BN / 4;        // float4 per B slab row
    static constexpr int A4 = BM * AQ;       // float4 per A slab
    static constexpr int B4 = BK * BQ;       // float4 per B slab
    static constexpr int NA = (A4 + NT - 1) / NT;  // A float4 per thread (last may idle)
    static constexpr int NB = (B4 + NT - 1) / NT;
    static constexpr int LDS_A = BM * SA;    // floats per A buffer
    static constexpr int LDS_B = BK * SB;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BK % 16 == 0, "BK must be a multiple of 16");
    static_assert(BN % 16 == 0, "B pitch needs BN % 16 == 0 for conflict-free reads");
    static_assert(BM % 16 == 0 && A4 % 64 == 0 && B4 % 64 == 0, "slab loads go in chunks of 64");
};

// The slab pipeline and epilogue of one workgroup.  EDGE selects masked
// loads of rows/columns (tiles crossing the matrix border); with EDGE false
// only a ragged last K slab is masked.
template <int BM, int BN, int BK, int WM, int WN, int ST, bool AVEC, bool BVEC, bool EDGE>
__device__ __forceinline__ void mfma_tile_body(const GemmArgs &g, int m0, int n0, float *As,
                                               float *Bs)
{
    using T = MfmaTile<BM, BN, BK, WM, WN>;
    constexpr int NT = T::NT, TM = T::TM, TN = T::TN, FM = T::FM, FN = T::FN;
    constexpr int SA = T::SA, SB = T::SB, AQ = T::AQ, BQ = T::BQ, NA = T::NA, NB = T::NB;
    const int M = g.M, N = g.N, K = g.K;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave / WN;
    const int wc = wave % WN;
    const int lm = lane & 15;  // row (A) / column (B, D) inside a 16-block
    const int lg = lane >> 4;  // k group (A, B) / row group (D)

    // Where this thread's slab loads come from (global) and go to (LDS).
    // Load i of a wave covers chunk c = wave + i * (NT / 64) of 64 float4.
    // The chunk count divides by 64, so whether a load is used is the same
    // for every lane of a wave (a scalar branch, no per-lane masking).
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    bool a_use[NA], b_use[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i)
        a_use[i] = (T::A4 % NT == 0) || wave_s + i * (NT / 64) < T::A4 / 64;
#pragma unroll
    for (int i = 0; i < NB; ++i)
        b_use[i] = (T::B4 % NT == 0) || wave_s + i * (NT / 64) < T::B4 / 64;
    // A chunk: 16 rows x 4 float4; lane -> row lane % 16, float4 lane / 16,
    // so the LDS store has the bank pattern of the fragment read below.
    // B: float4 f = tid + i * NT in row-major order over the BK x BN slab.
    // (Recomputed where needed rather than kept live across the K loop.)
    auto a_rc = [&](int i, int &r, int &c) {
        const int ch = a_use[i] ? wave_s + i * (NT / 64) : 0;
        r = 16 * (ch / (AQ / 4)) + lm;
        c = 4 * (4 * (ch % (AQ / 4)) + lg);
    };
    auto b_rc = [&](int i, int &r, int &c) {
        const int f = b_use[i] ? tid + i * NT : 0;
        r = f / BQ;
        c = (f % BQ) * 4;
    };
    int a_lds[NA], b_lds[NB];
    const float *a_src[NA];
    const float *b_src[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        int r, c;
        a_rc(i, r, c);
        a_lds[i] = r * SA + c;
        a_src[i] = g.A + (int64_t)(m0 + r) * g.lda + c;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        int r, c;
        b_rc(i, r, c);
        b_lds[i] = r * SB + c;
        b_src[i] = g.B + (int64_t)r * g.ldb + n0 + c;
    }

    f32x4 ra[NA], rb[NB];
    // Unmasked fetch: tile inside C, full K slab.
    auto fetch_fast = [&](int k0) {
        const int64_t boff = (int64_t)k0 * g.ldb;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            if (a_use[i]) ra[i] = load4<AVEC>(a_src[i] + k0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (b_use[i]) rb[i] = load4<BVEC>(b_src[i] + boff);
    };
    auto fetch_masked = [&](int k0) {
        const int64_t boff = (int64_t)k0 * g.ldb;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            if (a_use[i]) {
                int r, c;
                a_rc(i, r, c);
                ra[i] = load4_masked<AVEC>(a_src[i] + k0, m0 + r < M, k0 + c, K);
            }
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (b_use[i]) {
                int r, c;
                b_rc(i, r, c);
                rb[i] = load4_masked<BVEC>(b_src[i] + boff, k0 + r < K, n0 + c, N);
            }
    };
    auto fetch = [&](int k0) {
        if (!EDGE && k0 + BK <= K)
            fetch_fast(k0);
        else
            fetch_masked(k0);
    };
    auto stash = [&](int buf) {
        float *as = As + buf * T::LDS_A;
        float *bs = Bs + buf * T::LDS_B;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            if (a_use[i]) *reinterpret_cast<f32x4 *>(as + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (b_use[i]) *reinterpret_cast<f32x4 *>(bs + b_lds[i]) = rb[i];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int a_frag = (wr * TM + lm) * SA + 4 * lg;
    const int b_frag = (4 * lg) * SB + wc * TN + lm;
    // compute(buf, hook): the slab's MFMAs; hook() runs just before the
    // MFMAs of k-step 1 of the last 16-wide chunk.  The caller stores the
    // prefetched next slab to LDS there, so those writes finish while the
    // remaining MFMAs run and the barrier after the slab does not wait on
    // them (measured: 114 -> 121 TFLOPS at 5120^3 against storing after the
    // whole slab).
    auto compute = [&](int buf, auto hook) {
        const float *as = As + buf * T::LDS_A + a_frag;
        const float *bs = Bs + buf * T::LDS_B + b_frag;
#pragma unroll
        for (int q = 0; q < BK / 16; ++q) {
            f32x4 af[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[fm] = *reinterpret_cast<const f32x4 *>(as + fm * 16 * SA + 16 * q);
            float bf[4][FN];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    bf[s][fn] = bs[(16 * q + s) * SB + fn * 16];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (q == BK / 16 - 1 && s == 1) hook();
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            af[fm][s], bf[s][fn], acc[fm][fn], 0, 0, 0);
            }
        }
    };

    const int nslab = (K + BK - 1) / BK;
    fetch(0);
    stash(0);
    if constexpr (ST == 2) {
        __syncthreads();
        for (int t = 0; t < nslab; ++t) {
            const int cur = t & 1;
            const bool more = t + 1 < nslab;
            if (more) fetch((t + 1) * BK);
            compute(cur, [&] { if (more) stash(cur ^ 1); });
            __syncthreads();
        }
    } else if constexpr (ST == 0) {
        // Fragment prefetch (BK = 16): while slab t's last two k-steps run,
        // the wave already reads slab t + 1's MFMA operands from LDS into a
        // second register set, so a slab starts with its operands in
        // registers.  The barrier sits after k-step 1, behind MFMAs still in
        // flight.  Two LDS buffers: slab t + 1 is stored to buffer (t+1) & 1
        // after k-step 0 of slab t; that buffer held slab t - 1, whose
        // operands every wave had in registers before reaching the previous
        // barrier.
        static_assert(BK == 16, "fragment prefetch is written for 16-wide slabs");
        if (nslab > 1) fetch(BK);
        __syncthreads();
        f32x4 af0[FM], af1[FM];
        float bf0[4][FN], bf1[4][FN];
        auto read_frags = [&](int buf, f32x4 (&af)[FM], float (&bf)[4][FN]) {
            const float *as = As + buf * T::LDS_A + a_frag;
            const float *bs = Bs + buf * T::LDS_B + b_frag;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[fm] = *reinterpret_cast<const f32x4 *>(as + fm * 16 * SA);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    bf[s][fn] = bs[s * SB + fn * 16];
        };
        auto ksteps = [&](int s0, int s1, const f32x4 (&af)[FM], const float (&bf)[4][FN]) {
#pragma unroll
            for (int s = s0; s < s1; ++s)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            af[fm][s], bf[s][fn], acc[fm][fn], 0, 0, 0);
        };
        auto slab = [&](int t, const f32x4 (&af)[FM], const float (&bf)[4][FN],
                        f32x4 (&afn)[FM], float (&bfn)[4][FN]) {
            const bool more = t + 1 < nslab;
            ksteps(0, 1, af, bf);
            if (more) stash((t + 1) & 1);
            if (t + 2 < nslab) fetch((t + 2) * BK);
            ksteps(1, 2, af, bf);
            __syncthreads();
            if (more) read_frags((t + 1) & 1, afn, bfn);
            ksteps(2, 4, af, bf);
        };
        read_frags(0, af0, bf0);
        for (int t = 0; t < nslab; t += 2) {
            slab(t, af0, bf0, af1, bf1);
            if (t + 1 < nslab) slab(t + 1, af1, bf1, af0, bf0);
        }
    } else {
        // Three LDS buffers; slab t is read from buffer t % 3.  While slab t
        // runs, the registers hold slab t + 1, fetched one whole slab
        // earlier: they go to buffer (t + 1) % 3 inside slab t's MFMA
        // sequence and are then refilled with slab t + 2.  That buffer was
        // last read in slab t - 2, which every wave left before the barrier
        // that ended it.
        if (nslab > 1) fetch(BK);
        __syncthreads();
        int cur = 0;
        for (int t = 0; t < nslab; ++t) {
            const int nxt = cur == 2 ? 0 : cur + 1;
            const bool more = t + 1 < nslab;
            const bool more2 = t + 2 < nslab;
            compute(cur, [&] {
                if (more) {
                    stash(nxt);
                    if (more2) fetch((t + 2) * BK);
                }
            });
            __syncthreads();
            cur = nxt;
        }
    }

    // Epilogue: C = alpha*acc + beta*C over the valid window.
    const float alpha = g.alpha, beta = g.beta;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wr * TM + fm * 16 + 4 * lg + i;
            if (EDGE && row >= M) continue;
            float *crow = g.C + (int64_t)row * g.ldc;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int col = n0 + wc * TN + fn * 16 + lm;
                if (!EDGE || col < N) {
                    float v = alpha * acc[fm][fn][i];
                    if (beta != 0.f) v = fmaf(beta, crow[col], v);
                    crow[col] = v;
                }
            }
        }
    }
}

// WPE: waves per SIMD the register allocation must allow (the kernel is
// meant to run OCC = WPE * 4 / (WM*WN) workgroups per CU).
// ST: LDS buffers per operand (2 or 3), i.e. pipeline stages.
template <int BM, int BN, int BK, int WM, int WN, int WPE, int ST, bool AVEC, bool BVEC>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
mfma_tile_kernel(GemmArgs g)
{
    using T = MfmaTile<BM, BN, BK, WM, WN>;
    static_assert(ST == 0 || ST == 2 || ST == 3, "pipeline: 0 fragment prefetch, 2 or 3 LDS stages");
    constexpr int NBUF = ST == 3 ? 3 : 2;
    __shared__ __attribute__((aligned(16))) float As[NBUF * T::LDS_A];
    __shared__ __attribute__((aligned(16))) float Bs[NBUF * T::LDS_B];

    int tm, tn;
    tile_of_block(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const bool interior = m0 + BM <= g.M && n0 + BN <= g.N;
    if (interior)
        mfma_tile_body<BM, BN, BK, WM, WN, ST, AVEC, BVEC, false>(g, m0, n0, As, Bs);
    else
        mfma_tile_body<BM, BN, BK, WM, WN, ST, AVEC, BVEC, true>(g, m0, n0, As, Bs);
}

// Stream-K form: this workgroup's range of tile segments (sk_run).
template <int BM, int BN, int BK, int WM, int WN, int WPE, int ST, bool AVEC, bool BVEC>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
mfma_tile_sk_kernel(GemmArgs g, SkArgs s)
{
    using T = MfmaTile<BM, BN, BK, WM, WN>;
    constexpr int NBUF = ST == 3 ? 3 : 2;
    __shared__ __attribute__((aligned(16))) float As[NBUF * T::LDS_A];
    __shared__ __attribute__((aligned(16))) float Bs[NBUF * T::LDS_B];

    sk_run<BM, BN>(g, s, [&](const GemmArgs &a, int m0, int n0) __attribute__((always_inline)) {
        if (m0 + BM <= a.M && n0 + BN <= a.N)
            mfma_tile_body<BM, BN, BK, WM, WN, ST, AVEC, BVEC, false>(a, m0, n0, As, Bs);
        else
            mfma_tile_body<BM, BN, BK, WM, WN, ST, AVEC, BVEC, true>(a, m0, n0, As, Bs);
    });
}

}  // namespace sgemm
