// fp32 MFMA tile kernel with direct global -> LDS slab loads (gfx950).
//
// The mathematics of the register-staged tile kernel in mfma_tile.hpp (one
// workgroup per BM x BN tile of C, K in 16-wide slabs,
// v_mfma_f32_16x16x4_f32 with lane group g taking k = 4g + s at step s),
// but the slabs travel from HBM to LDS with
// global_load_lds_dwordx4: lane l of the instruction writes its 16 bytes
// to LDS at M0 + 16 l, so no registers hold slab data and no LDS store
// instructions are issued.  The registers this frees hold a second set of
// MFMA operands, so a wave reads slab t+1's operands while slab t's last
// MFMAs run.
//
// Used when A rows are 16-byte aligned, for every tile of the launch: in a
// tile that sticks out of C, A rows past M fetch row M - 1 and B pieces past
// column N - 1 fetch the piece that holds it.  Those values reach only
// outputs outside C, which are not stored, so they need no zero fill.  The
// K % 16 columns after the last whole slab are a slab of their own, loaded
// through registers with zeros past K.  B rows are either 16-byte aligned
// or, in the shifted form (BSH), start anywhere: then each B row of a slab
// is fetched from the 16-byte boundary at or below its first column, d
// floats early (d = 0..3, the row's own misalignment), into one more chunk
// than the tile needs, and the operand reads add d back.  Every fetched
// 16-byte piece holds at least one element of the row segment, so no fetch
// leaves the pages B lies in.
//
// LDS: NBUF buffers (a ring; three unless the tile says otherwise) of
// (BM + BN) / 16 chunks of 1 KB (256 floats).  The
// position of every float inside a chunk is chosen so that each MFMA
// operand read of a wave is one contiguous run of LDS:
//   A chunk cm (rows 16 cm .. 16 cm + 15 of the tile), 16-byte slot j holds
//     A[16 cm + j % 16][k0 + 4 (j / 16) .. + 3]; lane l's 128-bit operand
//     read for block cm is slot l, i.e. the wave reads 1 KB in order.
//   B chunk cb (columns 16 cb .. 16 cb + 15), float e = 64 s + 16 g + c
//     holds B[k0 + 4 g + s][16 cb + c]; at step s lane l reads float
//     64 s + l, i.e. the wave reads 256 contiguous bytes.
// Both patterns touch every bank once, so operand reads are conflict-free.
// Shifted form: chunk cb holds columns 16 cb - d .. 16 cb - d + 15 of each
// row (d of that row), and chunk CB the next four.  Rows 4 apart share d
// (16-byte pieces hold four floats), so at step s one d serves the wave:
// lane 16 g + c reads float 64 s + 16 g + (c + d) of its block's chunk,
// spilling into the next chunk's first d floats when c + d >= 16; the
// banks stay distinct.
//
// Pipeline of slab t (its operands already in registers):
//   k-steps 0, 1: MFMAs, with the loads of slab t+NBUF-1 spread over them,
//     into the buffer slab t-1 used (every wave's reads of slab t-1's
//     operands had returned at the previous barrier, so the buffer is free).
//   Wait until this wave's loads of slab t+1 have landed; barrier.
//   k-steps 2, 3: MFMAs, with slab t+1's operand reads placed one per MFMA,
//     in the order the next slab first uses them.
// A slab's loads are issued about NBUF - 1.5 slabs before its operands are
// read.  Three buffers suit tiles of 128 and 160, whose slabs take long
// enough to cover the load latency; a 64 x 64 slab is 16 MFMAs per wave,
// and with one tile per CU its kernel keeps four buffers (three to five
// measured alike; eight, twelve and sixteen slower, more loads ahead of the
// first slab).  The spacing matters: issued back to back right after the
// barrier, reads and loads stall the wave's MFMA issue (measured at 5120^3:
// 125 TFLOPS clustered, 140 with reads and loads spread over the second
// half, 143 with the loads moved to the first half).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace sgemm {

typedef __attribute__((address_space(3))) float lds_float;

// Lane l's 16 bytes at src go to LDS bytes [lds + 16 l, lds + 16 l + 16).
// lds must be the same for the whole wave.  Completion is tracked with the
// vector memory counter (vmcnt).  An LDS DMA needs one wait state after the
// M0 write (the s_nop).
__device__ __forceinline__ void load_lds16(const float *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}

// Wait until at most N of this wave's vector memory loads are in flight and
// all of its LDS reads have returned, then meet the workgroup at a barrier.
// The LDS wait makes the ring's reuse rule hold by construction: the loads
// issued after barrier t overwrite the buffer of slab t, whose last operand
// reads every wave issued before barrier t, so they must have completed
// there (they were issued half a slab earlier, so the wait costs nothing).
template <int N>
__device__ __forceinline__ void wait_vm_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Wait until at most min(k, KMAX) slabs of L loads each are in flight (none
// if k <= 0), then meet the workgroup at a barrier.  vmcnt takes an
// immediate, so each count is a branch of its own; k is the same for the
// whole workgroup.
template <int L, int KMAX>
__device__ __forceinline__ void wait_slabs_barrier(int k)
{
    if constexpr (KMAX > 0) {
        if (k >= KMAX)
            wait_vm_barrier<KMAX * L>();
        else
            wait_slabs_barrier<L, KMAX - 1>(k);
    } else {
        wait_vm_barrier<0>();
    }
}

template <int BM, int BN, int WM, int WN, int NBUF_ = 3, bool BSH = false>
struct MfmaDl {
    static constexpr int NW = WM * WN;
    static constexpr int FM = BM / WM / 16;        // 16x16 blocks per wave along M
    static constexpr int FN = BN / WN / 16;        // ... along N
    static constexpr int CA = BM / 16;             // A chunks per slab
    static constexpr int CB = BN / 16;             // B chunks per slab (+1 shifted)
    static constexpr int CT = CA + CB + (BSH ? 1 : 0);
    // Loads per wave per slab: L, and one more for waves 0 .. X-1.
    static constexpr int L = CT / NW;
    static constexpr int X = CT % NW;
    static constexpr int LMAX = L + (X > 0 ? 1 : 0);
    static constexpr int BUF = CT * 256;           // floats per LDS buffer
    static constexpr int NBUF = NBUF_;
    static constexpr int LDS = NBUF * BUF;         // floats of LDS
    // The first half of a slab (2 FM FN MFMAs) carries up to LMAX loads, one
    // every STRIDE MFMAs; the second half R operand reads, one per MFMA.
    static constexpr int R = FM + 2 * FN;
    static constexpr int STRIDE = 2 * FM * FN / (LMAX + 1);
    static_assert(L >= 1, "every wave loads");
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile must be 16-aligned");
    static_assert(STRIDE >= 1 && R <= 2 * FM * FN, "too few MFMAs per slab for the reads and loads");
    static_assert(NBUF >= 3, "the ring needs a buffer being read, one landing, one free");
    static_assert(LMAX * (NBUF - 1) <= 63, "loads in flight must fit the vmcnt field");
};

// EDGE: the tile may stick out of C (clamped sources, masked stores); the
// interior copy carries neither.  KT: K need not be a multiple of 16 (the
// stream-K forms are only launched when it is, which keeps their scalar
// registers within budget).
template <int BM, int BN, int WM, int WN, int NBUF_, bool BSH, bool EDGE, bool KT>
__device__ __forceinline__ void mfma_dl_body(const GemmArgs &g, int m0, int n0, float *lds)
{
    using D = MfmaDl<BM, BN, WM, WN, NBUF_, BSH>;
    constexpr int NW = D::NW, FM = D::FM, FN = D::FN, CA = D::CA, CB = D::CB, L = D::L;
    constexpr int X = D::X, LMAX = D::LMAX, BUF = D::BUF;
    constexpr int NBUF = D::NBUF, R = D::R, S1 = D::STRIDE;
    constexpr int TM = BM / WM, TN = BN / WN;
    const int nslab = g.K / 16;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / WN;
    const int wc = wave % WN;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_float *)lds;
    // Waves 0 .. X-1 issue one load more per slab than the others.
    const bool extra = X > 0 && wave < X;

    // Shifted form: shift[s] is the misalignment, in floats, of column n0 in
    // B rows k with k % 4 == s (the same for every slab, 16 rows apart).
    int shift[4] = {0, 0, 0, 0};
    if constexpr (BSH) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            shift[s] = (int)((reinterpret_cast<uintptr_t>(g.B + (int64_t)s * g.ldb + n0) >> 2) & 3);
    }

    // Load i of this wave fills chunk c = wave + i * NW of every slab: A
    // block c if c < CA, else B chunk c - CA (the shifted form's chunk CB:
    // the row's four floats after chunk CB - 1, or, where the row needs none,
    // its last four floats again, unread).  Sources past C's edge are
    // clamped (rows to M - 1, B pieces to the one holding column N - 1).
    const float *src[LMAX];
    uint32_t dst[LMAX];
    bool is_a[LMAX];
#pragma unroll
    for (int i = 0; i < LMAX; ++i) {
        const int c = wave + i * NW;
        dst[i] = (uint32_t)c * 1024u;
        is_a[i] = c < CA;
        if (c < CA) {
            int r = m0 + 16 * c + (lane & 15);
            if constexpr (EDGE) r = r < g.M ? r : g.M - 1;
            src[i] = g.A + (int64_t)r * g.lda + 4 * (lane >> 4);
        } else {
            const int k = 4 * ((lane >> 2) & 3) + (lane >> 4);
            const int d = shift[lane >> 4];
            const float *row = g.B + (int64_t)k * g.ldb;
            int col = c < CA + CB ? n0 - d + 16 * (c - CA) + 4 * (lane & 3)
                                  : n0 - d + BN - (d > 0 ? 0 : 4);
            if constexpr (EDGE) {
                // The 16-byte piece holding column N - 1 starts e floats before it.
                const int e = (int)((reinterpret_cast<uintptr_t>(row + g.N - 1) >> 2) & 3);
                const int last = g.N - 1 - e;
                col = col < last ? col : last;
            }
            src[i] = row + col;
        }
    }
    const int64_t a_step = 16, b_step = 16 * g.ldb;
    // Load i of the next unissued slab into the buffer at byte offset bb.
    auto load = [&](int i, uint32_t bb) {
        load_lds16(src[i], bb + dst[i]);
        src[i] += is_a[i] ? a_step : b_step;
    };
    auto buffer_bytes = [&](int buf) { return lds_base + (uint32_t)buf * (BUF * 4); };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Operand sets: A as one f32x4 per 16-row block (element s for k-step
    // s), B as one float per k-step and 16-column block.
    f32x4 afs[2][FM];
    float bfs[2][4][FN];
    // Operand read number r (0 .. R-1) of the slab in buffer buf, in order
    // of first use: A blocks, then B k-steps 0-1, then B k-steps 2-3.
    // Shifted form: lane's float offset, inside its block's chunk, at step s.
    int boff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int x = (lane & 15) + shift[s];
        boff[s] = 64 * s + 16 * (lane >> 4) + (x & 15) + (x >= 16 ? 256 : 0);
    }
    auto read_op = [&](int r, int buf, f32x4 (&af)[FM], float (&bf)[4][FN]) {
        const float *base = lds + buf * BUF;
        if (r < FM) {
            af[r] = *reinterpret_cast<const f32x4 *>(base + (wr * FM + r) * 256 + 4 * lane);
        } else {
            const int h = (r - FM) / FN, fn = (r - FM) % FN;
            if constexpr (BSH) {
                const float *bs = base + (CA + wc * FN + fn) * 256;
                bf[2 * h][fn] = bs[boff[2 * h]];
                bf[2 * h + 1][fn] = bs[boff[2 * h + 1]];
            } else {
                const float *bs = base + (CA + wc * FN + fn) * 256 + 128 * h + lane;
                bf[2 * h][fn] = bs[0];
                bf[2 * h + 1][fn] = bs[64];
            }
        }
    };
    // k-steps s0..s1-1; hook(n) runs before the n-th MFMA of the call.
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
    auto no_hook = [](int) {};

    // Slab t from buffer buf with operands in set P; slab t+1's operands go
    // to set P ^ 1.  After the last slab the reads fetch a stale buffer (in
    // bounds; the values go unused) so that no branch separates the reads
    // from the waits the compiler places for them.
    auto slab = [&](auto P, int t, int buf) {
        constexpr int p = decltype(P)::value;
        // First half: the loads of slab t+NBUF-1 into the buffer slab t-1
        // used (every wave's reads of it had returned at barrier t-1).
        const bool more = t >= 1 && t + NBUF - 1 < nslab;
        const uint32_t bb = buffer_bytes(buf == 0 ? NBUF - 1 : buf - 1);
        ksteps(0, 2, afs[p], bfs[p], [&](int n) {
            if (n > 0 && n % S1 == 0 && n / S1 <= LMAX) {
                if (more && (n / S1 <= L || extra)) load(n / S1 - 1, bb);
            }
        });
        __builtin_amdgcn_sched_barrier(0);
        // In flight: slab t+1's loads, then those of the slabs after it up to
        // t+NBUF-1 (as far as they exist): wait for slab t+1's.
        if (extra)
            wait_slabs_barrier<LMAX, NBUF - 2>(nslab - 2 - t);
        else
            wait_slabs_barrier<L, NBUF - 2>(nslab - 2 - t);
        const int nb = buf + 1 == NBUF ? 0 : buf + 1;
        ksteps(2, 4, afs[p], bfs[p], [&](int n) {
            if (n < R) {
                read_op(n, nb, afs[p ^ 1], bfs[p ^ 1]);
                // Keep the compiler from gathering the reads into one burst.
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };

    // Prologue: slabs 0 .. NBUF-1 in flight, wait for slab 0.
#pragma unroll
    for (int b = 0; b < NBUF; ++b)
        if (b < nslab) {
#pragma unroll
            for (int i = 0; i < LMAX; ++i)
                if (i < L || extra) load(i, buffer_bytes(b));
        }
    if (extra)
        wait_slabs_barrier<LMAX, NBUF - 1>(nslab - 1);
    else
        wait_slabs_barrier<L, NBUF - 1>(nslab - 1);
    // (slab 0 issues no loads: slabs 1 .. NBUF-1 are already in flight)
#pragma unroll
    for (int r = 0; r < R; ++r) read_op(r, 0, afs[0], bfs[0]);

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

    // K not a multiple of 16: the last K % 16 columns of A and rows of B go
    // through registers into buffer 0, in the same chunk layout, with zeros
    // for k >= K (and for B columns outside the row), then one more slab of
    // MFMAs.  Every operand of the ring is in registers by now.
    if (KT && g.K % 16 != 0) {
        __syncthreads();
        const int kt = nslab * 16;
#pragma unroll
        for (int i = 0; i < LMAX; ++i) {
            const int c = wave + i * NW;
            if (i >= L && !extra) continue;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (c < CA) {
                int r = m0 + 16 * c + (lane & 15);
                r = r < g.M ? r : g.M - 1;
                const int k = kt + 4 * (lane >> 4);
                const float *p = g.A + (int64_t)r * g.lda + k;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (k + j < g.K) v[j] = p[j];
            } else {
                const int k = kt + 4 * ((lane >> 2) & 3) + (lane >> 4);
                const int col = n0 - shift[lane >> 4] + 16 * (c - CA) + 4 * (lane & 3);
                if (k < g.K) {
                    const float *p = g.B + (int64_t)k * g.ldb + col;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (col + j >= 0 && col + j < g.N) v[j] = p[j];
                }
            }
            *reinterpret_cast<f32x4 *>(lds + c * 256 + 4 * lane) = v;
        }
        __syncthreads();
        f32x4 af[FM];
        float bf[4][FN];
#pragma unroll
        for (int r = 0; r < R; ++r) read_op(r, 0, af, bf);
        ksteps(0, 4, af, bf, no_hook);
    }

    // Epilogue: C = alpha*acc + beta*C inside C's M x N window.
    const float alpha = g.alpha, beta = g.beta;
    const int lm = lane & 15, lg = lane >> 4;
    const int col0 = n0 + wc * TN + lm;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wr * TM + fm * 16 + 4 * lg + i;
            if (EDGE && row >= g.M) continue;
            float *crow = g.C + (int64_t)row * g.ldc + col0;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if (EDGE && col0 + fn * 16 >= g.N) continue;
                float v = alpha * acc[fm][fn][i];
                if (beta != 0.f) v = fmaf(beta, crow[fn * 16], v);
                crow[fn * 16] = v;
            }
        }
    }
}

// One BM x BN tile per workgroup; border tiles through the EDGE copy.
template <int BM, int BN, int WM, int WN, int WPE, int NBUF = 3, bool BSH = false>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
mfma_dl_kernel(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) float lds[MfmaDl<BM, BN, WM, WN, NBUF, BSH>::LDS];

    int tm, tn;
    tile_of_block(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    if (m0 + BM <= g.M && n0 + BN <= g.N)
        mfma_dl_body<BM, BN, WM, WN, NBUF, BSH, false, true>(g, m0, n0, lds);
    else
        mfma_dl_body<BM, BN, WM, WN, NBUF, BSH, true, true>(g, m0, n0, lds);
}

// Stream-K form: this workgroup's range of tile segments (sk_run), each
// through the same bodies; K must be a multiple of 16.
template <int BM, int BN, int WM, int WN, int WPE, int NBUF = 3, bool BSH = false>
__global__ void __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
mfma_dl_sk_kernel(GemmArgs g, SkArgs s)
{
    __shared__ __attribute__((aligned(16))) float lds[MfmaDl<BM, BN, WM, WN, NBUF, BSH>::LDS];

    sk_run<BM, BN>(g, s, [&](const GemmArgs &a, int m0, int n0) __attribute__((always_inline)) {
        if (m0 + BM <= a.M && n0 + BN <= a.N)
            mfma_dl_body<BM, BN, WM, WN, NBUF, BSH, false, false>(a, m0, n0, lds);
        else
            mfma_dl_body<BM, BN, WM, WN, NBUF, BSH, true, false>(a, m0, n0, lds);
    });
}

}  // namespace sgemm
