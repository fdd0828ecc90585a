/*
 * libsgemm -- single-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain sizes, scalars and device pointers;
 * nothing here depends on PyTorch.
 *
 * The operation is the one every SGEMM kernel of the NVIDIA_SGEMM_PRACTICE
 * README computes (kernel 1 section: C = alpha * A*B + beta * C), on
 * row-major fp32 matrices addressed the way that README's OFFSET(row, col,
 * ld) macro does (kernel 6 section): element (r, c) of a matrix with leading
 * dimension ld lives at index r*ld + c.
 */
#ifndef LIBSGEMM_SGEMM_H
#define LIBSGEMM_SGEMM_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel families for sgemm_f32_variant(). */
enum sgemm_variant {
    SGEMM_VARIANT_AUTO = 0, /* shape-driven selection (what sgemm_f32 does) */
    SGEMM_VARIANT_MFMA = 1, /* fp32 matrix-core tile kernel, tile chosen by shape */
    SGEMM_VARIANT_VALU = 2, /* vector-FMA register-tile kernel (8x8 per thread) */
    SGEMM_VARIANT_SKINNY = 3, /* streaming kernel for M <= 64, K <= 240 (A resident
                               * in LDS, B and C streamed once); other shapes
                               * return SGEMM_ERR_VARIANT_SHAPE */
    /* SGEMM_VARIANT_MFMA_TILE + i forces entry i of the MFMA tile table
     * (0 <= i < sgemm_num_mfma_tiles()), bypassing the selector; sgemm_plan
     * names the tile.  For tests and tuning. */
    SGEMM_VARIANT_MFMA_TILE = 16,
    /* SGEMM_VARIANT_LADDER + r forces rung r (0 <= r < SGEMM_LADDER_RUNGS)
     * of the optimisation ladder the pages climb on SIMT cores, each rung a
     * kernel of its own with vector FMAs (NVIDIA_SGEMM_PRACTICE README,
     * kernels 1-7; UNIVERSAL_SGEMM_CUDA README, "Results" section, modes
     * 0-4; cnblogs matmul_opt.cu, naive / optimized / advanced kernels):
     *   0 naive: one thread per element of C, operands from global memory;
     *   1 coalesced: lanes of a wave on consecutive columns;
     *   2 lds: 32 x 32 tiles of A and B staged in LDS;
     *   3 tile1d: 64 x 64 tile, 8 rows of C per thread;
     *   4 tile2d: 128 x 128 tile, 8 x 8 block of C per thread;
     *   5 regcache: as 4, operands copied to registers, outer product;
     *   6 vec4: as 5, 128-bit loads, A slab stored k-major;
     *   7 dbuf: as 6, double-buffered slabs (= SGEMM_VARIANT_VALU).
     * Any shape runs.  For measurement beside the pages' tables; the
     * selector never picks them. */
    SGEMM_VARIANT_LADDER = 32,
    /* SGEMM_VARIANT_STREAMK_TILE + i forces entry i of the MFMA tile table
     * run stream-K: resident workgroups take equal ranges of (tile,
     * k-slab) units and a second kernel adds the partial tiles (the
     * selector does this by itself when it pays).  For tests and tuning. */
    SGEMM_VARIANT_STREAMK_TILE = 48
};

#define SGEMM_LADDER_RUNGS 8

/* Status values other than 0 and the hipError_t codes. */
#define SGEMM_ERR_BAD_VARIANT (-100)   /* variant value unknown */
#define SGEMM_ERR_VARIANT_SHAPE (-101) /* variant cannot run this shape */
/* A forced stream-K variant (SGEMM_VARIANT_STREAMK_TILE + i) that cannot have
 * a workspace slot (see "Workspace" under sgemm_f32); nothing was queued: */
#define SGEMM_ERR_WORKSPACE (-102) /* its partial tiles exceed a slot */
#define SGEMM_ERR_NO_SLOT (-103)   /* every slot is busy with other streams' work */
#define SGEMM_ERR_CAPTURING (-104) /* the stream is being captured into a graph */

/*
 * sgemm_f32 -- C <- alpha * A * B + beta * C, all row-major fp32.
 *
 *   M, N, K   sizes: A is M x K, B is K x N, C is M x N.  Each must be >= 0.
 *   alpha     scale of the product.  alpha == 0: A and B are not read.
 *   A, lda    device pointer to A(0,0); A(i,k) is A[i*lda + k]; lda >= max(1,K).
 *   B, ldb    device pointer to B(0,0); B(k,j) is B[k*ldb + j]; ldb >= max(1,N).
 *   beta      scale of the old C.  beta == 0: C is written but not read, so
 *             NaN or Inf already in C does not reach the result.
 *   C, ldc    device pointer to C(0,0); C(i,j) is C[i*ldc + j]; ldc >= max(1,N).
 *             Only the M x N window is read or written; padding between
 *             rows is never touched.  C must not overlap A or B.
 *   stream    HIP stream the work is queued on (0 = the null stream).
 *
 * Ownership and synchronisation: all buffers belong to the caller and stay
 * on the current HIP device.  The call copies and synchronises nothing; it
 * queues kernels on `stream` and returns.  Results are visible once the
 * stream has been synchronised.
 *
 * Workspace: the call allocates, frees and synchronises nothing.  Shapes
 * that the selector runs stream-K (when whole tiles would leave the last
 * round of resident workgroups part-empty; see SGEMM_VARIANT_STREAMK_TILE)
 * keep partial tiles in a workspace slot: 64 MiB of a 256 MiB static device
 * array that the HIP runtime places when it loads the library's code and
 * keeps until the process ends, one copy per device.  A slot serves one
 * stream at a time, in stream order; each use sets the slot's event to the
 * completion of its last kernel (the event rides on that kernel's launch),
 * and a call on another stream takes the slot over only once that event has
 * completed (a query, not a wait).  So calls on different
 * streams never share partials, whatever they overlap.  When all four slots
 * of the device are busy with other streams' queued work, or when `stream`
 * is being captured into a graph, the selector's choice runs one tile per
 * workgroup instead (same result for integer data; within the accuracy
 * bound below otherwise); forced stream-K variants return
 * SGEMM_ERR_NO_SLOT or SGEMM_ERR_CAPTURING then.  A slot is tied to the
 * stream handle: destroying a stream with stream-K work still queued and
 * creating another that gets the same handle is not supported.
 *
 * Graph capture: the call only launches kernels on `stream` (no copies, no
 * memsets, no synchronisation, no allocation, no event records under
 * capture), so it may be captured into a HIP graph and replayed on any
 * stream; a captured call holds no pointer into the workspace.  A replay
 * computes what an eager call of the captured plan computes, bit for bit.
 * sgemm_tune may not be captured.
 *
 * Pointers need only float (4-byte) alignment; 16-byte aligned operands
 * with leading dimensions divisible by 4 take 128-bit load paths.
 *
 * Quick returns: M == 0 or N == 0 does nothing and returns 0 without any
 * HIP call.  K == 0 or alpha == 0 scales C by beta (beta == 0: C <- 0).
 *
 * Returns 0 on success; -p when parameter p (counting M as 1) is invalid:
 *   -1 M < 0,  -2 N < 0,  -3 K < 0,
 *   -5 A is NULL (while M*K > 0 and alpha != 0) or not 4-byte aligned,
 *   -6 lda < max(1,K),
 *   -7 B is NULL (while K*N > 0 and alpha != 0) or not 4-byte aligned,
 *   -8 ldb < max(1,N),
 *  -10 C is NULL (while M*N > 0) or not 4-byte aligned,
 *  -11 ldc < max(1,N);
 * all argument checks happen before any HIP call.  A positive value is the
 * hipError_t of a failed HIP call (device query or kernel launch); in that
 * case nothing was queued.
 *
 * Accuracy: each element is a fp32 sum of fp32 products (matrix-core
 * accumulation) scaled by alpha plus beta times the old value; stream-K
 * adds the partial sums of a tile in a fixed order, so a plan's results
 * repeat bit for bit from call to call.  (A stream-K shape called while
 * every workspace slot is busy on other streams, or under capture, runs
 * one tile per workgroup, whose fp32 sums may round differently; with
 * one stream doing stream-K work at a time, its plan never changes.)  It is
 * within 1e-5 * (|alpha| * sum_k |A(i,k) B(k,j)| + |beta C(i,j)|) + 1e-6 of
 * the exact result for data like the benchmark's, and exact for integer
 * data whose partial sums stay below 2^24.
 *
 * Thread safety: re-entrant; the shared state is a per-device cache of the
 * compute-unit count, filled once, the workspace slots, under a mutex held
 * while a stream-K call queues its kernels, and the table of tuned choices
 * (sgemm_tune), under another.
 */
int sgemm_f32(int M, int N, int K, float alpha, const float *A, int lda,
              const float *B, int ldb, float beta, float *C, int ldc,
              hipStream_t stream);

/*
 * sgemm_f32_variant -- as sgemm_f32, but with the kernel family forced to
 * `variant` (enum sgemm_variant).  This mirrors the page-2 driver's
 * GEMM_MODE switch (UNIVERSAL_SGEMM_CUDA README, "Results" section), which
 * picks one kernel of the optimisation ladder per run; it exists to
 * benchmark and test each family on its own.  SGEMM_VARIANT_AUTO behaves
 * exactly like sgemm_f32.  Returns SGEMM_ERR_BAD_VARIANT for an unknown
 * variant (checked first), then the argument checks of sgemm_f32, then
 * SGEMM_ERR_VARIANT_SHAPE if the forced kernel cannot run this shape;
 * otherwise exactly what sgemm_f32 returns.
 */
int sgemm_f32_variant(int variant, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb,
                      float beta, float *C, int ldc, hipStream_t stream);

/*
 * sgemm_plan -- describe, without touching any GPU, the kernel that
 * sgemm_f32_variant would launch for this problem on a device with
 * `num_cus` compute units, assuming 16-byte aligned base pointers.
 * Writes a NUL-terminated text such as
 *   "mfma bm=160 bn=160 bk=16 waves=2x2 occ=2 vecA=1 vecB=1 grid=1024 group=8
 *    load=direct streamk=0 dp=0 split=0 ws=0"
 * (on one line: tile, waves, workgroups per CU, 128-bit paths, tiles, raster
 * group, slab load path -- "direct" straight to LDS, "shifted" the same for
 * B rows not 16-byte aligned, "regs" through registers -- stream-K
 * workgroups, tiles run whole, tiles split, workspace bytes of the partial
 * tiles -- the plan of a call that finds a free workspace slot)
 * into buf (at most buflen bytes, truncated if needed).  The leading word
 * names the kernel: "none" (nothing to do), "scale" (K == 0 or alpha == 0),
 * "mfma", "valu", "skinny", "stream16" or "ladder".  Returns 0, or the same negative codes as
 * sgemm_f32_variant (pointer checks excepted), or -12 when num_cus < 1 or
 * buf is NULL with buflen > 0.
 */
int sgemm_plan(int variant, int M, int N, int K, int lda, int ldb, int ldc,
               float alpha, int num_cus, char *buf, int buflen);

/*
 * sgemm_tune -- measure which kernel runs this problem fastest on the
 * caller's operands, make it the one sgemm_f32 launches from then on for
 * problems with the same key, and compute C <- alpha * A * B + beta * C
 * with it.  This automates, by measurement, the block-size trade-off the
 * NVIDIA_SGEMM_PRACTICE README reasons through by hand (kernel 3 section:
 * larger blocks cut global traffic but leave compute units idle and need
 * more shared memory) and the tile-parameter choice matmul_opt.cu's design
 * notes justify (item 6).
 *
 *   M ... stream   as sgemm_f32; on return C holds exactly what sgemm_f32
 *                  computes with the chosen kernel.
 *   reps           timed launches per candidate (>= 1), after one untimed.
 *   chosen         if not NULL, receives the chosen variant (an
 *                  enum sgemm_variant value; SGEMM_VARIANT_AUTO when the
 *                  selector's own choice was fastest).
 *   us             if not NULL, receives its mean time per launch, in
 *                  microseconds.
 *
 * Candidates: the selector's choice, the skinny kernel when it can run the
 * shape, and every entry of the MFMA tile table run one tile per workgroup
 * and run stream-K.  The timed launches write into a temporary buffer the
 * size of C's window, at the same offset from a 16-byte boundary as C,
 * allocated with hipMalloc and freed before returning; candidates see the
 * same A and B.  The call synchronises `stream` and waits for the device;
 * do not call it under graph capture.
 *
 * Key: device, M, N, K, lda, ldb, ldc, and whether each of A, B and C takes
 * the 128-bit paths (16-byte aligned base, leading dimension divisible by
 * 4).  sgemm_f32 and SGEMM_VARIANT_AUTO look the key up while any choice is
 * recorded; sgemm_plan(SGEMM_VARIANT_AUTO, ...) describes the tuned kernel
 * and appends " tuned=<variant>".  Forced variants are never redirected.
 * A tuned stream-K choice that finds no free workspace slot (or a stream
 * under capture) runs one tile per workgroup, as the selector's choice does.
 *
 * Quick-return problems (M, N or K zero, or alpha zero) are computed as by
 * sgemm_f32 and record nothing.  Returns the argument checks of sgemm_f32,
 * then -13 if reps < 1, all before any HIP call; a positive hipError_t if
 * an allocation, event or synchronisation fails; otherwise the status of
 * the final launch.  Candidates that cannot run the problem are skipped;
 * if none can, the first one's status is returned.
 *
 * Thread safety: the table of choices is under a mutex.  Tuning one key
 * from two threads at once records one of the two results.
 */
int sgemm_tune(int M, int N, int K, float alpha, const float *A, int lda,
               const float *B, int ldb, float beta, float *C, int ldc,
               hipStream_t stream, int reps, int *chosen, float *us);

/* Forget every tuned choice: sgemm_f32 returns to the shape-driven
 * selector for all problems.  Thread-safe; no HIP call. */
void sgemm_tune_reset(void);

/* Number of entries in the MFMA tile table (see SGEMM_VARIANT_MFMA_TILE). */
int sgemm_num_mfma_tiles(void);

/* Short English text for a status value returned above (never NULL). */
const char *sgemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBSGEMM_SGEMM_H */
