/*
 * mi_sgemm.h -- single-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 * Operation (every compute entry point)
 * -------------------------------------
 *     C <- alpha * A * B + beta * C,     C_ij = sum_{t=0}^{k-1} A_it * B_tj
 * The sum is the GEMM of page "GEMM优化原理" (hatrix.site), section 问题定义,
 * eq. 1 (A is m x k, B is k x n, C is m x n); the two scalars are those of the
 * kernel signature shown on page "gemm优化" (blog.lightlisten.com), section
 * 性能分析, read with the usual BLAS meaning.
 *
 * Layout.  All matrices are row-major with a leading dimension (the distance,
 * in elements, between the starts of consecutive rows):
 *     A_it = A[i*lda + t],   B_tj = B[t*ldb + j],   C_ij = C[i*ldc + j].
 * Elements beyond the logical width of a row (the padding up to ld) are never
 * read or written.  The _ex entry points also take A or B transposed (the
 * BLAS op(X) = X^T): trans_a = 1 means A is stored k x m, A_it = A[t*lda + i]
 * with lda >= max(1, m); trans_b = 1 means B is stored n x k,
 * B_tj = B[j*ldb + t] with ldb >= max(1, k).  Column-major operands are the
 * transposed row-major ones, so every BLAS storage order is covered.
 * Pointers need no particular alignment (beyond that of a float) and ld
 * values need not be multiples of 4: tiles of A and B move to on-chip memory
 * 16 bytes per lane when both are 16-byte aligned with lda and ldb multiples
 * of 4, and 4 bytes per lane otherwise.
 *
 * Memory and streams.  A, B, C and the workspace are device memory owned by
 * the caller; the library never allocates or frees memory in these calls.
 * `stream` is a hipStream_t (NULL = the null stream) of the current device.
 * Compute calls are asynchronous: they return once the kernels are enqueued.
 * C must not overlap A, B or the workspace.  Results are deterministic: the
 * same call on the same inputs gives the same bits (mi_sgemm_splitk_atomic
 * excepted).
 *
 * Special cases.
 *  - m == 0 or n == 0: nothing is done (no pointer is touched).
 *  - k == 0 or alpha == 0: C <- beta * C; A and B are not read.
 *  - beta == 0: C is written without being read (NaN or Inf in C do not
 *    propagate).
 *
 * Errors.  Every argument is checked before anything is enqueued; on an error
 * nothing is written.  Return values are mi_status codes; mi_status_string()
 * gives a text.  A failure reported by the HIP runtime at launch time maps to
 * MI_SGEMM_ERROR_LAUNCH; a current device that is not gfx950 (or no device)
 * maps to MI_SGEMM_ERROR_DEVICE.
 */
#ifndef MI_SGEMM_H
#define MI_SGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mi_status {
    MI_SGEMM_SUCCESS = 0,
    MI_SGEMM_ERROR_INVALID_VALUE = 1, /* m, n or k < 0; splits < 0 or > k; a transpose
                                         flag other than 0 or 1; unknown kernel or
                                         config id; a launch of 2^31 or more
                                         workgroups or 2^32 or more work-items
                                         (a C of about 2^36 elements, or a forced
                                         slice count of that order); refused
                                         before anything is enqueued */
    MI_SGEMM_ERROR_INVALID_LD = 2,    /* lda < max(1,k), ldb < max(1,n) or ldc < max(1,n)
                                         (m for lda, k for ldb when transposed) */
    MI_SGEMM_ERROR_NULL_POINTER = 3,  /* NULL for an operand that would be read or written */
    MI_SGEMM_ERROR_WORKSPACE = 4,     /* workspace NULL or smaller than required */
    MI_SGEMM_ERROR_LAUNCH = 5,        /* the HIP runtime rejected a kernel launch */
    MI_SGEMM_ERROR_DEVICE = 6,        /* no current HIP device, or it is not gfx950 */
    MI_SGEMM_ERROR_SCRATCH_LIMIT = 7  /* mi_sgemm_splitk_noalloc: the forced plan needs more
                                         than MI_SGEMM_NOALLOC_SCRATCH_BYTES of scratch */
} mi_status;

/*
 * mi_sgemm -- the matrix-core path.
 * Blocked through the memory hierarchy as described on page "GEMM优化原理",
 * sections "从 global memory 到 shared memory 再到 register" and
 * "prefetch 和双缓冲": workgroup tiles of A and B prefetched one to three k
 * steps ahead into an LDS ring of two to four buffers (three or four for the
 * tiles the automatic choice uses), per-wave tiles of C accumulated by FP32 MFMA
 * instructions, and a grouped, XCD-aware workgroup order for L2 reuse (page
 * "gemm优化", section 杂项：预取缓存1， Swizzle 增强L2缓存命中).  The tile
 * configuration is chosen from the sizes of C (mi_sgemm_get_plan reports it).
 * Arguments: m, n, k >= 0 sizes; alpha, beta scalars; A, B read-only inputs;
 * C input (when beta != 0) and output; lda, ldb, ldc leading dimensions in
 * elements; stream a hipStream_t or NULL.  Returns a mi_status.
 */
int mi_sgemm(int m, int n, int k, float alpha,
             const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream);

/* Transpose flags of the _ex entry points. */
typedef enum mi_op {
    MI_SGEMM_OP_N = 0, /* operand as given (A: m x k, B: k x n, row-major) */
    MI_SGEMM_OP_T = 1  /* operand given transposed (A stored k x m, B stored n x k) */
} mi_op;

/*
 * mi_sgemm_ex -- mi_sgemm with op(A) and op(B): C <- alpha * op(A) op(B) +
 * beta * C.  A transposed operand is staged into LDS in its memory layout
 * (m- or n-contiguous rows of k) and read back as MFMA fragments with a
 * swizzle that keeps those transposed reads free of bank conflicts (the
 * conflict case of page "GEMM优化原理", section 基于 register 计算).
 * trans_a, trans_b: MI_SGEMM_OP_N or MI_SGEMM_OP_T.  Other arguments,
 * semantics and errors as mi_sgemm; mi_sgemm(...) equals
 * mi_sgemm_ex(MI_SGEMM_OP_N, MI_SGEMM_OP_N, ...).
 */
int mi_sgemm_ex(int trans_a, int trans_b, int m, int n, int k, float alpha,
                const float *A, int lda, const float *B, int ldb,
                float beta, float *C, int ldc, void *stream);

/*
 * mi_sgemm_valu -- the register-tiled VALU path, kept as a measured
 * comparison.  It follows the worked example of page "GEMM优化原理", section
 * 一个具体的例子: 128 x 128 workgroup tiles, k step 8, 256 threads each owning
 * an 8 x 8 block of C updated by outer products of 8 A and 8 B values
 * (page aerisun.top, section "Register Tiling 与线程内复用"), with a
 * double-buffered LDS stage.  When every CU gets at most one tile (at most
 * 256 tiles) and A and B allow 16-byte loads, two such groups of 256 threads
 * share a tile (512 threads per workgroup), each taking every other k step,
 * and the first adds the second's sums before the store (a fixed order, so
 * results are reproducible); VALU configuration ids: 0 one group, 1 two.
 * Same arguments, semantics and errors as mi_sgemm.  It is bound by the
 * FP32 vector peak (non-packed FMA).
 */
int mi_sgemm_valu(int m, int n, int k, float alpha,
                  const float *A, int lda, const float *B, int ldb,
                  float beta, float *C, int ldc, void *stream);

/*
 * mi_sgemm_splitk_workspace_bytes -- bytes of device workspace that
 * mi_sgemm_splitk needs for these sizes and this split request (splits = 0
 * asks the library to choose).  The workspace holds the raw partial sums of
 * the S slices of the big iteration over K (page "GEMM优化原理", section
 * 基于 shared memory 计算): S slices of m * n floats, each slice rounded up
 * to a multiple of 64 floats, plus 256 bytes so that the slices can start on
 * a 256-byte boundary inside any buffer -- S * ceil(m*n / 64) * 64 * 4 + 256
 * bytes.  When the plan is the stream-K schedule instead (plan field
 * stream_k_grid > 0) it is two tiles of floats per stream-K workgroup, plus
 * the same 256 bytes.  Returns 0 when no workspace is needed (m == 0,
 * n == 0 or k == 0, or a plan of one slice) and also for invalid arguments
 * (m, n, k < 0, splits < 0 or splits > k).
 */
size_t mi_sgemm_splitk_workspace_bytes(int m, int n, int k, int splits);

/*
 * mi_sgemm_splitk -- the same product with the k range cut into S slices.
 * The sum over t of page "GEMM优化原理" (section 基于 shared memory 计算,
 * the "big iteration" over K) is split: workgroup (tile, s) sums its slice of
 * t into raw FP32 partials in the workspace, then a second kernel adds the S
 * partials of every C element -- each lane summing some slices, then a
 * cross-lane wavefront reduction (page aerisun.top, sections
 * "先在线程内累加，再交换部分和" and "Warp shuffle 的数据交换") -- and applies
 * alpha and beta.  splits: requested S (the library may use fewer slices
 * so that each is a whole number of k steps), or 0: the library chooses the
 * tile configuration and S with a time model of MI355X (workgroup rounds
 * over the 256 CUs, per-workgroup overhead, the combine's cost), keeping
 * the workspace under 512 MiB.  A plan of one slice runs the single-pass
 * kernel directly, with the same result as mi_sgemm_ex, and needs no
 * workspace (ws may then be NULL).  ws / ws_bytes: caller-owned device
 * workspace of at least mi_sgemm_splitk_workspace_bytes(m, n, k, splits)
 * bytes, 256-byte aligned for best speed; its contents on return are
 * unspecified.  Two calls that share a workspace must be ordered on one
 * stream.  Other arguments and errors as mi_sgemm, plus
 * MI_SGEMM_ERROR_WORKSPACE.
 */
int mi_sgemm_splitk(int m, int n, int k, float alpha,
                    const float *A, int lda, const float *B, int ldb,
                    float beta, float *C, int ldc,
                    int splits, void *ws, size_t ws_bytes, void *stream);

/*
 * mi_sgemm_splitk_ex -- mi_sgemm_splitk with op(A) and op(B) as in
 * mi_sgemm_ex.  The workspace size does not depend on the transposes
 * (mi_sgemm_splitk_workspace_bytes).
 */
int mi_sgemm_splitk_ex(int trans_a, int trans_b, int m, int n, int k, float alpha,
                       const float *A, int lda, const float *B, int ldb,
                       float beta, float *C, int ldc,
                       int splits, void *ws, size_t ws_bytes, void *stream);

/* Bytes of the static device scratch that mi_sgemm_splitk_noalloc uses. */
#define MI_SGEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * mi_sgemm_splitk_noalloc -- mi_sgemm_splitk_ex for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same plans and kernels, with the
 * workspace replaced by a static scratch buffer of
 * MI_SGEMM_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each
 * device it runs on until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); the caller passes only the
 * operands.  splits = 0: the automatic plan, kept within the scratch (a plan
 * mi_sgemm_splitk_ex would run with more workspace is replaced by the best
 * one that fits, down to the single-pass kernel; where the automatic plan of
 * mi_sgemm_splitk_ex fits, it is the same plan and gives the same bits).  A
 * forced split count whose plan needs more than the scratch returns
 * MI_SGEMM_ERROR_SCRATCH_LIMIT before anything is enqueued.  Every call on one
 * device shares that device's scratch (it keeps the last call's contents;
 * nothing in it needs to start at zero): calls that overlap in time on one
 * device -- on different streams, or from different host threads without
 * ordering -- race and give wrong results; order them on one stream.  Other
 * arguments, semantics and errors as mi_sgemm_splitk_ex (without
 * MI_SGEMM_ERROR_WORKSPACE); a failure to obtain the scratch's device
 * address gives MI_SGEMM_ERROR_LAUNCH.
 */
int mi_sgemm_splitk_noalloc(int trans_a, int trans_b, int m, int n, int k, float alpha,
                            const float *A, int lda, const float *B, int ldb,
                            float beta, float *C, int ldc, int splits, void *stream);

/*
 * mi_sgemm_splitk_combine -- the second pass of mi_sgemm_splitk on its own:
 *     C_ij <- alpha * sum_{s < splits} ws[s * slice + i * n + j] + beta * C_ij
 * over the logical m x n extent of C (partial sums stored densely, row-major
 * with row length n, slice after slice).  The slices are added in two levels:
 * each lane sums a strided subset of them, then cross-lane exchanges of the
 * wavefront add the lanes' sums (page aerisun.top, sections
 * "先在线程内累加，再交换部分和" and "Warp shuffle 的数据交换"); the order is
 * fixed, so the result is the same bits on every run.  ws: device memory,
 * 16-byte aligned, read-only; slice: floats between the starts of two slices,
 * a multiple of 4 and at least m * n rounded up to a multiple of 4 (the
 * entries past m * n are read but not used).  beta == 0 writes C without
 * reading it; splits == 0 or alpha == 0 gives C <- beta * C without reading
 * ws.  Errors: INVALID_VALUE (m, n or splits < 0, or ws / slice outside the
 * rules above), INVALID_LD (ldc < max(1, n)), NULL_POINTER, LAUNCH, DEVICE.
 */
int mi_sgemm_splitk_combine(int m, int n, int splits, const float *ws, long long slice,
                            float alpha, float beta, float *C, int ldc, void *stream);

/*
 * mi_sgemm_splitk_atomic -- split-K without a workspace, kept as a measured
 * comparison for mi_sgemm_splitk: C is first scaled by beta (skipped when
 * beta == 1; beta == 0 writes zeros without reading C), then every
 * (tile, slice) workgroup adds alpha times its slice sum into C with hardware
 * float atomics -- the global-atomic combine of page aerisun.top, section
 * "全局原子操作互锁", applied once per output element and slice.  The order of
 * the additions varies between runs, so results are NOT bitwise
 * reproducible (they stay within the same error bound, and integer-valued
 * sums are exact).  Other arguments and errors as mi_sgemm_splitk, without
 * the workspace.
 */
int mi_sgemm_splitk_atomic(int m, int n, int k, float alpha,
                           const float *A, int lda, const float *B, int ldb,
                           float beta, float *C, int ldc, int splits, void *stream);

/* ------------------------------------------------------------------------
 * Sum of a float array.
 * ------------------------------------------------------------------------ */

/*
 * mi_reduce_sum -- out[0] = sum_{i<n} x[i] (page aerisun.top, section
 * "Reduce 的分层归约"): lanes accumulate many inputs in registers, waves add
 * their lanes with cross-lane operations (DPP row rotations and row swaps),
 * workgroups meet in LDS, and a second pass adds the workgroup partials; no
 * atomics, so the result is the same bits on every run.  x: n floats of
 * device memory (any 4-byte alignment; 16-byte aligned is faster); out: one
 * float of device memory, written (0 when n == 0); ws / ws_bytes: device
 * workspace of at least mi_reduce_sum_workspace_bytes(n) bytes.  Errors:
 * INVALID_VALUE (n < 0), NULL_POINTER, WORKSPACE, LAUNCH, DEVICE.
 */
int mi_reduce_sum(long long n, const float *x, float *out, void *ws, size_t ws_bytes,
                  void *stream);
size_t mi_reduce_sum_workspace_bytes(long long n);

/*
 * mi_reduce_sum_max_additions -- the largest number of floating-point
 * additions any input passes through on its way to out[0] for this n.  With
 * u = 2^-24, |computed - exact| <= max_additions * u * sum_i |x_i| (to first
 * order), which is the error bound of mi_reduce_sum.
 */
long long mi_reduce_sum_max_additions(long long n);

/* ------------------------------------------------------------------------
 * Clock measurement.
 * ------------------------------------------------------------------------ */

/*
 * mi_clock_probe -- measures the core clock on the GPU, in stream order (so
 * it reports the clock right before or after the kernels around it).  Page
 * "gemm优化" (blog.lightlisten.com), section 关于GPU频率影响, shows timings
 * changing with the core clock; this gives each timing its clock.  Each of
 * `workgroups` workgroups (placed on the XCDs round-robin: 8 cover each XCD
 * once) reads the shader-cycle counter and the constant-rate reference
 * counter, waits about spin_us microseconds, and reads both again:
 *     ticks[4w + 0] shader cycles at the start,  ticks[4w + 1] reference ticks,
 *     ticks[4w + 2] shader cycles at the end,    ticks[4w + 3] reference ticks;
 * the clock of workgroup w in MHz is
 *     (ticks[4w+2] - ticks[4w]) / (ticks[4w+3] - ticks[4w+1]) * ref_khz / 1000.
 * ticks: device memory for 4 * workgroups unsigned 64-bit values (written);
 * ref_khz: host int, receives the reference counter's rate in kHz.
 * Errors: INVALID_VALUE (workgroups outside 1..1024, spin_us outside
 * 1..100000), NULL_POINTER, DEVICE, LAUNCH.
 */
int mi_clock_probe(unsigned long long *ticks, int workgroups, int spin_us, int *ref_khz,
                   void *stream);

/*
 * mi_fma_rate_probe -- the issue rate of non-packed FP32 FMAs on the vector
 * ALUs, the bound of mi_sgemm_valu (page aerisun.top, section
 * "Register Tiling 与线程内复用", keeps the r_m x r_n outer product of the
 * inner loop in registers).  `workgroups` workgroups of 256 threads each run
 * `iters` iterations of one loop with no memory traffic:
 *   loop 0: an 8 x 8 outer product of register values (64 v_fma_f32 with
 *           every operand in a VGPR) plus 8 multiplies: 136 FLOP per thread
 *           per iteration -- the shape of mi_sgemm_valu's inner loop;
 *   loop 1: 16 independent chains x = x * a + b with a, b in scalar
 *           registers, 8 rounds: 256 FLOP per thread per iteration.
 * out: device memory for 256 * workgroups floats, written (one per thread,
 * so the loops are not optimised away).  Time the launch with events and
 * divide the FLOP count by it.  Errors: INVALID_VALUE (loop not 0 or 1,
 * workgroups outside 1..65536, iters outside 1..10^6), NULL_POINTER,
 * DEVICE, LAUNCH.
 */
int mi_fma_rate_probe(int loop, float *out, int workgroups, int iters, void *stream);

/*
 * Text for a mi_status value (a static string; never NULL).  The statuses
 * report the preconditions that page "GPU 访存与计算优化" (aerisun.top),
 * section "float4 向量化的条件", states for a vectorised kernel -- sizes that
 * are not negative, indices that do not overflow, arrays that hold the
 * elements addressed -- checked here before any launch instead of assumed;
 * alignment is not a precondition (unaligned operands take 4-byte loads).
 */
const char *mi_status_string(int status);

/* ------------------------------------------------------------------------
 * Planning queries (host only, no GPU needed) and forced configurations.
 * ------------------------------------------------------------------------ */

typedef enum mi_kernel {
    MI_SGEMM_KERNEL_MFMA = 0,
    MI_SGEMM_KERNEL_VALU = 1,
    MI_SGEMM_KERNEL_SPLITK = 2,
    MI_SGEMM_KERNEL_SPLITK_ATOMIC = 3
} mi_kernel;

/*
 * Launch geometry chosen for a call, in the vocabulary of page
 * "GEMM优化原理", section 问题定义, eq. 2 (b_m, b_n, b_k tiles; r_m x r_n per
 * thread; M x N blocks; K big iterations of b_k; b_k small iterations).
 */
typedef struct mi_sgemm_plan {
    int kernel;            /* mi_kernel */
    int config;            /* tile configuration id (see mi_sgemm_config_count) */
    int tile_m, tile_n, tile_k;   /* b_m, b_n, b_k */
    int micro_m, micro_n;  /* VALU: r_m, r_n per thread; MFMA: per-wave tile */
    int threads;           /* threads per workgroup */
    int tiles_m, tiles_n;  /* M = ceil(m / b_m), N = ceil(n / b_n) */
    long long workgroups;  /* grid size of the main kernel (stream-K: the
                              data-parallel tiles plus the stream-K workgroups) */
    int splits;            /* K slices (1 when not split) */
    int k_per_split;       /* length of every slice but possibly the last */
    int big_iterations;    /* b_k steps per workgroup: ceil(k_per_split / b_k) */
    int small_iterations;  /* per big iteration: b_k (VALU) or b_k / 2 (MFMA k steps) */
    int fma_per_small_iteration; /* per thread (VALU: r_m r_n FMAs) or per wave
                                    (MFMA: 32x32x2 instructions) */
    int outputs_per_thread;      /* C elements accumulated by one thread/lane */
    int a_elements_per_big_iteration; /* b_m * b_k */
    int b_elements_per_big_iteration; /* b_k * b_n */
    int group_m;           /* height, in tiles, of the grouped workgroup order */
    int vector_loads;      /* 1 when 16-byte loads of A and B are used */
    size_t workspace_bytes;
    int stream_k_grid;     /* > 0: the split-K entry runs a stream-K schedule for
                              this many concurrent workgroups (see
                              mi_sgemm_streamk; splits then 1, big_iterations
                              the tile's k steps) */
} mi_sgemm_plan;

/*
 * mi_sgemm_get_plan -- fills *plan with what a call of `kernel` would launch
 * for these sizes (lda/ldb multiples of 4 and aligned pointers assumed for
 * vector_loads; config = -1 for the automatic choice, else a forced id;
 * splits as for mi_sgemm_splitk, ignored otherwise).  Touches no GPU.
 * Returns MI_SGEMM_SUCCESS or MI_SGEMM_ERROR_INVALID_VALUE.
 */
int mi_sgemm_get_plan(int kernel, int config, int m, int n, int k, int splits,
                      mi_sgemm_plan *plan);

/* Number of tile configurations of `kernel` that can be forced (ids 0..count-1);
 * the split-K partial kernel takes the MI_SGEMM_KERNEL_MFMA ids. */
int mi_sgemm_config_count(int kernel);

/*
 * mi_sgemm_with_config -- mi_sgemm_ex / mi_sgemm_valu with a forced tile
 * configuration (for measured comparisons of tilings and for tests that
 * cover every configuration).  kernel is MI_SGEMM_KERNEL_MFMA or
 * MI_SGEMM_KERNEL_VALU (the VALU path takes operands as given only:
 * trans_a = trans_b = MI_SGEMM_OP_N); config < 0 means the automatic
 * choice.  Same semantics and errors as mi_sgemm_ex; an unknown config gives
 * MI_SGEMM_ERROR_INVALID_VALUE.
 */
int mi_sgemm_with_config(int kernel, int config, int trans_a, int trans_b,
                         int m, int n, int k, float alpha,
                         const float *A, int lda, const float *B, int ldb,
                         float beta, float *C, int ldc, void *stream);

/*
 * mi_sgemm_with_order -- mi_sgemm_with_config (matrix-core kernel) with the
 * workgroup order forced, for measured comparisons of the order against L2
 * reuse (page "gemm优化", section 杂项：预取缓存1， Swizzle 增强L2缓存命中).
 * The default order is xcd_remap = 1, group_m = 8: the workgroup ids the
 * hardware deals out to the 8 XCDs round-robin are renumbered so that each
 * XCD owns one contiguous range of tiles, and consecutive tiles walk down
 * groups of group_m tile rows before moving to the next tile column.
 * xcd_remap = 0 keeps the hardware numbering; group_m = 1 walks the tiles in
 * plain row-major order.  The order decides only which workgroup computes
 * which tile: the result is bitwise that of every other order.  config: as
 * mi_sgemm_with_config (< 0: automatic).  Errors as mi_sgemm_ex, plus
 * INVALID_VALUE for xcd_remap other than 0 or 1 or group_m < 1.
 */
int mi_sgemm_with_order(int config, int xcd_remap, int group_m, int trans_a, int trans_b,
                        int m, int n, int k, float alpha,
                        const float *A, int lda, const float *B, int ldb,
                        float beta, float *C, int ldc, void *stream);

/*
 * mi_sgemm_splitk_with_config -- mi_sgemm_splitk with a forced tile
 * configuration of the partial kernel (ids as for MI_SGEMM_KERNEL_MFMA;
 * config < 0 means the automatic choice) and op(A), op(B) as in mi_sgemm_ex.
 * The workspace it needs is given by
 * mi_sgemm_splitk_with_config_workspace_bytes (0 for invalid arguments or an
 * unknown config).  Same semantics and errors as mi_sgemm_splitk_ex.
 */
int mi_sgemm_splitk_with_config(int config, int trans_a, int trans_b,
                                int m, int n, int k, float alpha,
                                const float *A, int lda, const float *B, int ldb,
                                float beta, float *C, int ldc,
                                int splits, void *ws, size_t ws_bytes, void *stream);
size_t mi_sgemm_splitk_with_config_workspace_bytes(int config, int m, int n, int k,
                                                   int splits);

/*
 * mi_sgemm_streamk -- the product on a stream-K schedule, for shapes whose
 * tiles leave the last round of workgroups partly empty.  With G = grid
 * (0: one per resident workgroup slot of every CU; capped by the number of
 * (tile, k step) iterations and by 2048): when the tile count is a multiple
 * of G every tile gets a workgroup of its own, as in mi_sgemm.  Otherwise
 * all rounds of G tiles but the last full one do (data-parallel tiles), and
 * G more workgroups each take an equal share of the (tile, k step)
 * iterations of the remaining tiles (between one and two rounds' worth, or
 * all tiles when there are fewer than two rounds).  Such a workgroup
 * finishes the tiles whose whole k range falls in its share, leaves the raw
 * sums of the tiles cut at the ends of its share in its two workspace slots,
 * and a second kernel adds the parts of every cut tile in a fixed order --
 * deterministic, like mi_sgemm_splitk.  It is the big iteration over K of
 * page "GEMM优化原理" (section 基于 shared memory 计算) divided by work
 * rather than by tile.  mi_sgemm_splitk's automatic plan uses it when its
 * model prefers it; this entry forces it.  config: tile configuration (ids
 * as for MI_SGEMM_KERNEL_MFMA, < 0: the model's choice).  ws / ws_bytes: at
 * least mi_sgemm_streamk_workspace_bytes(config, m, n, k, grid) bytes, two
 * tiles per stream-K workgroup (0 for invalid arguments or when no tile is
 * shared; ws may then be NULL).  Other arguments, semantics and errors as
 * mi_sgemm_splitk_ex.
 */
int mi_sgemm_streamk(int config, int trans_a, int trans_b, int m, int n, int k, float alpha,
                     const float *A, int lda, const float *B, int ldb, float beta, float *C,
                     int ldc, int grid, void *ws, size_t ws_bytes, void *stream);
size_t mi_sgemm_streamk_workspace_bytes(int config, int m, int n, int k, int grid);

#ifdef __cplusplus
}
#endif

#endif /* MI_SGEMM_H */
