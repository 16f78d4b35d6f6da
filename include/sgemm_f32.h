/*
 * sgemm_f32.h -- single-precision matrix product C = A·B on one MI355X (gfx950).
 *
 * The operation.  For A (M x K), B (K x N) and C (M x N),
 *     C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 * as defined on the page "CUDA算子优化(4)：矩阵乘法" (section "矩阵乘法的数学定义")
 * and on the page "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结" (§三,
 * "数学公式").  This is alpha = 1, beta = 0: C is overwritten and never read.
 *
 * Layout.  All three matrices are row-major in device memory with element
 * strides (leading dimensions): A[i][k] = A[i*lda + k], B[k][j] = B[k*ldb + j],
 * C[i][j] = C[i*ldc + j].  The pages store dense rows (ld equal to the row
 * length); larger leading dimensions address sub-matrices and padded rows,
 * whose padding is never read or written.
 *
 * Arithmetic.  Products and sums are IEEE fp32 with round-to-nearest-even;
 * multiply-adds are fused.  The summation order over k is not specified
 * beyond this: any order is a correct result of the definition (its error is
 * bounded by K * 2^-24 * sum_k |A[i][k]| * |B[k][j]|).  For a fixed shape,
 * leading dimensions and algorithm, results are bitwise reproducible run to
 * run (no atomics).  NaN and Inf propagate as IEEE arithmetic dictates.
 *
 * Ownership.  The caller owns every buffer.  A, B and C are device pointers
 * (hipMalloc, torch or any other device allocation) that must stay valid
 * until the enqueued work completes.  The library allocates nothing, keeps
 * no pointer after returning, and holds no mutable global state other than
 * the per-device address of the scratch array of sgemm_f32_ex_noalloc()
 * (looked up once per device, under a lock); calls may come from several
 * host threads.
 *
 * Asynchrony.  Each call validates its arguments on the host, enqueues its
 * kernels on `stream` (0 is the null stream) and returns without waiting.
 * The caller synchronises (hipStreamSynchronize, events, ...).
 *
 * Errors (returned, never fatal; an argument error enqueues nothing):
 *   hipErrorInvalidValue   M, N or K negative; lda < max(1,K); ldb < max(1,N);
 *                          ldc < max(1,N); A or B NULL when M*N*K > 0; C NULL
 *                          when M*N > 0; the written extent of C overlapping
 *                          the read extent of A or B; unknown algorithm id;
 *                          a launch grid beyond the device's limits.
 *   otherwise              the status of the launch (for example
 *                          hipErrorNoDevice on a host without a GPU).
 * Empty cases: M == 0 or N == 0 returns hipSuccess and enqueues nothing.
 * K == 0 writes C[i][j] = 0 (the empty sum) for i < M, j < N.
 */
#ifndef SGEMM_F32_H
#define SGEMM_F32_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Algorithm ids for sgemm_f32_algo(): the rungs of the ladder the pages build,
 * from one thread per output element up to on-chip tiling, plus the rungs this
 * library adds for gfx950.  Each computes the same definition; they differ in
 * how the work is mapped, not in what is computed.
 *
 * SGEMM_F32_ALGO_NAIVE: one work-item per element of C, k loop in registers,
 *   operands read straight from global memory.  The naive kernel of page
 *   "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结" (§五) and of page
 *   "CUDA算子优化(4)：矩阵乘法" (section "版本V1朴素矩阵乘法"), with the &&
 *   bounds guard of the first page.
 * SGEMM_F32_ALGO_LDS_TILED: 16 x 16 tiles of A and B staged in LDS, one
 *   element of C per work-item, zero-filled tiles past the edges, one barrier
 *   after the tile load and one before it is overwritten.  The tiled kernel of
 *   the first page (§六, with the padded tile of §八 "避免Bank Conflict") and
 *   of page "CUDA算子优化(4)：矩阵乘法" (section "版本V1共享内存分块"); the
 *   index map is the one walked through on page "【infra之路】Tiled Matrix
 *   Multiplication详解".
 * SGEMM_F32_ALGO_VALU_REGBLOCK: the tiled kernel with an 8 x 8 block of C per
 *   work-item in registers, two LDS stages and an unrolled k loop of fused
 *   multiply-adds: the unrolling and fmaf steps of page "GPU programming with
 *   C++ and CUDA" (chapter 7) and the "optimise register use" and "double
 *   buffering" items of the first page's checklist (§八).
 * SGEMM_F32_ALGO_MFMA: the tiled kernel of "版本V1共享内存分块" with the block
 *   product done on the fp32 matrix cores (v_mfma_f32_32x32x2f32), 16-byte
 *   loads and an LDS ring: the "Tensor Core", "float4 loads" and "double
 *   buffering" items of the first page's checklist (§七, §八) on full-precision
 *   matrix cores.
 * SGEMM_F32_ALGO_SKINNY / SKINNY_N: products with at most 8 rows (columns) of
 *   C, whose arithmetic intensity I = MNK / (2(MK+KN+MN)) (page
 *   "CUDA算子优化(4)：矩阵乘法", section "计算强度") is near 0.5 flop/byte, so
 *   they are bound by memory bandwidth: the large operand is streamed once.
 * SGEMM_F32_ALGO_BF16X6: the fp32 product on the bf16 matrix cores (the
 *   "Tensor Core" step of the first page's §七 and §八), described below.
 */
#define SGEMM_F32_ALGO_AUTO 0          /* chosen from the shape */
#define SGEMM_F32_ALGO_NAIVE 1         /* one thread per element of C */
#define SGEMM_F32_ALGO_LDS_TILED 2     /* 16x16 tiles staged in LDS */
#define SGEMM_F32_ALGO_VALU_REGBLOCK 3 /* LDS double buffer, 8x8 register tiles, v_fma_f32 */
#define SGEMM_F32_ALGO_MFMA 4          /* LDS double buffer, fp32 matrix cores */
#define SGEMM_F32_ALGO_SKINNY 5        /* M <= 8: stream op(B) once (B as given: split K in the
                                          work-group; B transposed: split K across a wave) */
#define SGEMM_F32_ALGO_SKINNY_N 6      /* N <= 8: stream op(A) once (A as given: split K across
                                          a wave; A transposed: split K in the work-group) */
#define SGEMM_F32_ALGO_BF16X6 7        /* bf16 matrix cores, operands split in 3 parts (below) */
#define SGEMM_F32_ALGO_COUNT 8

/*
 * C = A·B with the algorithm chosen for the shape (SGEMM_F32_ALGO_AUTO).
 *   M, N, K      rows of A and C, columns of B and C, columns of A / rows of B.
 *   A, lda       device pointer to A (M x K), row stride lda elements.
 *   B, ldb       device pointer to B (K x N), row stride ldb elements.
 *   C, ldc       device pointer to C (M x N), row stride ldc elements; written only.
 *   stream       HIP stream the work is enqueued on.
 * Returns hipSuccess once the work is enqueued, or an error as listed above.
 */
hipError_t sgemm_f32(int M, int N, int K,
                     const float *A, int lda,
                     const float *B, int ldb,
                     float *C, int ldc,
                     hipStream_t stream);

/*
 * Same operation and contract as sgemm_f32(), forcing one algorithm of the
 * ladder (an SGEMM_F32_ALGO_* id; the rungs and the passages that define them
 * are listed above: the naive and tiled kernels of page "CUDA内存优化入门：从
 * Naive到Tiled矩阵乘法—Week2学习总结" §五 and §六 and of page
 * "CUDA算子优化(4)：矩阵乘法", sections "版本V1朴素矩阵乘法" and
 * "版本V1共享内存分块", and the unroll and fmaf steps of page "GPU programming
 * with C++ and CUDA", chapter 7).  Every algorithm accepts every valid
 * shape; SGEMM_F32_ALGO_SKINNY with M > 8 processes the rows in groups of 8,
 * SGEMM_F32_ALGO_SKINNY_N with N > 8 the columns in groups of 8.
 */
hipError_t sgemm_f32_algo(int M, int N, int K,
                          const float *A, int lda,
                          const float *B, int ldb,
                          float *C, int ldc,
                          hipStream_t stream, int algo);

/*
 * SGEMM_F32_ALGO_BF16X6 is never chosen automatically.  It computes the same
 * fp32 product on the bf16 matrix cores, the reduced-precision matrix step the
 * pages end with (their "Tensor Core" outlook): every value of A and B is split
 * exactly into three bf16 parts, x = x0 + x1 + x2, and the six part products
 * with p + q <= 2 are accumulated in fp32, smallest first.  The dropped terms
 * are below 2^-24 of each product, so the result has fp32 accuracy (within the
 * same bound as the other algorithms; all-ones, identity and small-integer
 * products are exact).  Differences from the fp32 rungs: an infinite input
 * gives NaN instead of +-Inf in its row or column (Inf times a zero part), and
 * values above about 3.39e38 in magnitude, whose bf16 rounding overflows,
 * become infinite.  Untransposed operands only.
 */

/*
 * The algorithm SGEMM_F32_ALGO_AUTO picks for these arguments (host-only:
 * no HIP call is made).  Returns an SGEMM_F32_ALGO_* id other than AUTO, or
 * -1 if the arguments are invalid.
 */
int sgemm_f32_select(int M, int N, int K,
                     const float *A, int lda,
                     const float *B, int ldb,
                     const float *C, int ldc);

/* Static, NUL-terminated name of an algorithm id ("invalid" if unknown). */
const char *sgemm_f32_algo_name(int algo);

/*
 * General form, as in the BLAS interface of the library the pages measure
 * themselves against (cuBLAS, page "CUDA算子优化(4)：矩阵乘法"):
 *     C = alpha * op(A) * op(B) + beta * C
 * with op(A) M x K and op(B) K x N, all arrays row-major:
 *   transa = SGEMM_F32_OP_N: A is the M x K array A[i*lda + k], lda >= max(1,K);
 *   transa = SGEMM_F32_OP_T: A is a K x M array and op(A)[i][k] = A[k*lda + i],
 *                            lda >= max(1,M);
 *   transb = SGEMM_F32_OP_N: B is the K x N array B[k*ldb + j], ldb >= max(1,N);
 *   transb = SGEMM_F32_OP_T: B is an N x K array and op(B)[k][j] = B[j*ldb + k],
 *                            ldb >= max(1,K);
 *   C is M x N, C[i*ldc + j], ldc >= max(1,N), read and written.
 * beta == 0 means C is not read (NaN or Inf there does not reach the result);
 * alpha == 0 or K == 0 means A and B are not read and C becomes beta*C.  The
 * scaling is alpha*sum + beta*C in fp32 after the sum, fused where possible.
 * Ownership, asynchrony, reproducibility and errors are as for sgemm_f32();
 * a transa or transb other than the two values below is hipErrorInvalidValue,
 * and A and B may be NULL when alpha == 0 or K == 0.  sgemm_f32() is
 * sgemm_f32_ex(N, N, M, N, K, 1, A, lda, B, ldb, 0, C, ldc), bit for bit.
 *
 * sgemm_f32_ex_algo() forces one rung.  AUTO, NAIVE, LDS_TILED, MFMA, SKINNY
 * and SKINNY_N accept either storage order; VALU_REGBLOCK and BF16X6 accept
 * only SGEMM_F32_OP_N for both operands (hipErrorInvalidValue otherwise).
 * AUTO uses the SKINNY and SKINNY_N rules of sgemm_f32() in every storage
 * order (SKINNY for M <= 8, else SKINNY_N for N <= 8; with A transposed and B
 * not, up to 24) and MFMA for every other product; see sgemm_f32_auto_plan() for how AUTO may split an MFMA product
 * into blocks and an edge strip.
 *
 * sgemm_f32_colmajor() takes the same arguments with every array column-major,
 * as in the reference BLAS sgemm: A is M x K (transa = N, lda >= max(1,M)) or
 * K x M (transa = T, lda >= max(1,K)), B is K x N (ldb >= max(1,K)) or N x K
 * (ldb >= max(1,N)), C is M x N with ldc >= max(1,M).  A column-major array is
 * the row-major array of its transpose, so this is the row-major product
 * C^T = alpha * op(B)^T * op(A)^T + beta * C^T, computed by sgemm_f32_ex().
 */
#define SGEMM_F32_OP_N 0 /* operand as stored */
#define SGEMM_F32_OP_T 1 /* operand transposed */

hipError_t sgemm_f32_ex(int transa, int transb, int M, int N, int K, float alpha,
                        const float *A, int lda,
                        const float *B, int ldb, float beta,
                        float *C, int ldc,
                        hipStream_t stream);
hipError_t sgemm_f32_ex_algo(int transa, int transb, int M, int N, int K, float alpha,
                             const float *A, int lda,
                             const float *B, int ldb, float beta,
                             float *C, int ldc,
                             hipStream_t stream, int algo);
hipError_t sgemm_f32_colmajor(int transa, int transb, int M, int N, int K, float alpha,
                              const float *A, int lda,
                              const float *B, int ldb, float beta,
                              float *C, int ldc,
                              hipStream_t stream);

/*
 * Tile configurations of the matrix-core rung (SGEMM_F32_ALGO_MFMA), for
 * tuning and tests.  The rung tiles C into BM x BN blocks, one work-group per
 * block, as in the shared-memory tiling of the page "CUDA算子优化(4)：矩阵乘法"
 * (section "版本V1共享内存分块"); a configuration fixes the block and k-window
 * sizes, the block of C held by each wave, the number of wave groups that split
 * each k window, and the number of LDS stages.  SGEMM_F32_ALGO_MFMA picks one
 * from a cost model of the shape.
 *
 * sgemm_f32_mfma_tiles()      number of configurations (ids 0 .. count-1).
 * sgemm_f32_mfma_tile_name()  static description such as
 *                             "256x256x16 w128x128 k1 s3" (BM x BN x BK, wave
 *                             block, wave groups, stages; the 128 x 192
 *                             configuration runs eight 32 x 96 waves in one
 *                             group instead when B alone is transposed); NULL
 *                             for an unknown id.
 * sgemm_f32_mfma_select()     the id SGEMM_F32_ALGO_MFMA uses for an M x N x K
 *                             product on a device with `compute_units` CUs
 *                             (<= 0 means 256); host-only, no HIP call; -1 if
 *                             M, N or K is negative.
 * sgemm_f32_mfma_tile()       same operation and contract as sgemm_f32(), on the
 *                             matrix-core rung with configuration `tile`; an
 *                             unknown id is hipErrorInvalidValue.
 * sgemm_f32_ex_mfma_tile()    the same for the general form of sgemm_f32_ex().
 */
int sgemm_f32_mfma_tiles(void);
const char *sgemm_f32_mfma_tile_name(int tile);
int sgemm_f32_mfma_select(int M, int N, int K, int compute_units);
hipError_t sgemm_f32_mfma_tile(int M, int N, int K,
                               const float *A, int lda,
                               const float *B, int ldb,
                               float *C, int ldc,
                               hipStream_t stream, int tile);
hipError_t sgemm_f32_ex_mfma_tile(int transa, int transb, int M, int N, int K, float alpha,
                                  const float *A, int lda,
                                  const float *B, int ldb, float beta,
                                  float *C, int ldc,
                                  hipStream_t stream, int tile);

/*
 * Split-k with a caller-provided workspace (the library still allocates
 * nothing).  Products with few blocks of C and a long k (for example 128 x 128
 * x 65536) leave most CUs idle on the matrix-core rung.  Given room,
 * sgemm_f32_ex_ws() splits k into S slices:
 * the first kernel writes each slice's unscaled partial product to a plane of
 * the workspace (S planes of M x N floats, row stride N), the second forms
 *     C = alpha * (plane 0 + plane 1 + ... + plane S-1) + beta * C
 * adding the planes in an order fixed by (M, N, S), so results are
 * reproducible run to run (they differ from sgemm_f32_ex() only in summation
 * order, within the same bound).  The choice of S and of the block
 * configuration comes from the same cost model as the rest of the automatic
 * choice; the split is taken only when modelled at least 10% faster, and the
 * planes never take more than 64 MiB.
 *
 * sgemm_f32_workspace_size()  bytes sgemm_f32_ex_ws() would use for these
 *                             arguments on the current device (0: no split;
 *                             also 0 for invalid arguments).  No GPU work.
 * sgemm_f32_ex_ws()           the general form of sgemm_f32_ex() with a device
 *                             workspace of workspace_bytes bytes, 16-byte
 *                             aligned, owned by the caller and not overlapping
 *                             A, B or C (hipErrorInvalidValue otherwise).  With
 *                             workspace == NULL or too few bytes it is exactly
 *                             sgemm_f32_ex().  Calls that overlap in time must
 *                             not share a workspace.
 */
size_t sgemm_f32_workspace_size(int transa, int transb, int M, int N, int K);
hipError_t sgemm_f32_ex_ws(int transa, int transb, int M, int N, int K, float alpha,
                           const float *A, int lda,
                           const float *B, int ldb, float beta,
                           float *C, int ldc,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * For callers that cannot allocate device memory (work recorded under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sgemm_f32_ex_noalloc() is sgemm_f32_ex_ws() with the workspace taken from a
 * device array inside the library instead of from the caller.
 *
 * The array is SGEMM_F32_SCRATCH_BYTES (32 MiB) of device memory, one copy per
 * GPU the library runs on, held until the process ends; its address on a device
 * is looked up on the first call made with that device current.  The call
 * allocates nothing and calls no allocating routine.  When the split planner
 * (the same as for sgemm_f32_ex_ws()) wants no split, the call is
 * sgemm_f32_ex(); when it wants one whose planes fit in the array, the planes go
 * there and the result is bit for bit that of sgemm_f32_ex_ws() with a large
 * enough workspace; when the planes would need more than
 * SGEMM_F32_SCRATCH_BYTES (sgemm_f32_workspace_size() tells beforehand), the
 * call returns hipErrorInvalidValue and enqueues nothing.
 *
 * Every call on one GPU shares that GPU's array, and each call overwrites the
 * part it uses (no part needs to start at zero), so calls whose work overlaps
 * in time on one GPU (on different streams, or from several host threads)
 * race and give wrong results: order them on one stream or with events.  Other
 * arguments, errors and asynchrony are as for sgemm_f32_ex().
 */
#define SGEMM_F32_SCRATCH_BYTES (32u << 20)

hipError_t sgemm_f32_ex_noalloc(int transa, int transb, int M, int N, int K, float alpha,
                                const float *A, int lda,
                                const float *B, int ldb, float beta,
                                float *C, int ldc,
                                hipStream_t stream);

/*
 * How SGEMM_F32_ALGO_AUTO runs an M x N x K product with the given storage
 * orders on a device with `compute_units` CUs (<= 0 means 256); host-only, no
 * HIP call.  Returns the algorithm id AUTO resolves to (as sgemm_f32_select()
 * for untransposed operands), or -1 for invalid arguments.  *m_main and
 * *n_main receive the extent of C that the chosen algorithm covers; when the
 * algorithm is SGEMM_F32_ALGO_MFMA and N (M) lies 1 to 8 past a multiple of
 * 32, AUTO may leave the last N % 32 columns (M % 32 rows) to a second kernel
 * sized for that strip (the SKINNY_N or SKINNY kernel) when the tile cost model says the
 * two launches finish sooner: the columns [n_main, N) of all rows, then the
 * rows [m_main, M) of columns [0, n_main).  The blocks of the main part use
 * configuration sgemm_f32_mfma_select(m_main, n_main, K, compute_units).
 * Every element of C is computed by exactly one kernel, so results are still
 * reproducible run to run; they match the forced MFMA rung within the error
 * bound, not bit for bit, in the strip.
 */
int sgemm_f32_auto_plan(int transa, int transb, int M, int N, int K, int compute_units,
                        int *m_main, int *n_main);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_H */
