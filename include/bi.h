/*
 * bi.h -- batch-invariant GEMM family and RMSNorm for AMD MI355X (gfx950).
 *
 * Contract shared by every entry point:
 *   - Output row i is a function of input row i (and the weights) only: it is
 *     bitwise identical whether computed with M = 1, with the full batch, or
 *     with the rows in any order, and identical from run to run.  This is the
 *     property the vLLM-Ascend "Batch Invariance" guide states in its opening
 *     section (output independent of batch size and request order), which
 *     the vLLM PR #39912 summary page checks row by row (section "key source
 *     snippets", test_nvfp4_gemm_batch_invariance) and the vLLM PR #51292 page
 *     checks run to run (section "Test Plan": 8 identical runs, 1 distinct
 *     output).
 *   - The arithmetic of each output depends on the operation and on (N, K)
 *     (H for RMSNorm) only, never on M: one MFMA instruction, one ascending
 *     K order, one lane accumulating each output over the whole K range,
 *     no split-K, no stream-K, no atomics.  The PR #39912 page calls the
 *     M-bucketed kernel configurations the thing batch-invariant mode must
 *     avoid (section "implementation breakdown": only the default config with
 *     a persistent scheduler), and the PR #51292 page names size-gated kernel
 *     selection as the bug class (root-cause comment).  Which kernel runs
 *     that arithmetic does depend on M: at small M a streaming kernel that
 *     spreads column items of the weight over the whole chip, else the tiled
 *     kernel with a tile shape picked by a cost model of M and N (the fewest
 *     rounds of tiles over the compute units, weighted by each shape's
 *     measured round time).  bi_plan_regimes lists every such choice and its
 *     row range; all of them give the same bits.
 *   - There is no mode switch and no environment variable: invariance is
 *     unconditional (the PR #39912 page lists a cached mode flag as a risk,
 *     section "risks and impact").
 *
 * Memory and streams:
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates or frees device memory and keeps no per-call state;
 *     calls are thread-safe.  The one memory it holds is the scratch array
 *     of bi_mla_decode_noalloc (BI_MLA_SCRATCH_BYTES per GPU, reserved with
 *     the library's code).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.  Kernel faults surface at
 *     the caller's next synchronisation.
 *   - bf16 data is passed as raw 16-bit patterns; all strides are in elements.
 *
 * Errors (returned as bi_status, never by aborting):
 *   - BI_ERR_NULL: a required pointer is NULL (pointers are not required
 *     when M == 0, which is a valid no-op).
 *   - BI_ERR_SHAPE: a negative M, a non-positive N/K/H/batch, a leading
 *     dimension smaller than its row, or a K/H that is not a multiple of 8
 *     (of 32 for NVFP4).
 *   - BI_ERR_ALIGN: a pointer not 16-byte aligned, or a leading dimension or
 *     batch stride that is not a multiple of 8 elements (of 32 for NVFP4 A).
 *   - BI_ERR_ALIAS: the output range overlaps an input range.
 *   - BI_ERR_UNSUPPORTED: no plan for this shape (an index that would
 *     overflow 32 bits inside a kernel: a dimension above 2^31-1, a leading
 *     dimension of 2^22 elements or more).  There is never a silent fallback to
 *     a non-invariant path: the fail-loud rule of the PR #51292 review thread.
 *   - BI_ERR_HIP: the HIP runtime refused the launch or a device query.
 *   - BI_ERR_VALUE: a scalar argument outside its domain (a global scale
 *     that is not a finite number > 0).
 */
#ifndef BI_H
#define BI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bi_status {
    BI_OK = 0,
    BI_ERR_NULL = 1,
    BI_ERR_SHAPE = 2,
    BI_ERR_ALIGN = 3,
    BI_ERR_ALIAS = 4,
    BI_ERR_UNSUPPORTED = 5,
    BI_ERR_HIP = 6,
    BI_ERR_VALUE = 7
} bi_status;

typedef enum bi_a_format {
    BI_A_BF16 = 0,  /* A is bf16 [M,K] */
    BI_A_NVFP4 = 1  /* A is NVFP4: codes [M,K/2] + E4M3 scales [M,K/16] */
} bi_a_format;

typedef enum bi_op {
    BI_OP_GEMM = 0,
    BI_OP_BMM = 1,
    BI_OP_NVFP4_GEMM = 2,
    BI_OP_RMSNORM = 3,
    BI_OP_NVFP4_QUANT = 4,
    BI_OP_REDUCE_RMSNORM = 5,
    BI_OP_GROUPED_GEMM = 6
} bi_op;

/*
 * The fixed recipe for one (op, N, K) -- or (op, H) for RMSNorm.  Every
 * field is a function of op and the shape key only.
 *   GEMM family: output tile bm x bn, bk columns of K staged per step through
 *   LDS, `waves` wavefronts per workgroup, MFMA block mfma_m x mfma_n x mfma_k
 *   (bf16 inputs, fp32 accumulation), K visited in ascending chunks of
 *   mfma_k, `lds_stages` LDS buffers.
 *   RMSNorm: `threads` threads per row, each summing `chunks_per_thread`
 *   16-byte chunks of the row; bm = bn = bk = 0.
 */
typedef struct bi_plan {
    int32_t op;
    int32_t bm, bn, bk;
    int32_t mfma_m, mfma_n, mfma_k;
    int32_t waves;
    int32_t lds_stages;
    int32_t threads;
    int32_t chunks_per_thread;
    int32_t reserved[5];
} bi_plan;

/*
 * Launch options for the *_ex entry points.  They change only which lanes
 * and workgroups compute which outputs, never how any output element is
 * computed, so results are bitwise identical for every value -- that is what
 * the grid- and tile-override invariance tests check.  They exist for those
 * tests and for tuning sweeps; production calls pass NULL.
 *   max_workgroups: cap on the persistent grid (0 = the library's default,
 *     the device's compute-unit count times the tiles one unit holds); for
 *     the GEMMs served by the streaming kernels (M <= 16; up to M = 128 for
 *     bf16 weights with N <= 12288 and to M = 64 for NVFP4 weights with
 *     K % 128 == 0; no tile_variant), a cap on the streaming wavefronts.
 *   tile_variant: GEMM family only; 0 = the plan's tile shape, v > 0 = the
 *     compiled tile shape v-1 (see bi_tile_shape).  BI_ERR_SHAPE if out of
 *     range.
 *   pipeline_depth: the streaming kernels only; weight load units in flight per
 *     wavefront (0 = the library's choice; otherwise rounded down to a
 *     supported power of two that divides the unit count).
 *   fixed_plan: GEMM family; nonzero = the tiled kernel with one tile shape
 *     for the operation, its operand formats and (N, K) at every M -- for a
 *     dense or NVFP4 GEMM with a bf16 A the shape bi_plan_query reports, for
 *     the grouped GEMM its many-rows shape -- so neither the kernel nor the
 *     tile is chosen from M.  For callers that require that by construction;
 *     the default choice (which also uses M) gives the same bits, faster at
 *     small and middle M.  tile_variant, when set, takes precedence; the
 *     BMM's plan never depends on M.
 */
typedef struct bi_launch_opts {
    int32_t max_workgroups;
    int32_t tile_variant;
    int32_t pipeline_depth;
    int32_t fixed_plan;
    int32_t reserved[4];
} bi_launch_opts;

/*
 * bi_gemm: Y = A . B^T, bf16 in, fp32 accumulation, bf16 out (round to
 * nearest even).  Operand orientation as in the unit test of the vLLM PR
 * #39912 summary page (section "key source snippets": a [m,k], b [n,k],
 * out [m,n]); the dense bf16 case of the batch-invariant GEMM family.
 *   A: bf16 [M,K], row stride lda >= K.
 *   B: bf16 [N,K], row stride ldb >= K (the weight; rows are output columns).
 *   Y: bf16 [M,N], row stride ldy >= N; must not overlap A or B.
 *   Y[i][j] = bf16_rne( fp32 MFMA chain over k ascending of A[i][k]*B[j][k] ).
 */
bi_status bi_gemm(const void *A, int64_t lda, const void *B, int64_t ldb, void *Y,
                  int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * bi_bmm: per head h < batch, Y[h] = A[h] . B[h], the batched GEMM the vLLM
 * batch-invariance tracking issue lists as a performance item (page
 * "[Feature]: Batch Invariant Feature and Performance Optimization", TODO
 * "BMM optimization").  Heads are independent; each head's rows obey the
 * row contract above, and a head's output does not depend on which other
 * heads are in the call.
 *   A: bf16 [batch,M,K], head stride sA, row stride lda >= K.
 *   B: bf16 [batch,K,N] (K rows of N), head stride sB, row stride ldb >= N.
 *   Y: bf16 [batch,M,N], head stride sY, row stride ldy >= N.
 */
bi_status bi_bmm(const void *A, int64_t sA, int64_t lda, const void *B, int64_t sB,
                 int64_t ldb, void *Y, int64_t sY, int64_t ldy, int64_t batch, int64_t M,
                 int64_t N, int64_t K, void *stream);

/*
 * bi_nvfp4_gemm: Y = alpha * (A . W^T) with W in NVFP4, the operation of
 * cutlass_scaled_fp4_mm in the vLLM PR #39912 unit test (summary page,
 * section "key source snippets"; alpha = 1 / (global scale of A * global
 * scale of W), or 1 / global scale of W when A is bf16).
 *   W: codes uint8 [N,K/2], dense; element 2j of a row in the low nibble of
 *      byte j, element 2j+1 in the high nibble; each nibble an FP4 E2M1 code.
 *   W_scales: uint8 [N,K/16], dense; one FP8 E4M3 (fn) scale per 16
 *      consecutive elements of a row.
 *   A (a_fmt == BI_A_BF16): bf16 [M,K], row stride lda elements; A_scales
 *      unused (may be NULL).
 *   A (a_fmt == BI_A_NVFP4): codes uint8 [M,K/2] with row stride lda/2 bytes,
 *      A_scales uint8 [M,K/16] with row stride lda/16 bytes; lda % 32 == 0.
 *   Y: bf16 [M,N], row stride ldy.  K % 32 == 0.
 *   Each weight element is decoded exactly to bf16 (e2m1 value * e4m3 scale
 *   has at most 6 significant bits); the product with alpha is one fp32
 *   multiply in the epilogue, then bf16 round-to-nearest-even.  With
 *   alpha == 1 the result is bitwise that of bi_gemm on the decoded weights.
 */
bi_status bi_nvfp4_gemm(const void *A, const void *A_scales, int a_fmt, int64_t lda,
                        const void *W, const void *W_scales, float alpha, void *Y,
                        int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * bi_rmsnorm: Y[i][h] = bf16_rne( x[i][h] * r_i * gamma[h] ),
 * r_i = rsqrt( (1/H) * sum_h x[i][h]^2 + eps ), fp32 arithmetic.  RMSNorm is
 * the row reduction fused after the tensor-parallel all-reduce on the vLLM
 * PR #51292 page (section "Purpose").  The sum over a row has one fixed order
 * for a given H: per-thread strided partial sums, a 64-lane butterfly, then
 * the wave partials in wave order.
 *   X: bf16 [M,H], row stride ldx.  gamma: bf16 [H].  Y: bf16 [M,H], row
 *   stride ldy (may equal X for an in-place update; any other overlap is
 *   BI_ERR_ALIAS).  H % 8 == 0 and H <= 32768.
 */
bi_status bi_rmsnorm(const void *X, int64_t ldx, const void *gamma, float eps, void *Y,
                     int64_t ldy, int64_t M, int64_t H, void *stream);

/*
 * bi_nvfp4_quant: row-local NVFP4 quantisation of bf16 activations, the
 * scaled_fp4_quant(x, global_scale) -> (codes, block scales) step that feeds
 * the W4A4 GEMM in the vLLM PR #39912 unit test (summary page, section "key
 * source snippets").  The pages do not define it; per block of 16
 * consecutive elements of a row this library computes, every step one IEEE
 * fp32 operation with round to nearest even:
 *   amax = max |x|;  v = min((amax * g) / 6, 448);
 *   scale = the E4M3 (fn) code nearest to v, ties to the even code;
 *   s = its value; if s == 0 every element code is 0, else r = g / s and each
 *   element code is the E2M1 magnitude code nearest to |x| * r (ties to the
 *   even code, saturating at 6), with the sign bit set for a negative x whose
 *   magnitude code is not 0.
 * Each row's bytes depend only on that row and g, so g must be fixed by the
 * caller (computed once, e.g. from a calibration batch) and not recomputed
 * per batch; then a row quantised alone equals the same row quantised inside
 * any batch.  The output is the NVFP4 A operand of bi_nvfp4_gemm with
 * a_fmt = BI_A_NVFP4 and lda = ldq.
 *   X: bf16 [M,K], row stride ldx elements (ldx % 8 == 0), 16-byte aligned.
 *   Q: codes uint8 [M,K/2], row stride ldq/2 bytes; element 2j of a row in
 *      the low nibble of byte j, element 2j+1 in the high nibble.  4-byte
 *      aligned.
 *   Q_scales: uint8 [M,K/16], row stride ldq/16 bytes.
 *   ldq >= K and ldq % 16 == 0 (BI_ERR_ALIGN otherwise; bi_nvfp4_gemm needs
 *   ldq % 32 == 0 and 16-byte aligned buffers to consume the result);
 *   K % 16 == 0.
 *   g: the global scale, finite and > 0, else BI_ERR_VALUE.
 *   Q and Q_scales must not overlap X or each other (BI_ERR_ALIAS).
 *   M * K / 8 >= 2^30 is BI_ERR_UNSUPPORTED.
 */
bi_status bi_nvfp4_quant(const void *X, int64_t ldx, float g, void *Q, void *Q_scales,
                         int64_t ldq, int64_t M, int64_t K, void *stream);

/*
 * bi_reduce_rmsnorm: the one-GPU share of the all-reduce + RMSNorm pair that
 * the vLLM PR #51292 page fuses (section "Purpose") and whose reduction must
 * run in one fixed order for batch invariance (its root-cause comment: a
 * size-dependent reduction path; its test plan: 8 identical runs, 1 distinct
 * output).  The inputs are the n_partials partial outputs of a row-parallel
 * layer (one per tensor-parallel rank), summed in rank order:
 *   R[i][h] = bf16_rne( ((t_0 + t_1) + t_2) + ... ) in fp32, the terms t
 *             being residual[i][h] (when residual != NULL) and then
 *             partials[0][i][h], ..., partials[n_partials-1][i][h], each
 *             widened exactly from bf16; the first term starts the sum;
 *   Y = RMSNorm(R) by the very instruction sequence of bi_rmsnorm, so Y is
 *       bitwise bi_rmsnorm(R, gamma, eps).
 * Each element's sum order is fixed by n_partials alone, never by M, the
 * grid or the row.  Changing the order of the partials may change bits;
 * the rank order is the contract.
 *   partials: HOST array of n_partials device pointers, each bf16 [M,H] with
 *     row stride ldp; 1 <= n_partials <= 8 (BI_ERR_SHAPE otherwise).
 *   residual: bf16 [M,H], row stride ldres, or NULL.
 *   gamma: bf16 [H].  R, Y: bf16 [M,H], row strides ldr, ldy.
 *   R may be the residual itself (same pointer and stride: an in-place
 *   residual update); every other overlap between R, Y and the inputs is
 *   BI_ERR_ALIAS.  H % 8 == 0 and H <= 32768, as for bi_rmsnorm.
 */
bi_status bi_reduce_rmsnorm(const void *const *partials, int n_partials, int64_t ldp,
                            const void *residual, int64_t ldres, const void *gamma, float eps,
                            void *R, int64_t ldr, void *Y, int64_t ldy, int64_t M, int64_t H,
                            void *stream);

/*
 * bi_grouped_gemm: the grouped GEMM of a mixture-of-experts layer.  The
 * vLLM-Ascend "Batch Invariance" guide lists MoE layers among the operations
 * whose results must not depend on batch composition; what batch
 * composition changes there is how many tokens each expert receives.  Rows
 * group_offsets[e] .. group_offsets[e+1]-1 of A (tokens sorted by expert) are
 * multiplied by expert e's weight:
 *   Y[t] = A[t] . W_e^T, W_e = bf16 [N,K] at W + e*sW (row stride ldw).
 * Each row is computed exactly as bi_gemm computes it for (N, K) -- the same
 * tile recipe, MFMA chain and K order -- so Y[t] is bitwise bi_gemm of row t
 * alone with W_e, whatever the other groups' sizes.
 *   A: bf16 [T,K], row stride lda.  Y: bf16 [T,N], row stride ldy.
 *   group_offsets: DEVICE int64 [E+1], group_offsets[0] = 0, ascending,
 *     group_offsets[E] = T; it is read only by the kernel (no host sync), which
 *     clamps every offset to [0, T], so malformed offsets never reach memory
 *     outside A and Y (their rows are then unspecified).  8-byte aligned.
 *   E >= 1 experts; sW >= (N-1)*ldw + K when E > 1; K % 8 == 0.  T == 0 is
 *   a no-op.  The kernel enumerates only the experts' non-empty tiles (at most
 *   (ceil(T/bm) + E) * ceil(N/bn)), so any routing spreads evenly over the
 *   persistent grid.  The tile shape follows N and the average rows per
 *   expert, ceil(T / E) (bi_plan_regimes lists the ranges); every shape
 *   gives the same bits.
 */
bi_status bi_grouped_gemm(const void *A, int64_t lda, const void *W, int64_t ldw, int64_t sW, void *Y,
                          int64_t ldy, const int64_t *group_offsets, int64_t E, int64_t T, int64_t N,
                          int64_t K, void *stream);

/*
 * bi_mla_decode: one decode step of attention over a latent KV cache, the
 * MLA form in which the key and value projections are absorbed into the
 * query and output (the vLLM batch-invariance tracking issue lists the MLA
 * attention backends among the operators batch-invariant mode must cover;
 * the vLLM-Ascend "Batch Invariance" guide requires deterministic attention).
 * Every cached token t < L_b of request b holds one latent row kv_t of Dqk
 * components, used whole as the key and its first Dv components as the
 * value:
 *   s_t = scale * (q . kv_t),  p = softmax over t < L_b of s,
 *   out[b][h] = sum over t of p_t * kv_t[0:Dv].
 * The order of every sum is fixed by L_b, Dqk and Dv alone: out[b][h] is
 * bitwise the same whatever other requests share the call, whatever their
 * lengths, B, H, the launch options and whether a workspace is passed.
 * In fp32, for Dqk in 545..576 with Dv in 385..512 (DeepSeek's 576 / 512),
 * Dqk in 97..128 or 33..64 with Dv <= 128 (the matrix-core kernel):
 * scores are MFMA chains over d ascending, weights the hardware exp2 of
 * (s_t - running max) * log2(e), the weighted values summed per 1024-token
 * chunk in a fixed order and the chunks folded in ascending order, one
 * division by the weight sum, bf16 round to nearest even.  Other shapes use
 * fp32 fma chains with one max over the whole request and no chunks.
 *   q: bf16 [B,H,Dqk] dense.  kv: bf16 [B,Lmax,Dqk] dense (request b's
 *     cache is Lmax contiguous rows; rows at or past L_b are never read).
 *   lens: DEVICE int32 [B], 4-byte aligned; read only by the kernels, which
 *     clamp each to [0, Lmax].  A request with L_b = 0 gets zeros.
 *   out: bf16 [B,H,Dv] dense; must not overlap q, kv or lens.
 *   workspace: NULL, or caller-owned device memory of at least
 *     bi_mla_decode_workspace_size() bytes, 16-byte aligned, overlapping
 *     nothing else (BI_ERR_SHAPE if too small).  With it, and when the
 *     (request, 16-head group) pairs are fewer than the device's compute
 *     units, every 1024-token chunk of every request gets its own workgroup
 *     (first chunks first) and a second kernel folds the chunks: the same
 *     bits, more of the chip busy.  Its contents need no initialisation and
 *     are clobbered.
 *   Dqk % 8 == 0, Dqk <= 1024; Dv % 8 == 0, Dv <= Dqk, Dv <= 1024;
 *   Lmax <= 16384.  q, kv, out 16-byte aligned.  scale finite
 *   (BI_ERR_VALUE otherwise).  B == 0 or H == 0 is a no-op.
 */
bi_status bi_mla_decode(const void *q, const void *kv, const int32_t *lens, float scale, void *out,
                        int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, void *workspace,
                        int64_t workspace_bytes, void *stream);

/*
 * bi_mla_decode_workspace_size: *bytes = the workspace bi_mla_decode uses
 * for this shape (0 when the shape is served without one; a workspace
 * passed then is ignored).  Validates the shape as bi_mla_decode does.
 * Host-only; makes no HIP call.
 */
bi_status bi_mla_decode_workspace_size(int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv,
                                       int64_t *bytes);

/*
 * bi_mla_decode_noalloc: bi_mla_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It takes no workspace and calls no
 * allocator: when the chunked schedule applies (fewer (request, 16-head
 * group) pairs than compute units and a shape with a nonzero
 * bi_mla_decode_workspace_size), its chunk partials go to a scratch array
 * the library holds on each GPU, BI_MLA_SCRATCH_BYTES (32 MiB) large,
 * reserved when the library's code is loaded on that GPU and kept until
 * the process ends.  The outputs are bitwise those of bi_mla_decode.
 *   Arguments, layouts, ownership and the other errors are bi_mla_decode's.
 *   BI_ERR_UNSUPPORTED when the chunked schedule would need more than
 *   BI_MLA_SCRATCH_BYTES (workspace size above it and fewer pairs than
 *   compute units); the caller can then use bi_mla_decode with a workspace.
 *   Every call on one GPU shares that GPU's array and overwrites it; calls
 *   that overlap in time on one GPU (e.g. on two streams) race and give
 *   undefined results.  Calls on one stream are ordered and safe.  The
 *   array needs no initialisation: every partial is written before it is
 *   read within the call.
 */
#define BI_MLA_SCRATCH_BYTES ((int64_t)32 << 20)
bi_status bi_mla_decode_noalloc(const void *q, const void *kv, const int32_t *lens, float scale, void *out,
                                int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, void *stream);

/* The *_ex variants take launch options (may be NULL = defaults). */
bi_status bi_gemm_ex(const void *A, int64_t lda, const void *B, int64_t ldb, void *Y,
                     int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream,
                     const bi_launch_opts *opts);
bi_status bi_bmm_ex(const void *A, int64_t sA, int64_t lda, const void *B, int64_t sB,
                    int64_t ldb, void *Y, int64_t sY, int64_t ldy, int64_t batch, int64_t M,
                    int64_t N, int64_t K, void *stream, const bi_launch_opts *opts);
bi_status bi_nvfp4_gemm_ex(const void *A, const void *A_scales, int a_fmt, int64_t lda,
                           const void *W, const void *W_scales, float alpha, void *Y,
                           int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream,
                           const bi_launch_opts *opts);
bi_status bi_rmsnorm_ex(const void *X, int64_t ldx, const void *gamma, float eps, void *Y,
                        int64_t ldy, int64_t M, int64_t H, void *stream,
                        const bi_launch_opts *opts);
bi_status bi_reduce_rmsnorm_ex(const void *const *partials, int n_partials, int64_t ldp,
                               const void *residual, int64_t ldres, const void *gamma, float eps,
                               void *R, int64_t ldr, void *Y, int64_t ldy, int64_t M, int64_t H,
                               void *stream, const bi_launch_opts *opts);
bi_status bi_grouped_gemm_ex(const void *A, int64_t lda, const void *W, int64_t ldw, int64_t sW, void *Y,
                             int64_t ldy, const int64_t *group_offsets, int64_t E, int64_t T, int64_t N,
                             int64_t K, void *stream, const bi_launch_opts *opts);
bi_status bi_nvfp4_quant_ex(const void *X, int64_t ldx, float g, void *Q, void *Q_scales,
                            int64_t ldq, int64_t M, int64_t K, void *stream,
                            const bi_launch_opts *opts);
bi_status bi_mla_decode_ex(const void *q, const void *kv, const int32_t *lens, float scale, void *out,
                           int64_t B, int64_t H, int64_t Lmax, int64_t Dqk, int64_t Dv, void *workspace,
                           int64_t workspace_bytes, void *stream, const bi_launch_opts *opts);

/*
 * bi_plan_query: the recipe the library uses for (op, N, K); for
 * BI_OP_RMSNORM and BI_OP_REDUCE_RMSNORM pass H as N and 0 as K (the two
 * share one row recipe); for BI_OP_NVFP4_QUANT pass K as N and
 * 0 as K (threads = 256 per workgroup, chunks_per_thread = 1: one thread per
 * 8 elements).  There is no M argument: the per-element recipe does not
 * depend on it.  For the dense and NVFP4 GEMMs the tile fields describe the
 * shape of calls with more than 4096 rows (for the grouped GEMM, more than
 * 4096 rows per expert on average); smaller calls may run another kernel or
 * shape (bi_plan_regimes lists them) with the same bits.  Returns
 * BI_ERR_SHAPE or BI_ERR_UNSUPPORTED for keys the matching entry point would
 * reject.  Host-only; makes no HIP call.
 */
bi_status bi_plan_query(int op, int64_t N, int64_t K, bi_plan *out);

/*
 * The kernels that serve the GEMM family.  Each runs the per-element chain
 * of bi_plan_query's recipe for (N, K) -- one 16x16x32 bf16 MFMA per 32-wide
 * K chunk in ascending order from +0, fp32 accumulation by one lane for the
 * whole K range, (alpha x) then bf16 round to nearest even -- so a row's bits
 * do not depend on which kernel computes it.
 */
typedef enum bi_kernel_kind {
    BI_KERNEL_TILED = 0,           /* persistent tiled kernel, bm x bn tiles (classic schedule) */
    BI_KERNEL_TILED_PINGPONG = 1,  /* the same tile, wavefronts alternating load and MFMA phases */
    BI_KERNEL_STREAM_A_LDS = 2,    /* weight streamed into registers in column items, A staged in LDS */
    BI_KERNEL_STREAM_REG = 3,      /* weight and A fragments streamed into registers, column items */
    BI_KERNEL_STREAM_RING = 4,     /* weight streamed through a per-wavefront LDS ring, column items */
    BI_KERNEL_BMM_STREAM = 5,      /* BMM: a 128-column B block kept in LDS, A streamed in 64-row tiles */
    BI_KERNEL_STREAM_A_CHUNKS = 6  /* weight streamed into registers in column items, A in LDS in K chunks */
} bi_kernel_kind;

/*
 * One row range of the kernel choice: calls with m_min <= M <= m_max run
 * `kernel` (m_max = 2^31-1: no bound).  row_blocks: 16-row MFMA blocks of A
 * that each weight fragment feeds (tiled: bm / 16); cols: output columns per
 * work item (tiled: bn); a_pairs: 1 when one load carries A rows 0-7 of two
 * K chunks; a_rows_staged: rows of A the LDS-ring kernel stages (4, 8, 16);
 * tile_variant: the tiled kernels' shape as bi_launch_opts.tile_variant
 * numbers it (1 + the bi_tile_shape index), 0 for the streaming kernels.
 */
typedef struct bi_regime {
    int32_t kernel;
    int32_t m_min, m_max;
    int32_t row_blocks;
    int32_t cols;
    int32_t a_pairs;
    int32_t a_rows_staged;
    int32_t tile_variant;
} bi_regime;

/*
 * bi_plan_regimes: every kernel an (op, N, K) call can run, with the row
 * ranges that select it, in ascending M; they cover M >= 1 with no gap.
 * This is the host's whole kernel-choice rule: the choice depends on M as
 * well as (op, N, K) -- a departure from a single tile per (N, K) -- and
 * never changes an output bit (every kernel runs the same chain; the
 * bitwise tests cross every edge listed here).
 *   a_fmt: BI_A_BF16, or BI_A_NVFP4 for an NVFP4 A (BI_OP_NVFP4_GEMM only).
 *   cus: compute units of the device the calls run on (the edges depend on
 *     it: the A-in-LDS limit 10 * M * cus <= 7 * N and the cost model's
 *     rounds of tiles), or 0 for the current device (one HIP attribute
 *     query).  Above 4096 rows the choice no longer changes with M.
 *   BI_OP_GROUPED_GEMM: M stands for the average rows per expert,
 *     ceil(T / E).
 *   out: room for `capacity` entries; *count = the number of regimes
 *   (BI_ERR_SHAPE, with *count set, when capacity is too small).
 *   Ops other than the GEMM family: BI_ERR_UNSUPPORTED.
 */
bi_status bi_plan_regimes(int op, int64_t N, int64_t K, int a_fmt, int cus, bi_regime *out, int capacity,
                          int *count);

/*
 * bi_tile_shape: describe compiled tile shape v (0-based) of the GEMM
 * mainloop: out->bm, bn, bk, waves, lds_stages and the MFMA block are filled,
 * out->op is -1.  Returns BI_ERR_SHAPE when v is out of range, and
 * BI_ERR_NULL for a NULL out.  Host-only.
 */
bi_status bi_tile_shape(int v, bi_plan *out);

/*
 * Measurement probes.  Not part of the batch-invariant path: they measure
 * the ceilings its kernels are reported against (the published peaks assume
 * a clock and a memory efficiency the machine may not reach under load).
 *
 * bi_probe_mfma: `grid` workgroups of 8 wavefronts; each wavefront issues
 *   iters * 8 v_mfma_f32_16x16x32_bf16 (the hot path's instruction) on eight
 *   independent accumulators, operands in registers.  The call performs
 *   grid * 8 * iters * 8 * 16384 flops.  out: device uint64 [grid * 8 * 3],
 *   8-byte aligned; per wavefront: shader-clock cycles of its loop
 *   (s_memtime), ticks of the constant 100 MHz clock over the same loop
 *   (s_memrealtime), and a sink word; cycles / (ticks / 1e8) is the clock
 *   the loop ran at.  iters in [1, 2^40], grid >= 1.
 * bi_probe_read: reads `bytes` of `src` (device, 16-byte aligned, bytes %
 *   16 == 0) once, with 16-byte loads from grid * 256 threads, folding them
 *   into sink (device uint32 [grid * 256], 4-byte aligned, not overlapping
 *   src).  Time it over a buffer larger than the last-level cache.
 * bi_probe_lds: `grid` workgroups of 8 wavefronts; each fills a 64 KB LDS
 *   buffer, then every wavefront issues iters * 16 ds_read_b128 over it
 *   (64 consecutive 16-byte slots per instruction: no bank conflict), i.e.
 *   iters * 16 KB per wavefront.  out: device uint64 [grid * 8 * 2], 8-byte
 *   aligned; per wavefront: shader-clock cycles of its loop (s_memtime) and a
 *   sink word.  8 * iters * 16 KB / (the workgroup's largest cycle count) is
 *   the LDS read rate of one compute unit in bytes per cycle.  iters in
 *   [1, 2^40], grid >= 1.
 */
bi_status bi_probe_mfma(void *out, int64_t iters, int grid, void *stream);
bi_status bi_probe_read(const void *src, int64_t bytes, void *sink, int grid, void *stream);
bi_status bi_probe_lds(void *out, int64_t iters, int grid, void *stream);

/* Static, human-readable name of a status code. */
const char *bi_status_str(bi_status s);

/* Library version string (static). */
const char *bi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
