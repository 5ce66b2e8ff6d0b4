/*
 * det_gemm -- batch-invariant deterministic bf16 GEMM for gfx950 (MI355X).
 *
 * Contract (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
 * (det_gemm)"; sections "Guarantees" and "Ascend NPU backend"):
 *   - bf16 inputs, fp32 accumulation, no split-K, fixed reduction order;
 *   - the reduction (length R) is cut into L = ceil(R/32) leaves of 32
 *     consecutive indices; each leaf's products are summed in fp32 and the sum
 *     is rounded once to bf16 (round to nearest, ties to even);
 *   - the leaves are merged by the mid-split tree of bf16 adds: a range of n
 *     leaves splits into floor(n/2) on the left and the rest on the right, and
 *     the two subtree roots are added in fp32 and rounded to bf16;
 *   - R is capped at 32768.
 * Hence an output row's bits depend only on that row of the left operand and on
 * the right operand: never on M, on padding rows, on leading dimensions or on
 * how the rows are split across calls; and when L is even, a GEMM over the first
 * (last) half of the reduction is exactly the left (right) child of the root.
 *
 * Conventions for every entry point below:
 *   - det_bf16 is the bf16 bit pattern (uint16_t).  All pointers are DEVICE
 *     pointers; all matrices are row-major with an explicit leading dimension
 *     in elements (row width <= ld <= 2^23 = DET_GEMM_MAX_LD, any alignment of
 *     the element type; the upper limit keeps the byte offsets inside one
 *     operand tile below 2^31).
 *   - The caller owns every buffer; the library allocates no device memory.
 *   - The call is asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream).  Outputs must not overlap inputs.
 *   - Return value: DET_GEMM_OK, or a negative status.  On any error the call
 *     launches nothing and writes nothing.
 *       DET_GEMM_EINVAL  null pointer with a non-empty shape, negative size,
 *                        leading dimension smaller than the row width or
 *                        larger than DET_GEMM_MAX_LD, a dimension or tile
 *                        count beyond 2^31 - 1, or an output range
 *                        overlapping an input range;
 *       DET_GEMM_EKCAP   reduction length R == 0 or R > 32768 (with a
 *                        non-empty output);
 *       DET_GEMM_EHIP    the HIP runtime reported an error (launch failure or
 *                        no gfx950 device).
 *     An empty output (M == 0 or N == 0; K == 0 for da/db outputs) is a
 *     successful no-op.  Unsupported inputs are rejected, never routed to a
 *     different arithmetic.
 *   - The reduction-internal order of a leaf is whatever the gfx950 bf16 MFMA
 *     does (fixed, shape-independent); the CPU definition adds the 32 products
 *     left to right.  The det_gemm_strict_* entry points add them left to right
 *     as well and are bit-exact to that definition (for products within fp32's
 *     normal range; see below).
 */
#ifndef DET_GEMM_H
#define DET_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t det_bf16;

#define DET_GEMM_OK 0
#define DET_GEMM_EINVAL (-1)
#define DET_GEMM_EKCAP (-2)
#define DET_GEMM_EHIP (-3)

#define DET_GEMM_LEAF 32
#define DET_GEMM_MAX_REDUCTION 32768
#define DET_GEMM_MAX_LD (INT64_C(1) << 23)

/* Forward (page section "Guarantees": C = A @ B).
 * A [M,K] (lda), B [K,N] (ldb), C [M,N] (ldc); reduction over K. */
int det_gemm_fwd(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                 det_bf16 *C, int64_t ldc, int64_t M, int64_t N, int64_t K, void *stream);

/* Forward with the weight given transposed, as nn.Linear stores it (page
 * section "Ascend NPU backend", entry point fwd_rhs_transposed):
 * C [M,N] = A [M,K] @ Bt [N,K]^T. */
int det_gemm_fwd_rhs_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *Bt,
                                int64_t ldbt, det_bf16 *C, int64_t ldc, int64_t M, int64_t N,
                                int64_t K, void *stream);

/* Forward with fp32 output (page section "Ascend NPU backend", Dtypes: the
 * fp32 forward returns FP32).  Same leaves and tree as det_gemm_fwd; the bf16
 * root is widened exactly to fp32, so the result equals det_gemm_fwd widened.
 * C is float [M,N] (ldc in floats). */
int det_gemm_fwd_fp32(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                      float *C, int64_t ldc, int64_t M, int64_t N, int64_t K, void *stream);

/* Input gradient (page section "Guarantees": dA = dC * B^T):
 * dA [M,K] = dC [M,N] @ B [K,N]^T; reduction over N (cap applies to N). */
int det_gemm_da(const det_bf16 *dC, int64_t lddc, const det_bf16 *B, int64_t ldb,
                det_bf16 *dA, int64_t ldda, int64_t M, int64_t N, int64_t K, void *stream);

/* Weight gradient (page section "Guarantees": dB = A^T * dC):
 * dB [K,N] = A [M,K]^T @ dC [M,N]; reduction over M (cap applies to M). */
int det_gemm_db(const det_bf16 *A, int64_t lda, const det_bf16 *dC, int64_t lddc,
                det_bf16 *dB, int64_t lddb, int64_t M, int64_t N, int64_t K, void *stream);

/* Weight gradient written directly in the [N,K] layout that an nn.Linear
 * weight uses (page section "Ascend NPU backend", entry point
 * db_transposed): dBt [N,K] with dBt[n][k] == dB[k][n] bit for bit. */
int det_gemm_db_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *dC, int64_t lddc,
                           det_bf16 *dBt, int64_t lddbt, int64_t M, int64_t N, int64_t K,
                           void *stream);

/* Strict-order variants of the six operations: the same contract with every
 * leaf summed by a scalar fp32 fused multiply-add chain in ascending index
 * order.  A product of two bf16 values has at most 16 significant bits, so it
 * is exact in fp32 unless it falls below 2^-126 (subnormal range) or above the
 * fp32 range; for such inputs the fused chain equals the left-to-right sum of
 * rounded products of the page's leaf definition, and the result is bit-exact
 * to the CPU definition.  Products that underflow or overflow fp32 are outside
 * this promise (the fused add rounds once where the definition rounds the
 * product first).  Slow by design.  Same arguments, ownership and errors as
 * the entry points above. */
int det_gemm_strict_fwd(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                        det_bf16 *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                        void *stream);
int det_gemm_strict_fwd_rhs_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *Bt,
                                       int64_t ldbt, det_bf16 *C, int64_t ldc, int64_t M,
                                       int64_t N, int64_t K, void *stream);
int det_gemm_strict_fwd_fp32(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                             float *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             void *stream);
int det_gemm_strict_da(const det_bf16 *dC, int64_t lddc, const det_bf16 *B, int64_t ldb,
                       det_bf16 *dA, int64_t ldda, int64_t M, int64_t N, int64_t K,
                       void *stream);
int det_gemm_strict_db(const det_bf16 *A, int64_t lda, const det_bf16 *dC, int64_t lddc,
                       det_bf16 *dB, int64_t lddb, int64_t M, int64_t N, int64_t K,
                       void *stream);
int det_gemm_strict_db_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *dC,
                                  int64_t lddc, det_bf16 *dBt, int64_t lddbt, int64_t M,
                                  int64_t N, int64_t K, void *stream);

/* Combination of K-shard partial products (page section "Ascend NPU backend",
 * bullet "Reduction tree": a contiguous half of the reduction is one child of
 * the tree, which is what makes TP = 2 equal TP = 1).  parts is a HOST array
 * of nparts device pointers, each an [M,N] bf16 matrix with leading dimension
 * ldp, in rank (reduction) order; out [M,N] (ldo) receives, element by
 * element, the mid-split tree of bf16 adds over the nparts values (a range of
 * n parts splits into floor(n/2) on the left; each add is the fp32 sum
 * rounded to bf16).  When the parts are det_gemm products over TP = 2^j
 * contiguous equal shards of a reduction whose leaf count L is a multiple of
 * TP, each part is a subtree of the full product's tree and out equals the
 * unsharded product bit for bit: this is the local step of a deterministic
 * reduce-scatter across GPUs.  1 <= nparts <= DET_GEMM_MAX_PARTS; out must
 * not overlap a part.  Same errors as above. */
#define DET_GEMM_MAX_PARTS 16
int det_gemm_shard_reduce(const det_bf16 *const *parts, int64_t nparts, int64_t ldp,
                          det_bf16 *out, int64_t ldo, int64_t M, int64_t N, void *stream);

/* Inspection: the bf16 leaves of the MFMA forward kernel (same leaf code as
 * det_gemm_fwd), for checking that the only difference from the CPU definition
 * is the order of additions inside a leaf.  leaves is [M][N][L] bf16,
 * L = ceil(K/32), fully packed (no leading dimension).  Same errors as
 * det_gemm_fwd. */
int det_gemm_debug_leaves(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                          det_bf16 *leaves, int64_t M, int64_t N, int64_t K, void *stream);

/* Inspection: element-wise device primitives exactly as the kernels use them.
 *   det_gemm_debug_round:  out[i] = bf16 rounding of x[i] (fp32), as the MFMA
 *                          kernel rounds leaves and tree nodes;
 *   det_gemm_debug_add:    out[i] = bf16 add of a[i] and b[i], as the MFMA
 *                          kernel merges two tree nodes.
 * Device pointers, n elements; asynchronous on stream. */
int det_gemm_debug_round(const float *x, det_bf16 *out, int64_t n, void *stream);
int det_gemm_debug_add(const det_bf16 *a, const det_bf16 *b, det_bf16 *out, int64_t n,
                       void *stream);

/* Inspection: the tree add exactly as the matrix-core kernels perform it
 * (page section "Ascend NPU backend", bullet "Reduction tree": nodes are
 * merged by bf16 adds).  Element-wise out[i] = a[i] (+) b[i], computed in
 * blocks of 256 pairs by one bf16 MFMA against a constant 0/1 selector matrix
 * whose products are exact, then rounded to bf16; a block with a non-finite
 * sum is redone with element-wise fp32 adds, as the kernels redo a tile whose
 * root is non-finite.  selector 0: the split selector of the wide and
 * direct-to-LDS kernels (the large-product path); selector 1: the pairwise
 * selector of the general kernel.  The decode kernel's VALU add is
 * det_gemm_debug_add.  Device pointers, n elements; asynchronous on stream;
 * DET_GEMM_EINVAL for n < 0, a null pointer or another selector. */
int det_gemm_debug_matrix_add(const det_bf16 *a, const det_bf16 *b, det_bf16 *out, int64_t n,
                              int selector, void *stream);

/* Issue-rate probe (inspection; no page defines it -- it measures the chip the
 * kernels run on).  Runs `workgroups` workgroups of 512 threads (two waves
 * per SIMD) on `stream`; each wave loops `iters` times over the instruction
 * mix of one pipeline stage of the 128x128 wide kernel without memory
 * traffic: 32 v_mfma_f32_16x16x32_bf16 and 64 v_cvt_pk_bf16_f32 per wave and
 * iteration, each conversion rounding an MFMA result that the next MFMA
 * consumes (mode 1), or the MFMAs alone (mode 0).  The caller times the
 * launch (e.g. with events on `stream`).  sink: device float[workgroups *
 * 512], written with meaningless values.  EINVAL: mode outside 0..1,
 * iters < 1, workgroups < 1, or sink null. */
int det_gemm_debug_issue_probe(int mode, int iters, int workgroups, float *sink, void *stream);

/* Inspection: pins the MFMA kernel's tile configuration (0 .. count-1) for
 * subsequent calls on this process, or restores automatic selection (-1).
 * Every configuration computes the same leaves and tree, so the results must
 * not change; tests use this to show it.  A call whose problem the pinned
 * configuration does not take (its shape, alignment, leaf count or row count)
 * returns DET_GEMM_EINVAL without launching.  Returns the number of
 * configurations, or DET_GEMM_EINVAL for an out-of-range value. */
int det_gemm_debug_force_config(int config);

/* Inspection: the tile configuration (0 .. count-1, the numbering of
 * det_gemm_debug_force_config) that the MFMA entry point of operation `op`
 * would run for these arguments, chosen from shape, alignment and leaf count
 * alone.  The arguments are those of that entry point, in its order (for
 * det_gemm_fwd: A, lda, B, ldb, C, ldc, M, N, K); the pointers are only
 * compared and tested for alignment, never dereferenced, and no device is
 * needed.  op: DET_GEMM_OP_FWD, _FWD_RHS_TRANSPOSED, _FWD_FP32, _DA, _DB or
 * _DB_TRANSPOSED.  Returns the configuration, the pinned one if
 * det_gemm_debug_force_config holds one, or the status the entry point would
 * return before launching: DET_GEMM_EINVAL (also for an empty product, which
 * launches nothing, and for an unknown op) or DET_GEMM_EKCAP. */
#define DET_GEMM_OP_FWD 0
#define DET_GEMM_OP_FWD_RHS_TRANSPOSED 1
#define DET_GEMM_OP_FWD_FP32 2
#define DET_GEMM_OP_DA 3
#define DET_GEMM_OP_DB 4
#define DET_GEMM_OP_DB_TRANSPOSED 5
int det_gemm_debug_config(int op, const void *P, int64_t ldp, const void *Q, int64_t ldq,
                          const void *Out, int64_t ldo, int64_t M, int64_t N, int64_t K);

/* Human-readable text for a status code (static storage). */
const char *det_gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DET_GEMM_H */
