/*
 * det_moe -- MoE grouped GEMM with a deterministic per-token reduction
 * epilogue, for gfx950 (MI355X).
 *
 * Source: reading notes "Bitwise-Deterministic Pretraining at Scale: How
 * Megatron Core Finds and Removes Every Flipped Bit", section "Kernel
 * redesign: the grouped-GEMM epilogue".  In the epilogue of the MoE grouped
 * GEMM several N-tiles of the output contribute to one per-token value
 * (dprob[token]); adding them atomically makes the sum depend on the order in
 * which tiles finish.  Here every N-tile writes a private slot, and once all
 * tiles are done the slots of a token are combined by a fixed tree.
 *
 * What one call computes, for rows grouped by expert (expert e owns rows
 * offsets[e] .. offsets[e+1]-1 of X, G, Y, slots and dprob):
 *   Y[r, :]     = det_gemm_fwd(X[r, :], W_e)            (det_gemm.h: the
 *                 same leaves and tree, hence the same bits as a det_gemm_fwd
 *                 call on that expert's rows, or on any subset of them);
 *   p(r, n)     = fp32 product of Y[r, n] and G[r, n]   (exact in fp32);
 *   slots[j*slot_ld + r], j < J = ceil(N/128):
 *                 the mid-split tree of fp32 adds over the 128 column
 *                 positions 128j .. 128j+127 (positions >= N hold +0);
 *   dprob[r]    = the mid-split tree of fp32 adds over the J slots of row r
 *                 (left child floor(n/2), as the leaves of det_gemm);
 *                 +0 when N == 0.
 * Every add rounds to nearest even.  A row's Y, slots and dprob depend only on
 * that row of X and G and on its expert's weight: never on the other experts,
 * on how many rows each expert has, or on the tile that computes it.
 *
 * Conventions (as det_gemm.h):
 *   - det_bf16 is the bf16 bit pattern; X, W, G, Y, slots, dprob are DEVICE
 *     pointers, row-major with leading dimensions in elements; `offsets` is a
 *     HOST array of E + 1 int64 (offsets[0] = 0, nondecreasing,
 *     offsets[E] = T).
 *   - W_e = W + e * w_stride is a [K,N] matrix with leading dimension ldw.
 *   - slots is a caller-owned fp32 buffer of J rows of slot_ld >= T floats;
 *     the call overwrites the first T entries of each row.  The library
 *     allocates no device memory.
 *   - Asynchronous on `stream`.  Y, slots and dprob must not overlap each
 *     other or any input.
 *   - Returns DET_GEMM_OK or a negative status; on error nothing is launched
 *     and nothing is written:
 *       DET_GEMM_EINVAL  null pointer with a non-empty shape, negative size,
 *                        E < 1 or E > DET_MOE_MAX_EXPERTS, offsets not as
 *                        above, a leading dimension smaller than its row
 *                        width, slot_ld < T, or overlapping outputs;
 *       DET_GEMM_EKCAP   K == 0 or K > 32768 (with T > 0);
 *       DET_GEMM_EHIP    a HIP runtime error or no gfx950 device.
 *     T == 0 is a successful no-op.
 */
#ifndef DET_MOE_H
#define DET_MOE_H

#include <stdint.h>

#include "det_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define DET_MOE_SLOT 128
#define DET_MOE_MAX_EXPERTS 128

/* The grouped GEMM and its per-token epilogue (section "Kernel redesign: the
 * grouped-GEMM epilogue").  X [T,K] (ldx), W [E][K,N], G [T,N] (ldg),
 * Y [T,N] (ldy), slots [ceil(N/128)][slot_ld], dprob [T]. */
int det_moe_fwd_dprob(const det_bf16 *X, int64_t ldx, const det_bf16 *W, int64_t ldw,
                      int64_t w_stride, const int64_t *offsets, int64_t E, const det_bf16 *G,
                      int64_t ldg, det_bf16 *Y, int64_t ldy, float *slots, int64_t slot_ld,
                      float *dprob, int64_t T, int64_t N, int64_t K, void *stream);

/* Test-only: the slot writer as a kernel of its own over given Y and G
 * (slots[j*slot_ld + r] as above), the form used when the grouped GEMM does
 * not write the slots itself.  Same errors. */
int det_moe_debug_slots(const det_bf16 *Y, int64_t ldy, const det_bf16 *G, int64_t ldg,
                        float *slots, int64_t slot_ld, int64_t T, int64_t N, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DET_MOE_H */
