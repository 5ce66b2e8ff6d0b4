/*
 * det_norm -- batch-invariant RMSNorm for gfx950 (MI355X).
 *
 * Source: the summary page of "Defeating Nondeterminism in LLM Inference",
 * section on batch-invariant kernel design, RMSNorm: a data-parallel
 * strategy in which each row of the batch is reduced by one core, with the
 * same strategy whatever the batch size; splitting a row's reduction across
 * cores when the batch is small would give up batch invariance, so it is
 * never done here.
 *
 * What is computed for each row x[0..H) (bf16), weight w[0..H) (bf16), eps:
 *   squares        x_i^2 in fp32;
 *   ss             the mid-split tree of fp32 adds over the H squares (a
 *                  range of n splits into floor(n/2) on the left and the rest
 *                  on the right), an order that depends on H alone;
 *   rstd           1 / sqrt(ss / H + eps), each operation rounded once (fp32);
 *   y_i            bf16 (nearest even) of (x_i * rstd) * w_i in fp32.
 * One workgroup owns one row, so a row's bits never depend on R, on the other
 * rows or on how the batch is split into calls.
 *
 * Conventions (as det_gemm.h): det_bf16 bit patterns; DEVICE pointers;
 * row-major x [R,H] (ldx) and y [R,H] (ldy) in elements; rstd [R] fp32 (may
 * be NULL); asynchronous on `stream`; the library allocates nothing; y and
 * rstd must not overlap the inputs.  Returns DET_GEMM_OK, or
 * DET_GEMM_EINVAL (negative R, H < 1 or H > DET_NORM_MAX_H, null pointer,
 * leading dimension below H, overlap) or DET_GEMM_EHIP; on error nothing is
 * launched and nothing is written.  R == 0 is a successful no-op.
 */
#ifndef DET_NORM_H
#define DET_NORM_H

#include <stdint.h>

#include "det_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define DET_NORM_MAX_H 1048576

/* y = RMSNorm(x) * w per row, and rstd per row (section on batch-invariant
 * kernel design, RMSNorm). */
int det_rmsnorm(const det_bf16 *x, int64_t ldx, const det_bf16 *w, float eps, det_bf16 *y,
                int64_t ldy, float *rstd, int64_t R, int64_t H, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DET_NORM_H */
