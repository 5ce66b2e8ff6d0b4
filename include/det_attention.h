/*
 * det_attention -- batch-invariant decode attention with a fixed split-KV
 * size, for gfx950 (MI355X).
 *
 * Source: the summary page of "Defeating Nondeterminism in LLM Inference",
 * section on batch-invariant kernel design, attention: a split-KV
 * (FlashDecoding) reduction keeps batch invariance only with a fixed split
 * size, so that the order of the reduction never depends on the batch or on
 * how a sequence is cut; the cached keys and values keep one layout.
 *
 * What is computed, for sequence b with len[b] cached positions and query
 * head h (key/value head h / G, G = Hq / Hkv):
 *   o[b, h] = softmax(scale * K[b, h/G, :len] q[b, h]) V[b, h/G, :len]
 * as follows (fp32 throughout, bf16 output):
 *   splits     the positions are cut into splits of DET_ATTN_SPLIT = 256
 *              from position 0, whatever the batch, the lengths of the other
 *              sequences or Smax;
 *   per split  scores s_j = (sum over d of q_d k_jd) * scale * log2(e), the
 *              dot product in sixteen 8-wide parts c = 0..15, each a chain
 *              of 4 bf16-pair dot instructions in ascending d, the parts
 *              joined in a balanced tree that pairs c with c + 8, then with
 *              c + 4, c + 2, c + 1; m = max s_j;
 *              p_j = 2^(s_j - m); l = pairwise sum of p_j over the split's
 *              256 slots (empty slots 0); acc_d = sum of p_j v_jd in
 *              ascending j;
 *   combine    M = max of the splits' m; L and o_d are the sums over splits
 *              in ascending order of l and acc_d times 2^(m - M);
 *              o_d = bf16(o_d / L).  len 0 gives o = 0.
 * The bits of o[b, h] therefore depend only on q[b, h], the first len[b]
 * keys and values of its head and len[b].
 *
 * Layouts (row-major, DEVICE pointers): Q [B, Hq, D], K and V [B, Hkv, Smax,
 * D], lens [B] int32 (values outside [0, Smax] are clamped into it), O [B,
 * Hq, D] bf16, work: a caller-owned fp32 buffer of
 * B * Hq * ceil(Smax / 256) * (D + 2) floats (the per-split partial results;
 * the library allocates nothing).  D must be 128; G = Hq / Hkv must divide
 * evenly and be at most 8.  Asynchronous on `stream`.  Returns DET_GEMM_OK,
 * DET_GEMM_EINVAL (negative or unsupported sizes, null pointer, overlapping
 * output) or DET_GEMM_EHIP; nothing is launched on error.  B == 0 is a no-op.
 */
#ifndef DET_ATTENTION_H
#define DET_ATTENTION_H

#include <stdint.h>

#include "det_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define DET_ATTN_SPLIT 256
#define DET_ATTN_HEAD_DIM 128
#define DET_ATTN_MAX_GROUP 8

/* Decode attention with fixed 256-position splits (section on batch-invariant
 * kernel design, attention). */
int det_attention_decode(const det_bf16 *Q, const det_bf16 *K, const det_bf16 *V,
                         const int32_t *lens, int64_t B, int64_t Hq, int64_t Hkv, int64_t Smax,
                         int64_t D, float scale, float *work, det_bf16 *O, void *stream);

/* Chunked prefill with the decode arithmetic (same section: a query's result
 * must not depend on how the sequence is cut into chunks, nor on whether its
 * keys came from the cache or from the current chunk).  Query rows Q [NQ, Hq,
 * D] (bf16, contiguous) are grouped by sequence: the rows of sequence b are
 * row_offsets[b] .. row_offsets[b+1] - 1 (row_offsets: a HOST array of B + 1
 * entries, 0 first and NQ last, nondecreasing).  Row r attends the first
 * lens[r] positions of its sequence's K and V [B, Hkv, Smax, D] (lens: DEVICE
 * int32 [NQ], clamped into [0, Smax]); a causal chunk at positions p0 .. p0 +
 * C - 1 is the rows with lens p0 + 1 .. p0 + C.  Every (row, head) is
 * computed exactly as det_attention_decode computes a query of that length
 * (same splits, same orders), so O [NQ, Hq, D] holds, bit for bit, what a
 * decode call would return for each row -- whatever the chunk sizes, the
 * other rows or their order.  work: a caller-owned fp32 buffer of
 * NQ * Hq * ceil(Smax / 256) * (D + 2) floats.  Rows of one sequence are
 * processed 8 / G at a time, so each split of keys and values is read once
 * per such tile.  B <= 128, NQ <= 65535; other conditions and errors as
 * det_attention_decode.  NQ == 0 is a no-op. */
int det_attention_prefill(const det_bf16 *Q, const det_bf16 *K, const det_bf16 *V,
                          const int64_t *row_offsets, const int32_t *lens, int64_t NQ, int64_t B,
                          int64_t Hq, int64_t Hkv, int64_t Smax, int64_t D, float scale,
                          float *work, det_bf16 *O, void *stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation and the same kernels as det_attention_decode, bit for bit, with
 * the per-split partials in a fixed device array of DET_ATTN_SCRATCH_FLOATS
 * floats (32 MiB) that the library holds on every device it runs on until the
 * process ends, instead of a work buffer.  The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.  The caller still
 * passes Q, K, V, lens and O as above.
 *   - A problem whose partials need more than the array,
 *     B * Hq * ceil(Smax / 256) * (D + 2) > DET_ATTN_SCRATCH_FLOATS, is
 *     refused with DET_ATTN_ESCRATCH before anything is launched (the
 *     64-sequence, 32-head, Smax = 4096 decode batch needs 4.3 M floats).
 *   - Every call on one device shares that device's array: calls that may
 *     run at the same time on one device (other streams, other threads)
 *     race and must be serialised by the caller.  Nothing in the array has
 *     to start at zero: each call writes every partial it reads.
 *   - Other errors as det_attention_decode. */
#define DET_ATTN_SCRATCH_FLOATS (INT64_C(8) << 20)
#define DET_ATTN_ESCRATCH (-4)
int det_attention_decode_noalloc(const det_bf16 *Q, const det_bf16 *K, const det_bf16 *V,
                                 const int32_t *lens, int64_t B, int64_t Hq, int64_t Hkv,
                                 int64_t Smax, int64_t D, float scale, det_bf16 *O,
                                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DET_ATTENTION_H */
