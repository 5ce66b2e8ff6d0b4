/*
 * det_fingerprint -- on-GPU tensor fingerprints and a first-mismatch
 * comparator for gfx950 (MI355X), the localiser of a determinism harness.
 *
 * Source: reading notes "Bitwise-Deterministic Pretraining at Scale: How
 * Megatron Core Finds and Removes Every Flipped Bit", section "5.
 * Fingerprinting Tensors on the GPU": digests are computed in GPU memory from
 * the bit patterns and recorded with shape, dtype and element count; a hash
 * that ignores positions cannot see a permutation, so order-sensitive data is
 * hashed per row or chunk; a byte-level comparison settles a suspected
 * difference.  Section "Reading the first mismatch": the origin of a
 * divergence is the first event whose input digests agree and whose output
 * digests differ.
 *
 * The digest of a byte string of n bytes (the pages name no hash; this one is
 * fixed here):
 *   w_i      little-endian 64-bit words of the bytes, i < ceil(n/8), bytes
 *            past n read as 0;
 *   mix(z)   SplitMix64's finalizer: z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *            z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31 (mod 2^64);
 *   S        sum over i of mix(w_i + 0x9E3779B97F4A7C15 * (i + 1)), mod 2^64;
 *   digest   mix(S + n).
 * Every term carries its position, so moving data changes the digest; terms
 * are combined by addition mod 2^64, which is associative, so the parallel
 * evaluation's grouping never changes a bit.  A row digest is the digest of
 * the row's bytes alone.
 *
 * Conventions: DEVICE pointers; `data`, `a`, `b` of any alignment (16-byte
 * aligned data takes the vector path); outputs are caller-owned device
 * buffers; asynchronous on `stream`; status codes of det_gemm.h:
 *   DET_GEMM_EINVAL  negative size, null pointer with a non-empty size,
 *                    ld_bytes < row_bytes, or an output overlapping an input;
 *   DET_GEMM_EHIP    a HIP runtime error or no gfx950 device.
 * On error nothing is launched and nothing is written.  The library
 * allocates no device memory.
 */
#ifndef DET_FINGERPRINT_H
#define DET_FINGERPRINT_H

#include <stdint.h>

#include "det_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Digest of nbytes bytes at `data` (section "5. Fingerprinting Tensors on the
 * GPU", bit-pattern digest); written to digest[0] (device). */
int det_fingerprint(const void *data, int64_t nbytes, uint64_t *digest, void *stream);

/* Per-row digests of a 2-D byte layout: row r is the row_bytes bytes at
 * data + r * ld_bytes (same section: order-sensitive data hashed along a
 * dimension, row-wise or chunk-wise); written to digests[r] (device). */
int det_fingerprint_rows(const void *data, int64_t rows, int64_t row_bytes, int64_t ld_bytes,
                         uint64_t *digests, void *stream);

/* Smallest byte index k < nbytes with a[k] != b[k], or -1 (same section: the
 * byte-level comparison that settles a suspected difference); written to
 * index[0] (device). */
int det_first_mismatch(const void *a, const void *b, int64_t nbytes, int64_t *index,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DET_FINGERPRINT_H */
