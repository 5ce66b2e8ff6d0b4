/*
 * CPU oracle for the batch-invariant deterministic GEMM (det_gemm).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header or
 * table with the HIP library.
 *
 * What it computes (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
 * (det_gemm)"):
 *   - section "Guarantees": forward C = A @ B, backward dA = dC * B^T and
 *     dB = A^T * dC; bf16 inputs with fp32 accumulation; no split-K; a fixed
 *     K-loop order.
 *   - section "Ascend NPU backend", bullet "Reduction tree": the reduction is cut
 *     into 32-element leaves; each leaf is accumulated in fp32 in ascending order
 *     and rounded once to bf16 with round-to-nearest-even; the leaves are then
 *     merged by the mid-split tree of bf16 additions in ascending leaf order, so
 *     that a contiguous half-K product is one child of the tree.
 *   - same section, "Dtypes" paragraph: bf16 out (the fp32-output entry point
 *     returns fp32); the reduction length is capped at 32768.
 *   - same section, first bullet: the six entry points and their operand roles;
 *     db_transposed stores the weight gradient in [N,K].
 *
 * Readings where the page is silent (each one is also listed in the design
 * notes of this repository):
 *   - mid-split of an odd range: the left child takes floor(n/2) leaves;
 *   - a leaf starts from +0.0f and accumulates products in ascending reduction
 *     index, one multiply-accumulate per step (the exact product added, the
 *     sum rounded once: the fused chain of the strict kernel, and the MAC
 *     order the Ascend section describes); a product of two bf16 values is
 *     exact in fp32 unless it underflows, so this equals rounding each product
 *     and adding for every product in fp32's normal range;
 *   - a "bf16 add" is the fp32 sum of the two bf16 values rounded once to bf16
 *     (this equals the correctly rounded bf16 sum);
 *   - a partial last leaf (R % 32 != 0) holds only the remaining products;
 *   - the fp32-output entry point returns the same bf16 root widened to fp32;
 *   - R == 0 or R > 32768 is rejected; an empty output (I == 0 or J == 0) is a
 *     successful no-op.
 *
 * Build: plain C99, -O2 -fno-fast-math -ffp-contract=off -mfma, OpenMP over output
 * rows only (each output element is computed start to finish by one thread, in
 * the order above, so the thread count never changes a bit).
 *
 * bf16 values travel as their uint16_t bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_EKCAP (-2)
#define ORACLE_ENOMEM (-4)

#define ORACLE_LEAF 32
#define ORACLE_MAX_R 32768

/* bf16 bit pattern -> fp32 value (exact: bf16 is the top half of an fp32). */
static float widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even (page: leaves "round once to
 * BF16 (round-to-nearest-even)").  Written from the definition: keep the top 16
 * bits (this truncates the magnitude), then step the magnitude up by one bf16
 * ulp when the dropped 16 bits are more than half an ulp, or exactly half and
 * the kept value is odd.  A step up from the largest finite bf16 carries into
 * the exponent and gives infinity, as rounding requires.  NaN maps to the quiet
 * NaN with the same sign. */
static uint16_t round_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* The bf16 add of the tree: both operands are exact in fp32, their fp32 sum is
 * rounded once to bf16. */
static uint16_t add_bf16(uint16_t a, uint16_t b) {
    float s = widen(a) + widen(b);
    return round_bf16(s);
}

/* One leaf: the products x[r]*y[r] for r in [r0, r1), accumulated one by one
 * in ascending r into an fp32 sum that starts at +0 (each step a multiply-
 * accumulate: the exact product is added and the sum rounded once, fmaf),
 * then rounded once to bf16.  A product of two bf16 values has at most 16
 * significant bits, so for products in fp32's normal range this is the same
 * as rounding each product to fp32 and adding; the two differ only for
 * products below 2^-126. */
static uint16_t leaf(const uint16_t *x, int64_t sx, const uint16_t *y, int64_t sy,
                     int64_t r0, int64_t r1) {
    float s = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
        s = fmaf(widen(x[r * sx]), widen(y[r * sy]), s);
    return round_bf16(s);
}

/* Mid-split tree over leaves [lo, hi): a single leaf is itself; otherwise the
 * range splits at mid = lo + floor((hi - lo) / 2), both halves are reduced the
 * same way and their roots are joined by one bf16 add.  Also records the
 * largest magnitude of any node (leaf or inner) in *big. */
static uint16_t tree(const uint16_t *leaves, int64_t lo, int64_t hi, float *big) {
    uint16_t v;
    if (hi - lo == 1) {
        v = leaves[lo];
    } else {
        int64_t mid = lo + (hi - lo) / 2;
        uint16_t left = tree(leaves, lo, mid, big);
        uint16_t right = tree(leaves, mid, hi, big);
        v = add_bf16(left, right);
    }
    float m = fabsf(widen(v));
    if (!(m <= *big)) /* also takes NaN */
        *big = m;
    return v;
}

/*
 * The whole contraction, for any operand layout.
 *   output element (i, j), i < I, j < J, reduction index r < R;
 *   x(i, r) = X[i*sxi + r*sxr],  y(j, r) = Y[j*syj + r*syr];
 *   result written to C at element offset i*sci + j*scj, as bf16 (out_f32 == 0)
 *   or as the bf16 root widened to fp32 (out_f32 == 1).
 * Optional outputs (NULL to skip), indexed by i*J + j:
 *   leaves_out[(i*J + j)*L + l]  the bf16 leaves of element (i, j);
 *   big_out[i*J + j]             the largest node magnitude of its tree.
 */
static int contract(const uint16_t *X, int64_t sxi, int64_t sxr,
                    const uint16_t *Y, int64_t syj, int64_t syr,
                    void *C, int64_t sci, int64_t scj, int out_f32,
                    int64_t I, int64_t J, int64_t R,
                    uint16_t *leaves_out, float *big_out) {
    if (I < 0 || J < 0 || R < 0)
        return ORACLE_EINVAL;
    if (I == 0 || J == 0)
        return ORACLE_OK;
    if (R == 0 || R > ORACLE_MAX_R)
        return ORACLE_EKCAP;
    if (!X || !Y || !C)
        return ORACLE_EINVAL;
    const int64_t L = (R + ORACLE_LEAF - 1) / ORACLE_LEAF;
    int failed = 0;

#pragma omp parallel
    {
        uint16_t *lv = (uint16_t *)malloc((size_t)L * sizeof(uint16_t));
        if (!lv) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < I; ++i) {
            if (!lv)
                continue;
            for (int64_t j = 0; j < J; ++j) {
                const uint16_t *x = X + i * sxi;
                const uint16_t *y = Y + j * syj;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t r0 = l * ORACLE_LEAF;
                    int64_t r1 = r0 + ORACLE_LEAF < R ? r0 + ORACLE_LEAF : R;
                    lv[l] = leaf(x, sxr, y, syr, r0, r1);
                }
                float big = 0.0f;
                uint16_t root = tree(lv, 0, L, &big);
                int64_t off = i * sci + j * scj;
                if (out_f32)
                    ((float *)C)[off] = widen(root);
                else
                    ((uint16_t *)C)[off] = root;
                if (leaves_out)
                    memcpy(leaves_out + (i * J + j) * L, lv, (size_t)L * sizeof(uint16_t));
                if (big_out)
                    big_out[i * J + j] = big;
            }
        }
        free(lv);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ---- the six operations (page section "Ascend NPU backend", first bullet) ----
 * All matrices are row-major with the given leading dimension (elements). */

/* C[M,N] = A[M,K] @ B[K,N]; reduction over K. */
int oracle_det_gemm_fwd(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                        uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K) {
    return contract(A, lda, 1, B, 1, ldb, C, ldc, 1, 0, M, N, K, NULL, NULL);
}

/* C[M,N] = A[M,K] @ Bt[N,K]^T; the weight is given as [N,K]. */
int oracle_det_gemm_fwd_rhs_transposed(const uint16_t *A, int64_t lda, const uint16_t *Bt,
                                       int64_t ldbt, uint16_t *C, int64_t ldc, int64_t M,
                                       int64_t N, int64_t K) {
    return contract(A, lda, 1, Bt, ldbt, 1, C, ldc, 1, 0, M, N, K, NULL, NULL);
}

/* As det_gemm_fwd, with the bf16 root written as fp32. */
int oracle_det_gemm_fwd_fp32(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                             float *C, int64_t ldc, int64_t M, int64_t N, int64_t K) {
    return contract(A, lda, 1, B, 1, ldb, C, ldc, 1, 1, M, N, K, NULL, NULL);
}

/* dA[M,K] = dC[M,N] @ B[K,N]^T; reduction over N. */
int oracle_det_gemm_da(const uint16_t *dC, int64_t lddc, const uint16_t *B, int64_t ldb,
                       uint16_t *dA, int64_t ldda, int64_t M, int64_t N, int64_t K) {
    return contract(dC, lddc, 1, B, ldb, 1, dA, ldda, 1, 0, M, K, N, NULL, NULL);
}

/* dB[K,N] = A[M,K]^T @ dC[M,N]; reduction over M. */
int oracle_det_gemm_db(const uint16_t *A, int64_t lda, const uint16_t *dC, int64_t lddc,
                       uint16_t *dB, int64_t lddb, int64_t M, int64_t N, int64_t K) {
    return contract(A, 1, lda, dC, 1, lddc, dB, lddb, 1, 0, K, N, M, NULL, NULL);
}

/* dBt[N,K] = (A[M,K]^T @ dC[M,N])^T, stored directly in the [N,K] layout. */
int oracle_det_gemm_db_transposed(const uint16_t *A, int64_t lda, const uint16_t *dC,
                                  int64_t lddc, uint16_t *dBt, int64_t lddbt, int64_t M,
                                  int64_t N, int64_t K) {
    return contract(A, 1, lda, dC, 1, lddc, dBt, 1, lddbt, 0, K, N, M, NULL, NULL);
}

/* ---- inspection helpers for the tests ---- */

/* Forward product that also returns every element's leaves ([M][N][L]) and the
 * largest node magnitude of its tree ([M][N]); either may be NULL. */
int oracle_det_gemm_fwd_detail(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                               uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                               uint16_t *leaves, float *big) {
    return contract(A, lda, 1, B, 1, ldb, C, ldc, 1, 0, M, N, K, leaves, big);
}

/* Applies the mid-split tree to count given leaf sequences of length L each
 * (leaves[c*L + l]); writes each root to out[c] and its largest node magnitude
 * to big[c] (big may be NULL). */
int oracle_tree_from_leaves(const uint16_t *leaves, int64_t count, int64_t L, uint16_t *out,
                            float *big) {
    if (count < 0 || L < 1 || L * ORACLE_LEAF > ORACLE_MAX_R + ORACLE_LEAF - 1)
        return ORACLE_EINVAL;
    for (int64_t c = 0; c < count; ++c) {
        float b = 0.0f;
        out[c] = tree(leaves + c * L, 0, L, &b);
        if (big)
            big[c] = b;
    }
    return ORACLE_OK;
}

/* The two scalar primitives, element-wise, for exhaustive checks. */
void oracle_round_bf16_array(const float *x, uint16_t *out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = round_bf16(x[i]);
}

void oracle_add_bf16_array(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = add_bf16(a[i], b[i]);
}

/* Threads an OpenMP parallel region of this library uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ==== MoE grouped GEMM with a per-token reduction epilogue ====
 *
 * Reading notes "Bitwise-Deterministic Pretraining at Scale: How Megatron Core
 * Finds and Removes Every Flipped Bit", section "Kernel redesign: the
 * grouped-GEMM epilogue": a per-token value dprob[token] of the MoE grouped
 * GEMM's epilogue gathers contributions from several output column tiles.
 * Atomic accumulation would add them in whatever order the tiles finish; the
 * deterministic form keeps one private partial per column tile and reduces
 * those partials in a fixed tree after the last tile has written its own.
 *
 * What is computed here:
 *   - rows of X are grouped by expert: expert e owns rows [off[e], off[e+1]);
 *     Y[r, :] = det_gemm forward of X[r, :] with that expert's weight W_e [K,N]
 *     (the operation defined above, per segment);
 *   - dprob[r] is the reduction over n of p(r, n) = Y[r, n] * G[r, n]
 *     (G: the gradient of the expert output for that row);
 *   - slot j of row r holds the reduction of the products of columns
 *     [128 j, 128 j + 128); dprob[r] combines the slots of row r.
 *
 * Readings where the page is silent (each one is also listed in the design
 * notes of this repository):
 *   - the slot width is 128 columns (the output tile width of the kernels);
 *   - products are fp32 products of the two bf16 values (exact in fp32);
 *   - every add is an fp32 add, round to nearest even;
 *   - inside a slot the products are combined by the mid-split tree over the
 *     128 column positions of the slot, positions at or past N holding +0
 *     (for 128 positions the mid-split tree is the perfect pairwise tree);
 *   - the slots of a row are combined by the mid-split tree over the J slots
 *     (the same split rule as the leaves of det_gemm: left child floor(n/2));
 *   - N == 0 gives dprob = +0 and no slot.
 */
#define ORACLE_SLOT 128

/* Mid-split tree of fp32 adds over v[lo, hi) (hi > lo). */
static float tree_f32(const float *v, int64_t lo, int64_t hi) {
    if (hi - lo == 1)
        return v[lo];
    int64_t mid = lo + (hi - lo) / 2;
    float left = tree_f32(v, lo, mid);
    float right = tree_f32(v, mid, hi);
    return left + right;
}

/* slots[j*slot_ld + r] (J = ceil(N/128) slots per row) and dprob[r] for the
 * T rows of Y [T,N] and G [T,N].  slots may be NULL. */
int oracle_moe_dprob(const uint16_t *Y, int64_t ldy, const uint16_t *G, int64_t ldg,
                     int64_t T, int64_t N, float *slots, int64_t slot_ld, float *dprob) {
    if (T < 0 || N < 0 || (T > 0 && N > 0 && (ldy < N || ldg < N)) || (slots && slot_ld < T))
        return ORACLE_EINVAL;
    const int64_t J = (N + ORACLE_SLOT - 1) / ORACLE_SLOT;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < T; ++r) {
        float prod[ORACLE_SLOT];
        float *s = J > 0 ? malloc((size_t)J * sizeof *s) : NULL;
        if (J > 0 && !s) {
            failed = 1;
            continue;
        }
        for (int64_t j = 0; j < J; ++j) {
            for (int64_t c = 0; c < ORACLE_SLOT; ++c) {
                int64_t n = j * ORACLE_SLOT + c;
                prod[c] = n < N ? widen(Y[r * ldy + n]) * widen(G[r * ldg + n]) : 0.0f;
            }
            s[j] = tree_f32(prod, 0, ORACLE_SLOT);
            if (slots)
                slots[j * slot_ld + r] = s[j];
        }
        dprob[r] = J > 0 ? tree_f32(s, 0, J) : 0.0f;
        free(s);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* The whole operation: Y per expert segment (det_gemm forward), then the
 * slots and dprob.  off holds E + 1 row offsets, off[0] = 0, nondecreasing,
 * off[E] = T; W_e starts at W + e * w_stride. */
int oracle_moe_fwd_dprob(const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                         int64_t w_stride, const int64_t *off, int64_t E, const uint16_t *G,
                         int64_t ldg, uint16_t *Y, int64_t ldy, float *slots, int64_t slot_ld,
                         float *dprob, int64_t T, int64_t N, int64_t K) {
    if (E < 1 || off[0] != 0 || off[E] != T)
        return ORACLE_EINVAL;
    for (int64_t e = 0; e < E; ++e)
        if (off[e + 1] < off[e])
            return ORACLE_EINVAL;
    for (int64_t e = 0; e < E; ++e) {
        int rc = oracle_det_gemm_fwd(X + off[e] * ldx, ldx, W + e * w_stride, ldw,
                                     Y + off[e] * ldy, ldy, off[e + 1] - off[e], N, K);
        if (rc)
            return rc;
    }
    return oracle_moe_dprob(Y, ldy, G, ldg, T, N, slots, slot_ld, dprob);
}

/* ==== Tensor fingerprints and the first-mismatch comparator ====
 *
 * Reading notes "Bitwise-Deterministic Pretraining at Scale", section
 * "5. Fingerprinting Tensors on the GPU": digests are computed in GPU memory
 * from the bit patterns; a whole-tensor hash that ignores positions cannot see
 * a permutation, so order-sensitive data is hashed per row or chunk; the final
 * confirmation is a byte-level comparison.  Section "Reading the first
 * mismatch": the origin is the first traced event whose input digests agree
 * and whose output digests differ.
 *
 * The digest of a byte string of n bytes (a reading: the pages name no hash):
 *   words      w_i, i < ceil(n/8): little-endian 64-bit words of the bytes,
 *              bytes past n read as 0;
 *   mix(z)     the 64-bit finalizer of SplitMix64 (Steele, Lea and Flood,
 *              "Fast splittable pseudorandom number generators", 2014):
 *              z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 *              z *= 0x94D049BB133111EB; z ^= z >> 31   (all mod 2^64);
 *   S          sum over i of mix(w_i + GAMMA * (i + 1)) mod 2^64, with
 *              GAMMA = 0x9E3779B97F4A7C15 (SplitMix64's increment);
 *   digest     mix(S + n).
 * The position enters every term, so moving a word changes the digest; the
 * terms are combined by addition mod 2^64, which is associative, so a
 * parallel evaluation may add them in any grouping and get the same bits.
 * A row digest is the digest of the row's bytes alone (positions counted from
 * the row start).  The first mismatch is the smallest byte index where two
 * byte strings differ, or -1.
 */
#define ORACLE_GAMMA 0x9E3779B97F4A7C15ull

static uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

static uint64_t word_at(const uint8_t *p, int64_t n, int64_t i) {
    uint64_t w = 0;
    for (int b = 0; b < 8; ++b) {
        int64_t k = 8 * i + b;
        if (k < n)
            w |= (uint64_t)p[k] << (8 * b);
    }
    return w;
}

static uint64_t digest_bytes(const uint8_t *p, int64_t n) {
    uint64_t s = 0;
    int64_t W = (n + 7) / 8;
    for (int64_t i = 0; i < W; ++i)
        s += mix64(word_at(p, n, i) + ORACLE_GAMMA * (uint64_t)(i + 1));
    return mix64(s + (uint64_t)n);
}

uint64_t oracle_mix64(uint64_t z) { return mix64(z); }

int oracle_fingerprint(const void *data, int64_t nbytes, uint64_t *digest) {
    if (nbytes < 0 || (nbytes > 0 && !data))
        return ORACLE_EINVAL;
    *digest = digest_bytes((const uint8_t *)data, nbytes);
    return ORACLE_OK;
}

int oracle_fingerprint_rows(const void *data, int64_t rows, int64_t row_bytes, int64_t ld_bytes,
                            uint64_t *digests) {
    if (rows < 0 || row_bytes < 0 || (rows > 1 && ld_bytes < row_bytes))
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        digests[r] = digest_bytes((const uint8_t *)data + r * ld_bytes, row_bytes);
    return ORACLE_OK;
}

int64_t oracle_first_mismatch(const void *a, const void *b, int64_t nbytes) {
    const uint8_t *x = (const uint8_t *)a, *y = (const uint8_t *)b;
    for (int64_t k = 0; k < nbytes; ++k)
        if (x[k] != y[k])
            return k;
    return -1;
}

/* ==== Batch-invariant RMSNorm ====
 *
 * Summary page of "Defeating Nondeterminism in LLM Inference", section on
 * batch-invariant kernel design, RMSNorm: a data-parallel strategy, each row
 * of the batch reduced by one core with the same strategy whatever the batch
 * size (no split reduction, which would trade invariance for parallelism).
 *
 * What is computed for a row x[0..H) with weight w[0..H) (bf16) and eps:
 *   squares        s_i = x_i * x_i in fp32 (exact unless it leaves fp32's
 *                  normal range);
 *   ss             the mid-split tree of fp32 adds over s_0 .. s_{H-1}: a
 *                  range of n squares splits into floor(n/2) on the left and
 *                  the rest on the right, the two sums are added in fp32 (the
 *                  tree shape of det_gemm's leaves, over single elements);
 *   rstd           1 / sqrt(ss / H + eps), each operation rounded once (fp32);
 *   y_i            bf16 rounding (nearest even) of (x_i * rstd) * w_i, both
 *                  products in fp32.
 * The summation order is this design's reading: the page fixes only that the
 * strategy must not depend on the batch.  The mid-split tree depends on H
 * alone (not on a thread count or a chunk width), and has depth ceil(log2 H).
 */
/* ss of one row; s is scratch space for H floats. */
static float rms_sumsq(const uint16_t *x, int64_t H, float *s) {
    for (int64_t i = 0; i < H; ++i) {
        float v = widen(x[i]);
        s[i] = v * v;
    }
    return tree_f32(s, 0, H);
}

int oracle_rmsnorm(const uint16_t *x, int64_t ldx, const uint16_t *w, float eps, uint16_t *y,
                   int64_t ldy, float *rstd, float *sumsq, int64_t R, int64_t H) {
    if (R < 0 || H < 1 || (R > 1 && (ldx < H || ldy < H)))
        return ORACLE_EINVAL;
    int failed = 0;
#pragma omp parallel
    {
        float *s = (float *)malloc((size_t)H * sizeof(float));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < R; ++r) {
            if (!s)
                continue;
            const uint16_t *xr = x + r * ldx;
            float ss = rms_sumsq(xr, H, s);
            float mean = ss / (float)H;
            float rs = 1.0f / sqrtf(mean + eps);
            for (int64_t i = 0; i < H; ++i) {
                float v = widen(xr[i]) * rs;
                y[r * ldy + i] = round_bf16(v * widen(w[i]));
            }
            if (rstd)
                rstd[r] = rs;
            if (sumsq)
                sumsq[r] = ss;
        }
        free(s);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}
