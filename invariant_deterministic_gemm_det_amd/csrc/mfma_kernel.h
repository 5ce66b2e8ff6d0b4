// MFMA det_gemm kernel for gfx950.
//
// Contract (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
// (det_gemm)", sections "Guarantees" and "Ascend NPU backend"): each output is
// the mid-split tree of bf16 adds over L = ceil(R/32) leaves, a leaf being the
// fp32 sum of 32 consecutive products rounded once to bf16 (RNE); no split-K.
//
// Mapping to the hardware:
//   * A leaf of a 16x16 output block is exactly one v_mfma_f32_16x16x32_bf16
//     with a zero accumulator: lane l supplies X(i0 + l%16, 8*(l/16) .. +7) and
//     Y(j0 + l%16, the same 8 indices), so the instruction sums the leaf's 32
//     products.  Every configuration and every shape uses this one instruction
//     with this one lane assignment, so a leaf's bits never depend on M, N,
//     tiling or the position in the tile.
//   * One workgroup owns a BM x BN output tile and walks the whole reduction,
//     two leaves (64 indices) per pipeline stage, both operand tiles staged
//     through double-buffered LDS.  Nothing is shared between workgroups: no
//     atomics, no cross-workgroup merge.
//   * Tree nodes are carried as unrounded fp32 values; a node is rounded once,
//     together with its sibling, by the v_cvt_pk_bf16_f32 that forms the pair
//     its parent adds (bf16_device.h).
//   * When L = b * 2^a with b in {1, 3}, every subtree over an aligned block
//     of b * 2^k leaves has the same shape, so such a block (8 or 12 leaves) is
//     evaluated by a compile-time recursion over its leaf range (all register
//     indices static, no branches).  The block roots then climb the top a - k levels; the few
//     nodes parked there (one per level at most) wait in LDS, rounded to bf16
//     (rounding early does not change the value the parent adds).
//   * Any other L walks the leaves in order and keeps the pending left
//     siblings on a per-lane stack in LDS (streaming post-order: after leaf t,
//     as many merges as there are inner nodes whose range ends at t + 1).
//   * LDS stage tiles are [row][64] bf16 with 128-byte rows; the 16-byte chunk
//     c of row r is stored at chunk c ^ ((r ^ r>>3) & 7), which keeps the MFMA
//     fragment reads and the transposing 2-byte writes free of bank conflicts.
//   * Operands are read with buffer loads from a per-stage scalar base, so the
//     main loop spends no vector instructions on addresses.  An operand whose
//     reduction index is contiguous ("K-major") is copied in 16-byte chunks; one
//     whose row index is contiguous ("MN-major": B of the forward product, both
//     operands of the weight gradient) is loaded in 16-byte chunks along rows
//     and transposed by the LDS writes.
//   * Rows past the end of an operand are clamped to its last row (their
//     outputs are never stored and cannot affect other rows); reduction indices
//     past R are zero-filled on both operands.
#pragma once

#include <type_traits>

#include "bf16_device.h"

namespace detgemm {

enum OutMode { OUT_BF16 = 0, OUT_F32 = 1, OUT_BF16_T = 2, OUT_LEAVES = 3 };
enum TreeMode { TREE_BLOCK = 0, TREE_STACK = 1 };

struct MfmaParams {
    const uint16_t *x;   // X(i, r): K-major x[i*ldx + r]; MN-major x[i + r*ldx]
    int64_t ldx;
    const uint16_t *y;   // Y(j, r): K-major y[j*ldy + r]; MN-major y[j + r*ldy]
    int64_t ldy;
    void *c;             // OUT_BF16/F32: c[i*ldc + j]; OUT_BF16_T: c[j*ldc + i];
    int64_t ldc;         // OUT_LEAVES: c[(i*J + j)*L + leaf]
    int32_t I, J, R, L;
    int32_t tiles_j;
    int32_t xvec, yvec;  // 16-byte aligned rows/columns: vector loads allowed
    int32_t cvec;        // 16-byte aligned output rows: vector stores allowed
    int32_t levels;      // TREE_BLOCK: levels above the blocks; TREE_STACK: stack depth
    int32_t ynt;         // decode kernel: copy Y with non-temporal loads
};

// 16-byte chunk swizzle of the [row][64] stage tiles: measured on gfx950 at the
// full ds_read_b128 rate for the MFMA fragment pattern (16 consecutive rows,
// one chunk each).
__device__ __forceinline__ int lds_key(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, 0x00020000);
}

// ---------------------------------------------------------------- operand staging
//
// Loads one 64-index stage of one operand tile (NR rows) into registers and
// writes it to an LDS buffer.  Chunk geometry is fixed per thread for the whole
// tile; only the scalar base moves from stage to stage.
template <bool KMAJOR, int NR, int NT>
struct Stager {
    static constexpr int TOTAL = KMAJOR ? NR * 8 : (NR / 8) * 64;
    static constexpr int CH = (TOTAL + NT - 1) / NT;
    static_assert(NR % 16 == 0, "tile rows are a multiple of 16");

    const uint16_t *tile_base;  // element (row0, 0) of the operand
    int64_t ld;
    int rows_left;              // rows of the operand at or after row0
    bool vec;
    int voff[CH];      // byte offset of the chunk from the stage base
    int row[CH];       // K-major: tile row; MN-major: first of the chunk's 8 tile rows
    int col[CH];       // K-major: 16-byte chunk index 0..7; MN-major: reduction offset 0..63
    bool fullrows[CH]; // MN-major: all 8 rows of the chunk exist
    bool active[CH];
    u32x4 reg[CH];

    __device__ __forceinline__ void init(const uint16_t *base, int64_t ld_, int row0, int rows,
                                         bool vec_, int tid) {
        ld = ld_;
        rows_left = rows - row0;
        vec = vec_;
        tile_base = KMAJOR ? base + (int64_t)row0 * ld_ : base + row0;
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int c = tid + NT * q;
            active[q] = (TOTAL % NT == 0) || c < TOTAL;
            if (KMAJOR) {
                const int r = c >> 3, cc = c & 7;
                const int rr = r < rows_left ? r : rows_left - 1;
                voff[q] = (int)((int64_t)rr * ld_ * 2) + cc * 16;
                row[q] = r;
                col[q] = cc;
                fullrows[q] = true;
            } else {
                constexpr int RC = NR / 8;
                const int rc = c % RC, rl = c / RC;
                voff[q] = (int)((int64_t)rl * ld_ * 2) + rc * 16;
                row[q] = 8 * rc;
                col[q] = rl;
                fullrows[q] = 8 * rc + 8 <= rows_left;
            }
        }
    }

    // Issue the loads of stage s (reduction indices 64*s ...).
    __device__ __forceinline__ void load(int s, int R) {
        const int r0 = s * 64;
        const uint16_t *sb = KMAJOR ? tile_base + r0 : tile_base + (int64_t)r0 * ld;
        const bool full_stage = r0 + 64 <= R;
        if (vec && full_stage) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(sb);
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                if (!active[q])
                    continue;
                if (KMAJOR || fullrows[q])
                    reg[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[q], 0, 0);
                else
                    reg[q] = load_slow(sb, q, r0, R);
            }
        } else {
#pragma unroll
            for (int q = 0; q < CH; ++q)
                if (active[q])
                    reg[q] = load_slow(sb, q, r0, R);
        }
    }

    // Element-wise load of one chunk with zero fill past R and clamped rows.
    __device__ __forceinline__ u32x4 load_slow(const uint16_t *sb, int q, int r0, int R) const {
        uint16_t e[8];
        const uint16_t *ptr = reinterpret_cast<const uint16_t *>(
            reinterpret_cast<const char *>(sb) + voff[q]);
        if (KMAJOR) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                e[k] = (r0 + 8 * col[q] + k < R) ? ptr[k] : (uint16_t)0;
        } else {
            const bool rok = r0 + col[q] < R;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r = row[q] + k;
                const int shift = (r < rows_left ? r : rows_left - 1) - row[q];
                e[k] = rok ? ptr[shift] : (uint16_t)0;
            }
        }
        u32x4 v;
        v[0] = e[0] | ((uint32_t)e[1] << 16);
        v[1] = e[2] | ((uint32_t)e[3] << 16);
        v[2] = e[4] | ((uint32_t)e[5] << 16);
        v[3] = e[6] | ((uint32_t)e[7] << 16);
        return v;
    }

    // Write the registers of the last load to LDS buffer `buf`.
    __device__ __forceinline__ void store(char *buf) const {
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            if (!active[q])
                continue;
            if (KMAJOR) {
                const int off = row[q] * 128 + ((col[q] ^ lds_key(row[q])) << 4);
                *reinterpret_cast<u32x4 *>(buf + off) = reg[q];
            } else {
                const int rl = col[q];
                const int colbytes = (rl & 7) << 1;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int r = row[q] + k;
                    const int off = r * 128 + (((rl >> 3) ^ lds_key(r)) << 4) + colbytes;
                    const uint32_t w = reg[q][k >> 1];
                    *reinterpret_cast<uint16_t *>(buf + off) =
                        (k & 1) ? (uint16_t)(w >> 16) : (uint16_t)w;
                }
            }
        }
    }
};

// ---------------------------------------------------------------- fragments

template <int FM, int FN>
struct Frag {
    f32x4 v[FM][FN];
};

template <int FM, int FN>
__device__ __forceinline__ Frag<FM, FN> merge_frag(const Frag<FM, FN> &l, const Frag<FM, FN> &r) {
    Frag<FM, FN> o;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
            o.v[a][b] = merge4(l.v[a][b], r.v[a][b]);
    return o;
}

// ---------------------------------------------------------------- tree arithmetic
//
// Two ways to perform the tree's bf16 adds on a fragment (FM x FN blocks of
// 16x16 nodes, each node an unrounded fp32 value).  Both round the two children
// with v_cvt_pk_bf16_f32 and add them in fp32; they give identical bits for
// finite values.
//
// ValuAdd: v_dot2_f32_bf16 against (1.0, 1.0) per node.  Element positions
// never move.
//
// MatrixAdd: the packed pairs of a 16x16 block form the A operand of one
// v_mfma_f32_16x16x32_bf16 whose B operand is a constant 0/1 selector: output
// column p of A-row i is A[i][2p] + A[i][2p+1].  Both products are exact and
// every other product is zero, so the fp32 result equals the exact sum whenever
// that sum fits in 24 bits, and otherwise differs from it by less than the
// distance to the nearest bf16 rounding boundary; the bf16 rounding that follows
// is therefore that of the correctly rounded sum (checked on the device over all
// pairs of finite bf16 values).  An MFMA output row sums a whole A row, so one
// non-finite node (Inf * 0 = NaN) would spoil the other 15 sums of its row: the
// kernel detects non-finite roots and recomputes such a tile with ValuAdd.
// The add also moves element positions: the value of block element (r, c)
// ends up where (c, r) was, so a node's layout parity is the number of adds
// applied to it, i.e. its height in the tree modulo 2; siblings of different
// height parity are aligned by one "flip" (an add with a zero partner).
struct ValuAdd {
    static constexpr bool kTransposes = false;
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> merge(const Frag<FM, FN> &l,
                                                         const Frag<FM, FN> &r, bf16x8) {
        return merge_frag(l, r);
    }
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> flip(const Frag<FM, FN> &x, bf16x8) {
        return x;
    }
};

struct MatrixAdd {
    static constexpr bool kTransposes = true;
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> merge(const Frag<FM, FN> &l,
                                                         const Frag<FM, FN> &r, bf16x8 sel) {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                u32x4 pk;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    pk[v] = pair_bits(round_pair(l.v[a][b][v], r.v[a][b][v]));
                o.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, pk), sel, zero, 0, 0, 0);
            }
        return o;
    }
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> flip(const Frag<FM, FN> &x, bf16x8 sel) {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                u32x4 pk;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    pk[v] = pair_bits(round_pair(x.v[a][b][v], 0.0f));
                o.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, pk), sel, zero, 0, 0, 0);
            }
        return o;
    }
};

// Selector B operand for MatrixAdd: lane 16g + j holds B[8g .. 8g+7][j]; the
// entries B[2j][j] and B[2j+1][j] are 1.0 (they sit in lane 16*(j/4) + j, dword
// j % 4), all others 0.
__device__ __forceinline__ bf16x8 add_selector(int lane) {
    const int j = lane & 15, g = lane >> 4;
    u32x4 s = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q)
        s[q] = ((j >> 2) == g && (j & 3) == q) ? 0x3F803F80u : 0u;
    return __builtin_bit_cast(bf16x8, s);
}

// Height of the mid-split tree over n leaves: ceil(log2 n).
constexpr int tree_height(int n) { return n <= 1 ? 0 : 1 + tree_height(n - n / 2); }

// ---------------------------------------------------------------- engine
//
// The per-workgroup pipeline: operand staging, the two MFMA leaves of a stage,
// and the LDS slots where pending tree nodes wait.
template <bool XK, bool YK, int FM, int FN, int WM, int WN>
struct Engine {
    static constexpr int NW = WM * WN;
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 16 * FM * WM;
    static constexpr int BN = 16 * FN * WN;
    static constexpr int BUF = (BM + BN) * 128;             // one stage, both operands
    static constexpr int PARK_FRAG = NW * 64 * 8;           // one fragment of one level, all lanes
    static constexpr int PARK_LEVEL = FM * FN * PARK_FRAG;  // one parked level, all waves
    typedef Frag<FM, FN> F;

    const MfmaParams &p;
    char *smem;
    Stager<XK, BM, NT> sx;
    Stager<YK, BN, NT> sy;
    int ox[FM][2], oy[FN][2];
    int park_off;
    int S;

    static constexpr int lds_bytes(int levels) { return 2 * BUF + levels * PARK_LEVEL; }

    __device__ __forceinline__ Engine(const MfmaParams &p_, char *smem_, int i0, int j0)
        : p(p_), smem(smem_) {
        const int tid = threadIdx.x;
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = wave % WM, wn = wave / WM;
        sx.init(p.x, p.ldx, i0, p.I, p.xvec != 0, tid);
        sy.init(p.y, p.ldy, j0, p.J, p.yvec != 0, tid);
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            const int row = wm * FM * 16 + a * 16 + (lane & 15);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ox[a][h] = row * 128 + (((4 * h + (lane >> 4)) ^ lds_key(row)) << 4);
        }
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int row = wn * FN * 16 + b * 16 + (lane & 15);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                oy[b][h] = BM * 128 + row * 128 + (((4 * h + (lane >> 4)) ^ lds_key(row)) << 4);
        }
        park_off = 2 * BUF + (wave * 64 + lane) * 8;
        S = (p.R + 63) / 64;
    }

    // Stage 0 into LDS buffer 0, stage 1 into registers.
    __device__ __forceinline__ void prologue() {
        sx.load(0, p.R);
        sy.load(0, p.R);
        sx.store(smem);
        sy.store(smem + BM * 128);
        if (S > 1) {
            sx.load(1, p.R);
            sy.load(1, p.R);
        }
        __syncthreads();
    }

    // Both leaves of stage s, whose operands sit in LDS buffer PAR (= s & 1).
    // Also moves stage s+1 from registers to the other buffer, issues the loads
    // of stage s+2 and ends with the workgroup barrier.
    template <int PAR>
    __device__ __forceinline__ void stage(int s, F &l0, F &l1) {
        const char *buf = smem + PAR * BUF;
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 fa[FM], fb[FN];
#pragma unroll
            for (int a = 0; a < FM; ++a)
                fa[a] = *reinterpret_cast<const bf16x8 *>(buf + ox[a][h]);
#pragma unroll
            for (int b = 0; b < FN; ++b)
                fb[b] = *reinterpret_cast<const bf16x8 *>(buf + oy[b][h]);
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const f32x4 acc =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], zero, 0, 0, 0);
                    if (h == 0)
                        l0.v[a][b] = acc;
                    else
                        l1.v[a][b] = acc;
                }
        }
        if (s + 1 < S) {
            char *nbuf = smem + (PAR ^ 1) * BUF;
            sx.store(nbuf);
            sy.store(nbuf + BM * 128);
            if (s + 2 < S) {
                sx.load(s + 2, p.R);
                sy.load(s + 2, p.R);
            }
        }
        __syncthreads();
    }

    // Pending nodes wait in LDS rounded to bf16, each lane in its own slots.
    __device__ __forceinline__ void park(int slot, const F &v) {
        char *base = smem + park_off + slot * PARK_LEVEL;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                uint2 w;
                w.x = pair_bits(round_pair(v.v[a][b][0], v.v[a][b][1]));
                w.y = pair_bits(round_pair(v.v[a][b][2], v.v[a][b][3]));
                *reinterpret_cast<uint2 *>(base + (a * FN + b) * PARK_FRAG) = w;
            }
    }

    __device__ __forceinline__ F unpark(int slot) const {
        const char *base = smem + park_off + slot * PARK_LEVEL;
        F v;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const uint2 w = *reinterpret_cast<const uint2 *>(base + (a * FN + b) * PARK_FRAG);
                v.v[a][b][0] = __uint_as_float(w.x << 16);
                v.v[a][b][1] = __uint_as_float(w.x & 0xFFFF0000u);
                v.v[a][b][2] = __uint_as_float(w.y << 16);
                v.v[a][b][3] = __uint_as_float(w.y & 0xFFFF0000u);
            }
        return v;
    }
};

// ---------------------------------------------------------------- static block

// Evaluates the subtree over the BLK leaves of one aligned block, starting at
// global stage `s0` (even), by compile-time recursion over the leaf range.
template <class E, int BLK, class Arith>
struct BlockEval {
    typedef typename E::F F;
    E &e;
    int s0;
    bf16x8 sel;
    F odd;  // second leaf of the most recent stage

    template <int T>
    __device__ __forceinline__ F leaf() {
        if constexpr (T % 2 == 0) {
            F l0;
            e.template stage<(T / 2) & 1>(s0 + T / 2, l0, odd);
            return l0;
        } else {
            return odd;
        }
    }

    template <int LO, int HI>
    __device__ __forceinline__ F eval() {
        if constexpr (HI - LO == 1) {
            return leaf<LO>();
        } else {
            constexpr int MID = LO + (HI - LO) / 2;
            F l = eval<LO, MID>();
            const F r = eval<MID, HI>();
            // the left half is never taller; align layout parities of the two
            // children when their heights differ by one
            if constexpr (Arith::kTransposes &&
                          (tree_height(MID - LO) % 2) != (tree_height(HI - MID) % 2))
                l = Arith::flip(l, sel);
            return Arith::merge(l, r, sel);
        }
    }
};

// Number of inner nodes of the mid-split tree over [0, L) whose leaf range
// ends at leaf t (hi == t + 1).
__device__ __forceinline__ int merges_after(int t, int L) {
    int lo = 0, hi = L, count = 0;
    while (hi - lo > 1) {
        if (hi == t + 1)
            ++count;
        const int mid = lo + (hi - lo) / 2;
        if (t < mid)
            hi = mid;
        else
            lo = mid;
    }
    return count;
}

template <int FM, int FN>
__device__ __forceinline__ void quad_bits(const Frag<FM, FN> &x, int a, int b, uint16_t v4[4]) {
    const uint32_t lo = pair_bits(round_pair(x.v[a][b][0], x.v[a][b][1]));
    const uint32_t hi = pair_bits(round_pair(x.v[a][b][2], x.v[a][b][3]));
    v4[0] = (uint16_t)lo;
    v4[1] = (uint16_t)(lo >> 16);
    v4[2] = (uint16_t)hi;
    v4[3] = (uint16_t)(hi >> 16);
}

// Height of the mid-split tree over L leaves at run time: ceil(log2 L).
__device__ __forceinline__ int tree_height_rt(int L) { return L <= 1 ? 0 : 32 - __clz(L - 1); }

// Blocks of BLK leaves, then the climb through the levels above them; the
// pending left siblings of the upper levels wait in LDS.
template <class E, int BLK, class Arith>
__device__ __forceinline__ void run_blocks(E &e, const MfmaParams &p, bf16x8 sel,
                                           typename E::F &root) {
    const int nblk = p.L / BLK;
    for (int blk = 0; blk < nblk; ++blk) {
        BlockEval<E, BLK, Arith> ev{e, blk * (BLK / 2), sel};
        typename E::F v = ev.template eval<0, BLK>();
        int h = 0;
        while (h < p.levels && ((blk >> h) & 1)) {
            v = Arith::merge(e.unpark(h), v, sel);
            ++h;
        }
        if (h < p.levels)
            e.park(h, v);
        else
            root = v;
    }
}

// Rounds the root to bf16 and stores it.  With odd layout parity, lane
// 16g + c, register v holds block element (row c, column 4g + v); otherwise
// element (row 4g + v, column c).  A zero root is stored as +0, the sign the
// sequential definition gives every exact zero.
template <int OUT, int FM, int FN>
__device__ __forceinline__ void store_root(const MfmaParams &p, const Frag<FM, FN> &root,
                                           bool odd, int i0, int j0, int wm, int wn, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            uint16_t v4[4];
            quad_bits(root, a, b, v4);
            const int ib = i0 + wm * FM * 16 + a * 16;
            const int jb = j0 + wn * FN * 16 + b * 16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = ib + (odd ? c : 4 * g + v);
                const int j = jb + (odd ? 4 * g + v : c);
                const uint16_t h = (v4[v] & 0x7FFF) ? v4[v] : (uint16_t)0;
                if (i < p.I && j < p.J) {
                    if (OUT == OUT_BF16)
                        static_cast<uint16_t *>(p.c)[(int64_t)i * p.ldc + j] = h;
                    else if (OUT == OUT_F32)
                        static_cast<float *>(p.c)[(int64_t)i * p.ldc + j] =
                            __uint_as_float((uint32_t)h << 16);
                    else
                        static_cast<uint16_t *>(p.c)[(int64_t)j * p.ldc + i] = h;
                }
            }
        }
}

// ---------------------------------------------------------------- the kernel

template <bool XK, bool YK, int OUT, int TREE, int TB, int TK, int FM, int FN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void mfma_kernel(MfmaParams p) {
    typedef Engine<XK, YK, FM, FN, WM, WN> E;
    typedef typename E::F F;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int tile = blockIdx.x;
    const int i0 = (tile / p.tiles_j) * E::BM;
    const int j0 = (tile % p.tiles_j) * E::BN;

    E e(p, smem, i0, j0);
    e.prologue();
    F root;

    if constexpr (OUT == OUT_LEAVES) {
        uint16_t *out = static_cast<uint16_t *>(p.c);
        for (int s = 0; s < e.S; s += 2) {
            F l[4];
            e.template stage<0>(s, l[0], l[1]);
            if (s + 1 < e.S)
                e.template stage<1>(s + 1, l[2], l[3]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 2 * s + q;
                if (t >= p.L)
                    break;
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        uint16_t v4[4];
                        quad_bits(l[q], a, b, v4);
                        const int j = j0 + wn * FN * 16 + b * 16 + (lane & 15);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int i = i0 + wm * FM * 16 + a * 16 + 4 * (lane >> 4) + v;
                            if (i < p.I && j < p.J)
                                out[((int64_t)i * p.J + j) * p.L + t] = v4[v];
                        }
                    }
            }
        }
        return;
    } else if constexpr (TREE == TREE_BLOCK) {
        const bf16x8 sel = add_selector(lane);
        run_blocks<E, TB << TK, MatrixAdd>(e, p, sel, root);
        // A non-finite root may have spilled NaN into the other sums of its
        // MatrixAdd rows: recompute such a tile with per-element VALU adds.
        bool nonfinite = false;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    nonfinite |= !(__builtin_fabsf(root.v[a][b][v]) <= 3.40282347e38f);
        if (__syncthreads_or(nonfinite)) {
            e.prologue();
            run_blocks<E, TB << TK, ValuAdd>(e, p, sel, root);
            store_root<OUT>(p, root, false, i0, j0, wm, wn, lane);
        } else {
            store_root<OUT>(p, root, (tree_height_rt(p.L) & 1) != 0, i0, j0, wm, wn, lane);
        }
    } else {
        int top = 0;
        for (int s = 0; s < e.S; s += 2) {
            F l[4];
            e.template stage<0>(s, l[0], l[1]);
            if (s + 1 < e.S)
                e.template stage<1>(s + 1, l[2], l[3]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 2 * s + q;
                if (t >= p.L)
                    break;
                F v = l[q];
                const int m = merges_after(t, p.L);
                for (int k = 0; k < m; ++k) {
                    --top;
                    v = merge_frag(e.unpark(top), v);
                }
                if (t + 1 < p.L) {
                    e.park(top, v);
                    ++top;
                } else {
                    root = v;
                }
            }
        }
        store_root<OUT>(p, root, false, i0, j0, wm, wn, lane);
    }
}

}  // namespace detgemm
