// Wide-wave MFMA det_gemm kernel for gfx950, for leaf counts L = m * 2^a with
// m = 1, 3, 5, 7 or an odd m whose unit schedule is instantiated (11, 17, 19,
// 25, 27, 35, 37, 43).
//
// Same leaves and same tree as mfma_kernel.h and mfma_fast.h, hence the same
// bits (RL-Kernel operator page "Batch-Invariant Deterministic GEMM (det_gemm)",
// sections "Guarantees" and "Ascend NPU backend": 32-element leaves rounded once
// to bf16, mid-split tree of bf16 adds).  With L = 2^a the mid-split tree is the
// perfect binary tree, and its lowest inner nodes are the pairs (2s, 2s + 1),
// i.e. the two leaves of pipeline stage s; with L = m * 2^a it is the perfect
// tree over units of m leaves (WideTree below).  What differs is the work
// layout:
//   * each wave owns FM x FN blocks of 16x16 outputs (4 x 2: 64 x 32), so every
//     step of the tree is FM * FN independent matrix-core instructions and a
//     dependent step never waits on the latency of the previous one;
//   * a stage's two leaf MFMAs per block are rounded at once into one packed
//     pair (v_cvt_pk_bf16_f32), and the next stage begins with the tree add of
//     that pair on the matrix core (selector MFMA, mfma_fast.h), followed by the
//     climb of the resulting node; the leaf MFMAs of the stage come last, after
//     their fragment reads have had the tree work to complete;
//   * every node that waits for its right sibling is kept rounded and packed
//     (two registers per block), never as fp32;
//   * G = 2^GL stages are unrolled, so the pending nodes of the GL lowest levels
//     of the pair tree sit in registers with static indices; the root of a group
//     of stages climbs RU more levels held in registers (uniform branches on the
//     group index), then levels parked in LDS;
//   * operand staging is the direct global -> LDS copy of mfma_fast.h with
//     NBUF stage buffers; fragment reads use one base register per operand and
//     leaf half, the fragment index being an immediate offset.
#pragma once

#include "mfma_fast.h"

namespace detgemm {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A tree node rounded to bf16 and packed: per 16x16 block, the lane's four
// values as the pairs (v0, v1), (v2, v3).  Vector-typed so that the compiler
// keeps every node in registers.
template <int FM, int FN>
struct WPacked {
    u32x2 w[FM][FN];
};

template <int FM, int FN>
__device__ __forceinline__ WPacked<FM, FN> wpack(const Frag<FM, FN> &x) {
    WPacked<FM, FN> o;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            o.w[a][b].x = pair_bits(round_pair(x.v[a][b][0], x.v[a][b][1]));
            o.w[a][b].y = pair_bits(round_pair(x.v[a][b][2], x.v[a][b][3]));
        }
    return o;
}

// Tree adds of packed children on the matrix core: the A operand of a lane is
// (left child's four values, right child's four values), the B operand the
// split selector of mfma_fast.h; the parent's fp32 values land transposed.
struct WideMatrixAdd {
    static constexpr bool kTransposes = true;
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> add(const WPacked<FM, FN> &l,
                                                       const WPacked<FM, FN> &r, bf16x8 sel) {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const u32x4 A = __builtin_shufflevector(l.w[a][b], r.w[a][b], 0, 1, 2, 3);
                o.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A),
                                                                    sel, zero, 0, 0, 0);
            }
        return o;
    }
};

// The same adds element by element on the VALU: exact IEEE behaviour for
// non-finite values, and positions never move.
struct WideValuAdd {
    static constexpr bool kTransposes = false;
    __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> add(const WPacked<FM, FN> &l,
                                                       const WPacked<FM, FN> &r, bf16x8) {
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                o.v[a][b][0] = lo(l.w[a][b].x) + lo(r.w[a][b].x);
                o.v[a][b][1] = hi(l.w[a][b].x) + hi(r.w[a][b].x);
                o.v[a][b][2] = lo(l.w[a][b].y) + lo(r.w[a][b].y);
                o.v[a][b][3] = hi(l.w[a][b].y) + hi(r.w[a][b].y);
            }
        return o;
    }
};

// Stores a tile's roots (bf16, as [row][column] of the output, i.e. transposed
// for OUT_BF16_T) through LDS, so that global memory sees whole 16-byte chunks
// of output rows instead of 2-byte writes scattered over 16 rows.  The LDS rows
// are padded by 16 bytes, which spreads the lanes of a write over the banks.
// Needs every wave past a barrier that ends its use of `lds`.  A zero root is
// stored as +0, the sign the sequential definition gives every exact zero.
// ---- per-token epilogue of the MoE grouped GEMM (reading notes on
// bitwise-deterministic pretraining in Megatron Core, section "Kernel
// redesign: the grouped-GEMM epilogue": private per-N-tile slots and a fixed
// tree instead of atomic adds).  A slot is the mid-split tree of fp32 adds over
// the 128 column positions of one output tile row, positions past the last
// column holding +0; for 128 positions that is the perfect pairwise tree.
constexpr int kSlot = 128;

__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <class T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    return reinterpret_cast<T *>(uniform64(reinterpret_cast<int64_t>(p)));
}

// Row groups of a grouped launch (see mfma_wide_grouped_kernel) and the
// operands of the epilogue: g(i, j) = g[i*ldg + j] for the rows i of the
// whole launch; the tile at columns j0 .. j0+127 writes, for each of its rows
// i, the slot of c(i, j) * g(i, j) to slots[(j0/128)*slot_ld + i].
// slots == nullptr: no epilogue.
constexpr int kMaxGroups = 128;

struct GroupTable {
    int32_t groups;
    int32_t tile_start[kMaxGroups + 1];
    int32_t row_start[kMaxGroups];
    int32_t rows[kMaxGroups];
    int64_t y_stride;
    const uint16_t *g;
    int64_t ldg;
    float *slots;
    int64_t slot_ld;
    // Tail balancing: tiles split_from .. tile_start[groups]-1 each run as two
    // half-height tiles (workgroups split_from + 2 (t - split_from) and the
    // next), whose trees are split at the root over two wave groups
    // (split_levels: the levels above the groups of stages of one wave group).
    int32_t split_from;
    int32_t split_levels;
};

// What the epilogue of a grouped tile needs, written by the workgroup at the
// start of the dynamic LDS (its engine's buffers start kEpiLds bytes later):
// read back at the end of the tile rather than held in registers through the
// main loop.  r0: the first row of the tile's group.
struct EpiInfo {
    const uint16_t *g;
    float *slots;
    int64_t ldg, slot_ld;
    int32_t r0;
};
constexpr int kEpiLds = 64;

// The slot of one row whose 128 products are held two per lane (columns
// 2*lane and 2*lane + 1): level 1 is the lane's own pair, level k joins lanes
// 2^(k-2) apart.  IEEE addition is commutative, so the two lanes of a join hold
// the same node; every lane ends with the slot.
__device__ __forceinline__ float slot_tree(float p0, float p1) {
    float v = p0 + p1;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        v = v + __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// The same tree with 8 consecutive columns per lane and 16 lanes per row
// (lanes 16q .. 16q+15 hold one row): levels 1-3 inside the lane, levels 4-7
// join lanes 1, 2, 4, 8 apart; every lane of the 16 ends with the slot.
__device__ __forceinline__ float slot_tree8(const float (&pr)[8]) {
    float v = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
        v = v + __shfl_xor(v, m, 16);
    return v;
}

// Byte offset of byte `byte` of staged row r.  Padded (SWZ false): rows
// 2 * COLS + 16 bytes apart.  Swizzled (SWZ true): rows 2 * COLS bytes apart,
// 16-byte chunk c of row r stored at chunk c ^ (r mod 16) (at most 16 chunks
// per row), which spreads the 16 rows of one write over the banks as the
// padding does, in exactly ROWS * COLS * 2 bytes.
template <int COLS, bool SWZ>
__device__ __forceinline__ int staged_off(int r, int byte) {
    if constexpr (SWZ) {
        constexpr int CHM = (COLS / 8 < 16 ? COLS / 8 : 16) - 1;
        return r * (COLS * 2) + ((((byte >> 4) ^ (r & CHM)) << 4) | (byte & 15));
    } else {
        return r * (COLS * 2 + 16) + byte;
    }
}

// Publishes each wave's non-finite flag through one dword per wave of `flags`
// (LDS) with one barrier, which also publishes whatever the waves wrote to the
// LDS before it.  Returns whether any wave's flag is set; in that case a second
// barrier has retired every wave's read of the flags, so the caller may reuse
// the LDS.
template <int NW>
__device__ __forceinline__ bool publish_nonfinite(int *flags, bool nonfinite) {
    static_assert(NW % 4 == 0, "flags are read four at a time");
    const bool any = __builtin_amdgcn_ballot_w64(nonfinite) != 0;
    if ((threadIdx.x & 63) == 0)
        flags[threadIdx.x >> 6] = any ? 1 : 0;
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int q = 0; q < NW; q += 4) {
        const uint4 f = *reinterpret_cast<const uint4 *>(flags + q);
        r |= f.x | f.y | f.z | f.w;
    }
    if (r != 0) {
        __syncthreads();
        return true;
    }
    return false;
}

// Two rounded roots packed in a dword, with a zero of either sign stored as
// +0: within a half, x & 0x7FFF is nonzero exactly when adding 0x7FFF to it
// carries into bit 15 (no carry crosses into the other half), which selects
// the mask 0xFFFF or 0 for that half.
__device__ __forceinline__ uint32_t plus_zero_pair(uint32_t w) {
    const uint32_t nz = (((w & 0x7FFF7FFFu) + 0x7FFF7FFFu) & 0x80008000u) >> 15;
    return w & (nz * 0xFFFFu);
}

// Whether either bf16 of a packed pair is Inf or NaN (exponent all ones).
__device__ __forceinline__ bool pair_nonfinite(uint32_t w) {
    const uint32_t e = (w & 0x7F807F80u) ^ 0x7F807F80u;
    return (e & 0xFFFFu) == 0 || (e >> 16) == 0;
}

// Writes a tile's roots to the staged rows.  ROWROW: the lane's four values of
// a block lie in one staged row (one 8-byte write), else in four rows.
// Returns whether a rounded root of this lane is Inf or NaN (a non-finite
// fp32 root stays non-finite when rounded).
template <bool T, bool ROWROW, int FM, int FN, int COLS, bool SWZ>
__device__ __forceinline__ bool stage_roots(const Frag<FM, FN> &root, int wm, int wn, int lane,
                                            char *lds) {
    const int g = lane >> 4, c = lane & 15;
    bool nonfinite = false;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const uint32_t lo = plus_zero_pair(pair_bits(round_pair(root.v[a][b][0], root.v[a][b][1])));
            const uint32_t hi = plus_zero_pair(pair_bits(round_pair(root.v[a][b][2], root.v[a][b][3])));
            nonfinite |= pair_nonfinite(lo) | pair_nonfinite(hi);
            const int rb = wm * FM * 16 + a * 16, cb = wn * FN * 16 + b * 16;  // block origin (i, j)
            if constexpr (ROWROW) {
                const int r = T ? cb + c : rb + c;
                const int col = T ? rb + 4 * g : cb + 4 * g;
                *reinterpret_cast<uint2 *>(lds + staged_off<COLS, SWZ>(r, col * 2)) = make_uint2(lo, hi);
            } else {
                const uint16_t v4[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                        (uint16_t)(hi >> 16)};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = T ? cb + 4 * g + v : rb + 4 * g + v;
                    const int col = T ? rb + c : cb + c;
                    *reinterpret_cast<uint16_t *>(lds + staged_off<COLS, SWZ>(r, col * 2)) = v4[v];
                }
            }
        }
    return nonfinite;
}

// Copies a staged block of ROWS rows of COLS bf16 values to the output rows
// row0 .. and columns col0 .. (only the first rows_ok rows and cols_ok
// columns exist), 16 bytes per thread and pass; `tid` < 64 * NW.
template <int ROWS, int COLS, int NW, bool SWZ>
__device__ __forceinline__ void read_out_staged(const MfmaParams &p, const char *lds, int row0, int col0,
                                                int rows_ok, int cols_ok, int tid) {
    uint16_t *out = static_cast<uint16_t *>(p.c);
    constexpr int CH = COLS / 8;  // chunks per row
    static_assert(ROWS * CH % (64 * NW) == 0, "the passes cover the staged rows");
#pragma unroll
    for (int k = 0; k < ROWS * CH / (64 * NW); ++k) {
        const int q = tid + k * 64 * NW;
        const int r = q / CH, ch = q % CH;
        if (r >= rows_ok)
            continue;
        const uint4 w = *reinterpret_cast<const uint4 *>(lds + staged_off<COLS, SWZ>(r, ch * 16));
        uint16_t *dst = out + (int64_t)(row0 + r) * p.ldc + col0 + ch * 8;
        if (p.cvec && ch * 8 + 8 <= cols_ok) {
            *reinterpret_cast<uint4 *>(dst) = w;
        } else {
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (ch * 8 + e < cols_ok)
                    dst[e] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// EPI: also the slots of the epilogue (operands in the EpiInfo at the start of
// the dynamic LDS; this tile's rows start at its row r0).  FLAGS: the
// non-finite check of the rounded roots rides on the staging barrier
// (publish_nonfinite); a tile with a non-finite root is then not stored and
// true is returned.
template <int OUT, int FM, int FN, int BM, int BN, int NW, bool EPI = false, bool SWZ = false,
          bool FLAGS = false>
__device__ __forceinline__ bool store_staged(const MfmaParams &p, const Frag<FM, FN> &root, bool odd,
                                             int i0, int j0, int wm, int wn, int lane, char *lds,
                                             int *flags = nullptr) {
    constexpr bool T = OUT == OUT_BF16_T;
    constexpr int ROWS = T ? BN : BM, COLS = T ? BM : BN;  // of the staged block
    // Per-token epilogue: a row's slot is reduced by 16 lanes holding 8
    // columns each; a wave takes 4 rows per pass.  The G chunks are loaded
    // first, so that their latency overlaps the staging.
    constexpr bool kEpi = EPI && !T && COLS == kSlot;
    constexpr int EP = kEpi ? ROWS / (NW * 4) : 1;  // passes
    static_assert(!kEpi || EP * NW * 4 == ROWS, "the epilogue passes cover the tile rows");
    extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
    const EpiInfo *info = reinterpret_cast<const EpiInfo *>(dyn_lds);
    const uint16_t *eg = nullptr;
    float *eslots = nullptr;
    int64_t eldg = 0, eslot_ld = 0;
    int r0 = 0;
    if constexpr (kEpi) {
        eg = uniform_ptr(info->g);
        eslots = uniform_ptr(info->slots);
        eldg = uniform64(info->ldg);
        eslot_ld = uniform64(info->slot_ld);
        r0 = __builtin_amdgcn_readfirstlane(info->r0);
    }
    const bool epi = kEpi && eslots != nullptr;
    const int c8 = (lane & 15) * 8;
    const int erow = ((threadIdx.x >> 6) * 4 + (lane >> 4));  // + 4 * NW per pass
    uint4 gq[EP];
    if constexpr (kEpi) {
        if (epi) {
            const int rows_in = p.I - i0, cols_in = p.J - j0;
#pragma unroll
            for (int k = 0; k < EP; ++k) {
                const int r = erow + k * 4 * NW;
                gq[k] = make_uint4(0u, 0u, 0u, 0u);
                if (r < rows_in) {
                    const uint16_t *gr = eg + (int64_t)(r0 + i0 + r) * eldg + j0 + c8;
                    if (c8 + 8 <= cols_in) {
                        gq[k] = *reinterpret_cast<const uint4 *>(gr);
                    } else {
                        uint32_t w[4] = {0u, 0u, 0u, 0u};
                        for (int e = 0; e < 8 && c8 + e < cols_in; ++e)
                            w[e >> 1] |= (uint32_t)gr[e] << (16 * (e & 1));
                        gq[k] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                }
            }
        }
    }
    // the lane's four values of a block: odd parity (rb + c, cb + 4g + v), even
    // (rb + 4g + v, cb + c); they are contiguous in a staged row when that row
    // is i (odd, not T) or j (even, T).  One uniform branch on the parity, so
    // each variant is straight-line code.
    const bool staged_nonfinite = odd != T ? stage_roots<T, true, FM, FN, COLS, SWZ>(root, wm, wn, lane, lds)
                                           : stage_roots<T, false, FM, FN, COLS, SWZ>(root, wm, wn, lane, lds);
    if constexpr (FLAGS) {
        if (publish_nonfinite<NW>(flags, staged_nonfinite))
            return true;
    } else {
        __syncthreads();
    }
    // read out: 16-byte chunks of staged rows
    const int row0 = T ? j0 : i0, col0 = T ? i0 : j0;
    const int rows_ok = (T ? p.J : p.I) - row0, cols_ok = (T ? p.I : p.J) - col0;
    read_out_staged<ROWS, COLS, NW, SWZ>(p, lds, row0, col0, rows_ok, cols_ok, threadIdx.x);
    // Slots from the staged rows (the values just stored).  Columns past the
    // last one hold the product +0, as the slot definition requires (not y * 0,
    // which is -0 for negative y).
    if constexpr (kEpi) {
        if (epi) {
            float *slot = eslots + (int64_t)(col0 / kSlot) * eslot_ld + r0 + row0;
#pragma unroll
            for (int k = 0; k < EP; ++k) {
                const int r = erow + k * 4 * NW;
                const uint4 yq = *reinterpret_cast<const uint4 *>(lds + staged_off<COLS, SWZ>(r, c8 * 2));
                const uint32_t yw[4] = {yq.x, yq.y, yq.z, yq.w};
                const uint32_t gw[4] = {gq[k].x, gq[k].y, gq[k].z, gq[k].w};
                float pr[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pr[e] = c8 + e < cols_ok
                                ? bf16_value((yw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) *
                                      bf16_value((gw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu)
                                : 0.0f;
                const float v = slot_tree8(pr);
                if ((lane & 15) == 0 && r < rows_ok)
                    slot[r] = v;
            }
        }
    }
    return false;
}

// With NBUF >= 3 the copies are issued early: before the barrier that opens
// stage s, the first NP waves (the ones the issue arbiter favours, which reach
// the barrier first) issue the copies of stage s + NBUF - 2, so the copy issue
// happens in time those waves would spend waiting, and the waves that finish
// last issue no copies.  With NBUF == 2 every wave issues its share right
// after the barrier (the copies need a stage of lead time either way).
template <bool XK, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF>
struct WideEngine {
    static constexpr int kOUT = OUT, kWM = WM;
    static constexpr int NW = WM * WN;
    static constexpr int BM = 16 * FM * WM;
    static constexpr int BN = 16 * FN * WN;
    static constexpr int XB = BM * 128, YB = BN * 128;
    static constexpr int BUF = XB + YB;
    static constexpr int PARK_FRAG = NW * 64 * 8;
    static constexpr int PARK_LEVEL = FM * FN * PARK_FRAG;
    static constexpr int kFM = FM, kFN = FN;
    static constexpr int lds_bytes(int parked) { return NBUF * BUF + parked * PARK_LEVEL; }
    typedef Frag<FM, FN> F;
    typedef WPacked<FM, FN> P;
    static constexpr bool kEarly = NBUF >= 3;
    static constexpr int NP = kEarly ? NW / 2 : NW;  // waves issuing copies
    typedef DirectStager<XK, BM, NP> SX;
    typedef DirectStager<YK, BN, NP> SY;
    static constexpr int LOADS = SX::PER_WAVE + SY::PER_WAVE;
    static_assert(NBUF >= 2, "at least two stage buffers");

    char *lds;   // the workgroup's LDS allocation
    char *smem;  // the stage buffers
    SX sx;
    SY sy;
    bool producer;  // this wave issues copies
    int xoff[XK ? 2 : FM];  // K-major: per leaf half h; MN-major: per fragment
    int yoff[YK ? 2 : FN];
    char *park_lane;  // this lane's first parking slot
    const char *cur;  // stage buffer of the current stage
    int S;
    bf16x8 fa[2][FM], fb[2][FN];  // [leaf][fragment] of the current stage

    // Fragment read offsets of a K-major operand: rows r0 + 16a + i (i = lane
    // % 16), 16-byte chunk 4h + lane / 16 XOR-swizzled by (row >> 1) & 7, which
    // does not depend on a (16a / 2 is a multiple of 8), so fragment a is at the
    // fixed distance 16 * 128 * a.
    __device__ __forceinline__ static void kmajor_offsets(int *off, int r0, int lane) {
        const int row = r0 + (lane & 15);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            off[h] = row * 128 + (((4 * h + (lane >> 4)) ^ lds_key(row)) << 4);
    }

    // Fragment read offsets of an MN-major operand of NR rows per reduction
    // index (natural [r][row] layout, chunk swizzle mn_key of the reduction
    // index): lane 4m + q of group G reads reduction rows 32h + 8G + 4half + m,
    // operand rows 4q .. 4q+3 of its fragment.  The swizzle key depends only on
    // m and G, so the (h, half) variants are fixed distances from one base.
    template <int NR>
    __device__ __forceinline__ static int mnmajor_offset(int rbase, int lane) {
        constexpr int NC = NR / 8;
        const int i = lane & 15, G = lane >> 4;
        const int m = i >> 2, q = i & 3;
        const int r = 8 * G + m;
        const int col = rbase + 4 * q;
        const int lc = col >> 3;
        return r * (NR * 2) + (((lc ^ mn_key<NC>(r)) << 4) | ((col & 7) * 2));
    }

    // LDS: the parked tree levels first (`parked` of them), so that a lane's
    // slots are within the immediate offset of one address register, then the
    // NBUF stage buffers.
    // tid0: the first thread of the engine's waves (a workgroup may hold two
    // engines, one per wave group).
    __device__ __forceinline__ WideEngine(const MfmaParams &p, char *lds_, int parked, int i0, int j0,
                                          int tid0 = 0)
        : lds(lds_), smem(lds_ + parked * PARK_LEVEL) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x - tid0) >> 6);
        const int wm = wave % WM, wn = wave / WM;
        producer = wave < NP;
        sx.init(p.x, p.ldx, i0, p.I, producer ? wave : 0, lane);
        sy.init(p.y, p.ldy, j0, p.J, producer ? wave : 0, lane);
        if constexpr (XK) {
            kmajor_offsets(xoff, wm * FM * 16, lane);
        } else {
#pragma unroll
            for (int a = 0; a < FM; ++a)
                xoff[a] = mnmajor_offset<BM>(wm * FM * 16 + a * 16, lane);
        }
        if constexpr (YK) {
            kmajor_offsets(yoff, wn * FN * 16, lane);
            yoff[0] += XB;  // the Y tile follows the X tile in a stage buffer
            yoff[1] += XB;
        } else {
#pragma unroll
            for (int b = 0; b < FN; ++b)
                yoff[b] = XB + mnmajor_offset<BN>(wn * FN * 16 + b * 16, lane);
        }
        S = p.R / 64;
        park_lane = lds_ + (threadIdx.x - tid0) * 8;
    }

    // Stage buffer k (0 or 1) of the two that nothing can still read or fill
    // once every wave is past the barrier of the last stage S - 1: those of
    // stages S - 3 and S - 2 (or never used), all copies done (NBUF >= 3).
    __device__ __forceinline__ char *free_buffer(int k) const {
        static_assert(NBUF >= 3, "two free stage buffers at the end of the tile");
        return smem + ((unsigned)(S + k) % NBUF) * BUF;
    }

    __device__ __forceinline__ void issue(int s) {
        if (NP == NW || producer) {
            char *buf = smem + (s % NBUF) * BUF;
            sx.issue(s, buf);
            sy.issue(s, buf + XB);
        }
    }

    // Stages 0 .. NBUF-2 in flight (early issue: 0 .. NBUF-3; begin(0)
    // issues NBUF-2).
    __device__ __forceinline__ void prologue() {
#pragma unroll
        for (int q = 0; q < (kEarly ? NBUF - 2 : NBUF - 1); ++q)
            if (q < S)
                issue(q);
    }

    // Start of stage s: this wave's copies of stage s are complete (those of
    // later stages may stay in flight), then the workgroup joins -- after which
    // all of stage s is in LDS and every wave has consumed stage s - 1, whose
    // buffer is refilled with stage s + NBUF - 1 --, then the fragment reads of
    // stage s are issued.
    //
    // Early issue (NBUF >= 3): the copies of stage s + NBUF - 2 go out before
    // the barrier; their buffer held stage s - 2, which every wave finished
    // reading before the barrier of stage s - 1.
    template <int PAR = -1>
    __device__ __forceinline__ void begin(int s) {
        if constexpr (kEarly) {
            if (s + NBUF - 2 < S) {
                issue(s + NBUF - 2);
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NBUF - 2) * LOADS)
                             : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
        } else {
            if (s + NBUF - 2 < S)
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NBUF - 2) * LOADS)
                             : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (s + NBUF - 1 < S)
                issue(s + NBUF - 1);
        }
        cur = smem + (s % NBUF) * BUF;
        read<0>();
    }

    // Fragment reads of leaf half H of the current stage (the first half is
    // read by begin(), the second just before the first half's MFMAs, which
    // cover its latency; holding only one half through the tree work saves
    // registers).
    template <int H>
    __device__ __forceinline__ void read() {
        const char *buf = cur;
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            if constexpr (XK) {
                fa[H][a] = *reinterpret_cast<const bf16x8 *>(buf + xoff[H] + a * 16 * 128);
            } else {
                const char *q = buf + xoff[a] + H * 32 * BM * 2;
                fa[H][a] = tr_read(q, q + 4 * BM * 2);
            }
        }
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            if constexpr (YK) {
                fb[H][b] = *reinterpret_cast<const bf16x8 *>(buf + yoff[H] + b * 16 * 128);
            } else {
                const char *q = buf + yoff[b] + H * 32 * BN * 2;
                fb[H][b] = tr_read(q, q + 4 * BN * 2);
            }
        }
    }

    __device__ __forceinline__ static bf16x8 tr_read(const char *p0, const char *p1) {
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        return __builtin_bit_cast(bf16x8, v);
    }

    // The two leaves of the current stage, each rounded and packed per block.
    // The second leaf's conversions follow its MFMAs in the same stage (they
    // overlap the MFMAs still in flight), so the next stage opens with the
    // pair's matrix-core add on packed operands rather than with conversions
    // that both waves of a SIMD would run at once.
    __device__ __forceinline__ void leaves(P &x0, P &x1) {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        read<1>();
        F l0, l1;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                l0.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[0][a], fb[0][b], zero, 0, 0, 0);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                l1.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[1][a], fb[1][b], zero, 0, 0, 0);
        x0 = wpack(l0);
        x1 = wpack(l1);
    }

    // Workgroup-wide OR of a flag, through one dword per wave at the end of
    // the stage buffers (the output staging stays below it).  Two barriers:
    // the first also retires every wave's use of the LDS.  (Not the runtime's
    // block reduction, which reserves static LDS and so would shrink the
    // dynamic allocation below the full 160 KB.)
    __device__ __forceinline__ bool any_in_workgroup(bool flag) {
        int *slot = reinterpret_cast<int *>(smem + NBUF * BUF) - NW;
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const bool any = __builtin_amdgcn_ballot_w64(flag) != 0;
        __syncthreads();
        if ((threadIdx.x & 63) == 0)
            slot[w] = any ? 1 : 0;
        __syncthreads();
        int r = 0;
#pragma unroll
        for (int q = 0; q < NW; ++q)
            r |= slot[q];
        return r != 0;
    }

    // Leaf h of the current stage, rounded and packed.  SWAP exchanges the
    // operands of the MFMA: the same products, summed by the same instruction
    // for each output, land transposed -- the layout a matrix-core add
    // produces, so the leaf can meet a sibling one level taller.
    template <int H, bool SWAP>
    __device__ __forceinline__ P leaf() const {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        F l;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                l.v[a][b] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[H][b], fa[H][a], zero, 0, 0, 0)
                                 : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[H][a], fb[H][b], zero, 0, 0, 0);
        return wpack(l);
    }

    // This lane's first slot of parked level `slot`.  The level's offset is
    // made opaque, so that the address is formed where it is used: past the
    // 16-bit offset field (two levels) the compiler would otherwise keep one
    // address register per fragment and level alive through the whole loop,
    // for branches that run once or twice per tile.
    __device__ __forceinline__ char *park_slot(int slot) const {
        int off = slot * PARK_LEVEL;
        asm volatile("" : "+s"(off));
        return park_lane + off;
    }

    __device__ __forceinline__ void park(int slot, const P &v) {
        char *base = park_slot(slot);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                *reinterpret_cast<u32x2 *>(base + (a * FN + b) * PARK_FRAG) = v.w[a][b];
    }

    __device__ __forceinline__ P unpark(int slot) const {
        const char *base = park_slot(slot);
        P v;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                v.w[a][b] = *reinterpret_cast<const u32x2 *>(base + (a * FN + b) * PARK_FRAG);
        return v;
    }
};

// The perfect tree over the S = L / 2 stage pairs.  Level 1 holds the pair
// nodes; a node at level j waits, packed, until its right sibling arrives.
// Levels 1 .. GL belong to a group of G = 2^GL consecutive stages (static
// register slots); the group roots (level GL + 1) climb the `nup` levels above,
// the first RU of them in registers, the rest parked in LDS.
//
// Stage s: fragment reads; the climb of the pair node of stage s - 1; the leaf
// MFMAs of stage s, their rounding and their pair add, whose result is rounded
// and carried (packed) into stage s + 1.  Each phase is kept to itself by a
// scheduling barrier, which bounds the registers a wave holds at any time; the
// other wave of the SIMD overlaps its phases with this one's.
// EPI: the tile also writes the per-token slots of p (grouped launches).
template <class E, class Arith, int TB, int GL, int RU, bool EPI = false>
struct WideTree {
    static constexpr int G = 1 << GL;
    static_assert(TB == 1 || (TB % 2 == 1 && TB <= 255), "units of one leaf or of an odd count");
    static_assert(TB != 7 || GL <= 2, "seven-leaf groups of at most four pairs of units");
    static_assert(TB <= 7 || GL == 0, "generic units: one pair of units per group");
    static_assert(GL >= 1 || TB > 7, "groups of at least two stages");
    // RU >= 1: the zero-leaf step of group 0 writes the first upper slot,
    // which must then be a register (with no upper levels, no LDS slot exists).
    static_assert(RU >= 1, "the first upper level is held in registers");
    typedef typename E::F F;
    typedef typename E::P P;
    E &e;
    const MfmaParams &p;
    const bf16x8 sel;
    const int nup;
    const int i0, j0;
    const bool odd;  // layout parity of the root (matrix-core adds transpose)
    // Pending nodes in registers: levels 1 .. GL of a group (static slots
    // l0 .. l3), then the RU upper levels (u0 .. u3).  Plain members rather than
    // arrays, so that nothing keeps them from living in registers.
    P l0, l1, l2, l3, u0, u1, u2, u3;
    static_assert(GL <= 4 && RU <= 4, "at most four register levels of each kind");

    template <int J>
    __device__ __forceinline__ P &low() {
        if constexpr (J == 0)
            return l0;
        else if constexpr (J == 1)
            return l1;
        else if constexpr (J == 2)
            return l2;
        else
            return l3;
    }
    template <int Q>
    __device__ __forceinline__ P &upreg() {
        if constexpr (Q == 0)
            return u0;
        else if constexpr (Q == 1)
            return u1;
        else if constexpr (Q == 2)
            return u2;
        else
            return u3;
    }

    __device__ __forceinline__ WideTree(E &e_, const MfmaParams &p_, bf16x8 sel_, int i0_, int j0_,
                                        bool odd_)
        : e(e_), p(p_), sel(sel_), nup(p_.levels), i0(i0_), j0(j0_), odd(odd_) {}

    __device__ __forceinline__ void store(const F &root) {
        const int wave = threadIdx.x >> 6;
        store_root<E::kOUT>(p, root, odd, i0, j0, wave % E::kWM, wave / E::kWM, threadIdx.x & 63);
    }

    // An empty statement that takes a value and may change it: the value must
    // be complete at this point, and nothing computing it can move below it.
    __device__ __forceinline__ static void pin_p(P &x) {
#pragma unroll
        for (int a = 0; a < E::kFM; ++a)
#pragma unroll
            for (int b = 0; b < E::kFN; ++b)
                asm volatile("" : "+v"(x.w[a][b]));
    }
    __device__ __forceinline__ static void pin_f(F &x) {
#pragma unroll
        for (int a = 0; a < E::kFM; ++a)
#pragma unroll
            for (int b = 0; b < E::kFN; ++b)
                asm volatile("" : "+v"(x.v[a][b]));
    }

    __device__ __forceinline__ F add(const P &l, const P &r) { return Arith::add(l, r, sel); }

    // The pending node of upper level Q (static slot).
    template <int Q>
    __device__ __forceinline__ P upper(void) {
        if constexpr (Q < RU)
            return upreg<Q>();
        else
            return e.unpark(Q - RU);
    }
    template <int Q>
    __device__ __forceinline__ void set_upper(const P &x) {
        if constexpr (Q < RU) {
            upreg<Q>() = x;
            pin_p(upreg<Q>());
        } else {
            e.park(Q - RU, x);
        }
    }

    // Group root x (packed, level GL + 1) of a group t < T - 1 climbs from
    // upper level Q while it is a right child; t has a clear bit below nup,
    // where the climb stops.  Unrolled by recursion (at most 9 - GL upper levels:
    // L <= 1024), so every slot index is static; the branches are uniform.
    static constexpr int kMaxUp = 9 - GL;
    template <int Q>
    __device__ __forceinline__ void climb_up(const P &x, int t) {
        if constexpr (Q < kMaxUp) {
            if (!((t >> Q) & 1))
                set_upper<Q>(x);
            else
                climb_up<Q + 1>(wpack(add(upper<Q>(), x)), t);
        }
    }

    // Pair node x (packed, level J + 1) of stage U of group t climbs within the
    // group while it is a right child; a group root continues above.
    template <int U, int J>
    __device__ __forceinline__ void climb_low(const P &x, int t) {
        if constexpr (J == GL)
            climb_up<0>(x, t);
        else if constexpr ((U >> J) & 1)
            climb_low<U, J + 1>(wpack(add(low<J>(), x)), t);
        else {
            low<J>() = x;
            pin_p(low<J>());
        }
    }

    // The last stage's pair node: every step is a right child up to the root.
    template <int J>
    __device__ __forceinline__ F final_low(const P &x) {
        const F y = add(low<J>(), x);
        if constexpr (J + 1 < GL)
            return final_low<J + 1>(wpack(y));
        else
            return nup > 0 ? final_up<0>(wpack(y), y) : y;
    }
    __device__ __forceinline__ F final_chain(const P &x1) { return final_low<0>(x1); }
    template <int Q>
    __device__ __forceinline__ F final_up(const P &x, const F &y) {
        if constexpr (Q < kMaxUp) {
            if (Q == nup)
                return y;
            const F z = add(upper<Q>(), x);
            return final_up<Q + 1>(wpack(z), z);
        } else {
            return y;
        }
    }

    // Tree work of stage U of group t, whose leaves are x0 and x1 (rounded,
    // packed): their pair add, rounded, climbs while it is a right child.
    template <int U>
    __device__ __forceinline__ void step(const P &x0, const P &x1, int t) {
        climb_low<U, 0>(wpack(add(x0, x1)), t);
    }

    // Tree work of the last stage, then the root is rounded and stored.
    // Returns whether the root has a non-finite value.
    __device__ __forceinline__ bool finish(const P &x0, const P &x1) {
        return finish_root(final_chain(wpack(add(x0, x1))));
    }

    // With matrix-core adds, a tile whose root has a non-finite value is not
    // stored (true is returned, the caller recomputes it); element-wise adds
    // always store.  The barrier of the check also frees the LDS for staging.
    __device__ __forceinline__ bool finish_root(const F &root) {
        const int wave = threadIdx.x >> 6;
        const auto fp32_nonfinite = [&]() {
            bool nonfinite = false;
            if constexpr (Arith::kTransposes) {
#pragma unroll
                for (int a = 0; a < E::kFM; ++a)
#pragma unroll
                    for (int b = 0; b < E::kFN; ++b)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            nonfinite |= !(__builtin_fabsf(root.v[a][b][v]) <= 3.40282347e38f);
            }
            return nonfinite;
        };
        if constexpr (E::kEarly) {
            // One barrier: the staged tile goes to one free stage buffer, the
            // wave flags to the other (see WideEngine::free_buffer).
            int *flags = reinterpret_cast<int *>(e.free_buffer(1));
            if constexpr (E::kOUT == OUT_F32) {
                if (publish_nonfinite<E::NW>(flags, fp32_nonfinite()))
                    return true;
                store(root);
                return false;
            } else {
                // element-wise adds never need the recomputation
                return store_staged<E::kOUT, E::kFM, E::kFN, E::BM, E::BN, E::NW, EPI, true,
                                    Arith::kTransposes>(
                    p, root, odd, i0, j0, wave % E::kWM, wave / E::kWM, threadIdx.x & 63,
                    e.free_buffer(0), flags);
            }
        } else {
            if (e.any_in_workgroup(fp32_nonfinite()))
                return true;
            if constexpr (E::kOUT == OUT_F32) {
                store(root);
            } else {
                store_staged<E::kOUT, E::kFM, E::kFN, E::BM, E::BN, E::NW, EPI>(
                    p, root, odd, i0, j0, wave % E::kWM, wave / E::kWM, threadIdx.x & 63, e.lds);
            }
            return false;
        }
    }

    // Stage U of group t: the fragment reads of the stage, the tree work of
    // the previous stage (which covers the latency of the reads), then the
    // stage's leaves, which wait across the barrier, packed.
    // `pin` keeps the leaves where they are computed: without it the compiler
    // sinks their MFMAs into the next stage, behind its barrier.
    //
    // The first stage of group t > 0 finishes group t - 1.  Group 0 runs the
    // same code on zero leaves, as group index 0: its only effect is a write
    // of the first upper slot, which group 0's own root overwrites before any
    // read (group 1 reads it); a branch here would split the stage's code.
    template <int U>
    __device__ __forceinline__ void stage(int t, P &x0, P &x1) {
        e.template begin<U & 1>(t * G + U);
        if constexpr (U == 0)
            step<G - 1>(x0, x1, t > 0 ? t - 1 : 0);
        else
            step<U - 1>(x0, x1, t);
        e.leaves(x0, x1);
        pin_p(x0);
        pin_p(x1);
        if constexpr (U + 1 < G)
            stage<U + 1>(t, x0, x1);
    }

    // ---- L = 3 * 2^a.  The mid-split tree is the perfect tree over units of
    // three leaves, u = x0 (+) (x1 (+) x2).  Three stages (leaves a0 a1 | b0 b1
    // | c0 c1) hold two units, a0 (+) (a1 (+) b0) and b1 (+) (c0 (+) c1), whose
    // add is the six-leaf node that climbs (levels counted from it).  With
    // matrix-core adds the single leaves a0 and b1 are computed with swapped
    // operands, so they are laid out like the two-leaf nodes they meet.
    struct Carry {
        P a0, a1, b0, b1, u0, c0, c1, u1;
    };

    // Super-stage U of group t: stages A, B, C.  The tree work of super-stage
    // U - 1 (group t - 1's last one for U = 0, with the zero-leaf convention
    // of the one-leaf schedule) is spread over the stages so that each has
    // adds to cover the latency of its first fragment reads:
    //   A: the second unit u1 = b1 (+) (c0 (+) c1), then leaves a0, a1;
    //   B: the six-leaf node u0 (+) u1 climbs, then leaves b0, b1;
    //   C: the first unit u0 = a0 (+) (a1 (+) b0), then leaves c0, c1.
    template <int U>
    __device__ __forceinline__ void stage3(int t, Carry &c) {
        const int s = 3 * (t * G + U);
        e.template begin<U & 1>(s);
        c.u1 = wpack(add(c.b1, wpack(add(c.c0, c.c1))));
        e.template read<1>();
        c.a0 = e.template leaf<0, Arith::kTransposes>();
        c.a1 = e.template leaf<1, false>();
        pin_p(c.u1);
        pin_p(c.a0);
        pin_p(c.a1);
        e.template begin<(U + 1) & 1>(s + 1);
        if constexpr (U == 0)
            climb_low<G - 1, 0>(wpack(add(c.u0, c.u1)), t > 0 ? t - 1 : 0);
        else
            climb_low<U - 1, 0>(wpack(add(c.u0, c.u1)), t);
        e.template read<1>();
        c.b0 = e.template leaf<0, false>();
        c.b1 = e.template leaf<1, Arith::kTransposes>();
        pin_p(c.b0);
        pin_p(c.b1);
        e.template begin<U & 1>(s + 2);
        c.u0 = wpack(add(c.a0, wpack(add(c.a1, c.b0))));
        e.template read<1>();
        c.c0 = e.template leaf<0, false>();
        c.c1 = e.template leaf<1, false>();
        pin_p(c.u0);
        pin_p(c.c0);
        pin_p(c.c1);
        if constexpr (U + 1 < G)
            stage3<U + 1>(t, c);
    }

    __device__ __forceinline__ bool run3() {
        const int T = e.S / (3 * G);
        e.prologue();
        Carry c;
#pragma unroll
        for (int a = 0; a < E::kFM; ++a)
#pragma unroll
            for (int b = 0; b < E::kFN; ++b) {
                c.a0.w[a][b] = c.a1.w[a][b] = c.b0.w[a][b] = c.b1.w[a][b] = u32x2{0u, 0u};
                c.u0.w[a][b] = c.c0.w[a][b] = c.c1.w[a][b] = c.u1.w[a][b] = u32x2{0u, 0u};
            }
        for (int t = 0; t < T; ++t)
            stage3<0>(t, c);
        const P u1 = wpack(add(c.b1, wpack(add(c.c0, c.c1))));
        return finish_root(final_chain(wpack(add(c.u0, u1))));
    }

    // ---- L = 5 * 2^a.  Units of five leaves, u = (x0 (+) x1) (+) (x2 (+) (x3
    // (+) x4)); five stages (a0 a1 | b0 b1 | c0 c1 | d0 d1 | e0 e1) hold two
    // units, (a0 (+) a1) (+) (b0 (+) (b1 (+) c0)) and (c1 (+) d0) (+) (d1 (+)
    // (e0 (+) e1)).  With matrix-core adds the leaves one level above the
    // deepest (a0 a1 b0, c1 d0 d1) are computed with swapped operands, so both
    // children of every add share a layout.  The tree work of the previous
    // super-stage and of this one's first unit is spread over the stages:
    //   A: u1 = pcd (+) (d1 (+) (e0 (+) e1)), then leaves a0, a1;
    //   B: the ten-leaf node u0 (+) u1 climbs, then leaves b0, b1;
    //   C: p01 = a0 (+) a1, then leaves c0, c1;
    //   D: u0 = p01 (+) (b0 (+) (b1 (+) c0)), then leaves d0, d1;
    //   E: pcd = c1 (+) d0, then leaves e0, e1.
    struct Carry5 {
        P a0, a1, b0, b1, c0, c1, d0, d1, e0, e1, p01, u0, u1, pcd;
    };

    template <int U>
    __device__ __forceinline__ void stage5(int t, Carry5 &c) {
        constexpr bool T = Arith::kTransposes;
        const int s = 5 * (t * G + U);
        e.template begin<U & 1>(s);
        c.u1 = wpack(add(c.pcd, wpack(add(c.d1, wpack(add(c.e0, c.e1))))));
        e.template read<1>();
        c.a0 = e.template leaf<0, T>();
        c.a1 = e.template leaf<1, T>();
        pin_p(c.u1);
        pin_p(c.a0);
        pin_p(c.a1);
        e.template begin<(U + 1) & 1>(s + 1);
        if constexpr (U == 0)
            climb_low<G - 1, 0>(wpack(add(c.u0, c.u1)), t > 0 ? t - 1 : 0);
        else
            climb_low<U - 1, 0>(wpack(add(c.u0, c.u1)), t);
        e.template read<1>();
        c.b0 = e.template leaf<0, T>();
        c.b1 = e.template leaf<1, false>();
        pin_p(c.b0);
        pin_p(c.b1);
        e.template begin<U & 1>(s + 2);
        c.p01 = wpack(add(c.a0, c.a1));
        e.template read<1>();
        c.c0 = e.template leaf<0, false>();
        c.c1 = e.template leaf<1, T>();
        pin_p(c.p01);
        pin_p(c.c0);
        pin_p(c.c1);
        e.template begin<(U + 1) & 1>(s + 3);
        c.u0 = wpack(add(c.p01, wpack(add(c.b0, wpack(add(c.b1, c.c0))))));
        e.template read<1>();
        c.d0 = e.template leaf<0, T>();
        c.d1 = e.template leaf<1, T>();
        pin_p(c.u0);
        pin_p(c.d0);
        pin_p(c.d1);
        e.template begin<U & 1>(s + 4);
        c.pcd = wpack(add(c.c1, c.d0));
        e.template read<1>();
        c.e0 = e.template leaf<0, false>();
        c.e1 = e.template leaf<1, false>();
        pin_p(c.pcd);
        pin_p(c.e0);
        pin_p(c.e1);
        if constexpr (U + 1 < G)
            stage5<U + 1>(t, c);
    }

    __device__ __forceinline__ bool run5() {
        const int T = e.S / (5 * G);
        e.prologue();
        Carry5 c;
        zero_p(c.a0, c.a1, c.b0, c.b1, c.c0, c.c1, c.d0);
        zero_p(c.d1, c.e0, c.e1, c.p01, c.u0, c.u1, c.pcd);
        for (int t = 0; t < T; ++t)
            stage5<0>(t, c);
        const P u1 = wpack(add(c.pcd, wpack(add(c.d1, wpack(add(c.e0, c.e1))))));
        return finish_root(final_chain(wpack(add(c.u0, u1))));
    }

    // ---- L = 7 * 2^a.  Units of seven leaves, u = (x0 (+) (x1 (+) x2)) (+)
    // ((x3 (+) x4) (+) (x5 (+) x6)); seven stages (a0 a1 | ... | g0 g1) hold
    // two units, (a0 (+) (a1 (+) b0)) (+) ((b1 (+) c0) (+) (c1 (+) d0)) and
    // (d1 (+) (e0 (+) e1)) (+) ((f0 (+) f1) (+) (g0 (+) g1)); with matrix-core
    // adds a0 and d1 (one level above the deepest) use swapped operands.
    //   A: u1 = n (+) (o (+) (g0 (+) g1)), then leaves a0, a1;
    //   B: the fourteen-leaf node u0 (+) u1 climbs, then leaves b0, b1;
    //   C: y = a0 (+) (a1 (+) b0), then leaves c0, c1;
    //   D: z = b1 (+) c0, then leaves d0, d1;
    //   E: u0 = y (+) (z (+) (c1 (+) d0)), then leaves e0, e1;
    //   F: n = d1 (+) (e0 (+) e1), then leaves f0, f1;
    //   G: o = f0 (+) f1, then leaves g0, g1.
    // A group is four pairs of units at most (GL <= 2): the recomputation with
    // element-wise adds is a called function, and at eight pairs its code
    // outgrew the range of a short branch; the compiler's long branches then
    // reused the registers of the return address, and the call never returned.
    struct Carry7 {
        P a0, a1, b0, b1, c0, c1, d0, d1, e0, e1, f0, f1, g0, g1, y, z, u0, u1, n, o;
    };
    template <int U>
    __device__ __forceinline__ void stage7(int t, Carry7 &c) {
        constexpr bool T = Arith::kTransposes;
        const int s = 7 * (t * G + U);
        e.template begin<U & 1>(s);
        c.u1 = wpack(add(c.n, wpack(add(c.o, wpack(add(c.g0, c.g1))))));
        e.template read<1>();
        c.a0 = e.template leaf<0, T>();
        c.a1 = e.template leaf<1, false>();
        pin_p(c.u1);
        pin_p(c.a0);
        pin_p(c.a1);
        e.template begin<(U + 1) & 1>(s + 1);
        if constexpr (U == 0)
            climb_low<G - 1, 0>(wpack(add(c.u0, c.u1)), t > 0 ? t - 1 : 0);
        else
            climb_low<U - 1, 0>(wpack(add(c.u0, c.u1)), t);
        e.template read<1>();
        c.b0 = e.template leaf<0, false>();
        c.b1 = e.template leaf<1, false>();
        pin_p(c.b0);
        pin_p(c.b1);
        e.template begin<U & 1>(s + 2);
        c.y = wpack(add(c.a0, wpack(add(c.a1, c.b0))));
        e.template read<1>();
        c.c0 = e.template leaf<0, false>();
        c.c1 = e.template leaf<1, false>();
        pin_p(c.y);
        pin_p(c.c0);
        pin_p(c.c1);
        e.template begin<(U + 1) & 1>(s + 3);
        c.z = wpack(add(c.b1, c.c0));
        e.template read<1>();
        c.d0 = e.template leaf<0, false>();
        c.d1 = e.template leaf<1, T>();
        pin_p(c.z);
        pin_p(c.d0);
        pin_p(c.d1);
        e.template begin<U & 1>(s + 4);
        c.u0 = wpack(add(c.y, wpack(add(c.z, wpack(add(c.c1, c.d0))))));
        e.template read<1>();
        c.e0 = e.template leaf<0, false>();
        c.e1 = e.template leaf<1, false>();
        pin_p(c.u0);
        pin_p(c.e0);
        pin_p(c.e1);
        e.template begin<(U + 1) & 1>(s + 5);
        c.n = wpack(add(c.d1, wpack(add(c.e0, c.e1))));
        e.template read<1>();
        c.f0 = e.template leaf<0, false>();
        c.f1 = e.template leaf<1, false>();
        pin_p(c.n);
        pin_p(c.f0);
        pin_p(c.f1);
        e.template begin<U & 1>(s + 6);
        c.o = wpack(add(c.f0, c.f1));
        e.template read<1>();
        c.g0 = e.template leaf<0, false>();
        c.g1 = e.template leaf<1, false>();
        pin_p(c.o);
        pin_p(c.g0);
        pin_p(c.g1);
        if constexpr (U + 1 < G)
            stage7<U + 1>(t, c);
    }
    __device__ __forceinline__ bool run7() {
        const int T = e.S / (7 * G);
        e.prologue();
        Carry7 c;
        zero_p(c.a0, c.a1, c.b0, c.b1, c.c0, c.c1, c.d0, c.d1, c.e0, c.e1);
        zero_p(c.f0, c.f1, c.g0, c.g1, c.y, c.z, c.u0, c.u1, c.n, c.o);
        for (int t = 0; t < T; ++t)
            stage7<0>(t, c);
        const P u1 = wpack(add(c.n, wpack(add(c.o, wpack(add(c.g0, c.g1))))));
        return finish_root(final_chain(wpack(add(c.u0, u1))));
    }

    // ---- L = m * 2^a for another odd m (TB = m; 43 for K = 11008, 27 for
    // K = 13824), one pair of units per group (GL = 0: the recomputation with
    // element-wise adds is a called function, whose code must stay within
    // the range of a short branch).  The mid-split tree over the m leaves of a unit is walked in
    // post-order with its pending left siblings on a stack of static register
    // slots: the tree is fixed by m, so where each leaf stands (its depth,
    // the adds that follow it, the stack height before it) is computed at
    // compile time.  m stages hold two units (leaves j = 0 .. 2m - 1 of the
    // pair: unit j / m, leaf j % m).  A leaf at depth d of a unit of height h
    // is computed with swapped operands when h - d is odd (matrix-core adds),
    // so both children of every add share a layout.  Stage k of a pair opens
    // with the tree work of the previous stage's two leaves (for k = 0: the
    // previous pair's last two, which close its second unit, whose node with
    // the first climbs), then computes its own two leaves.
    static constexpr int unit_depth(int t) {
        int lo = 0, hi = TB, d = 0;
        while (hi - lo > 1) {
            const int mid = lo + (hi - lo) / 2;
            if (t < mid)
                hi = mid;
            else
                lo = mid;
            ++d;
        }
        return d;
    }
    static constexpr int unit_merges(int t) {   // inner nodes whose range ends at t + 1
        int lo = 0, hi = TB, m = 0;
        while (hi - lo > 1) {
            if (hi == t + 1)
                ++m;
            const int mid = lo + (hi - lo) / 2;
            if (t < mid)
                hi = mid;
            else
                lo = mid;
        }
        return m;
    }
    static constexpr int unit_height() {
        int h = 0;
        for (int t = 0; t < TB; ++t)
            h = unit_depth(t) > h ? unit_depth(t) : h;
        return h;
    }
    static constexpr int unit_sp(int t) {   // pending nodes before leaf t
        int sp = 0;
        for (int q = 0; q < t; ++q)
            sp += 1 - unit_merges(q);
        return sp;
    }
    static constexpr bool unit_swap(int t) {
        return Arith::kTransposes && ((unit_height() - unit_depth(t)) & 1) != 0;
    }
    struct CarryU {
        P cur0, cur1, r0, st0, st1, st2, st3, st4, st5, st6, st7;
    };
    template <int D>
    __device__ __forceinline__ static P &slot(CarryU &c) {
        static_assert(D >= 0 && D < 8, "unit stacks of at most eight pending nodes");
        if constexpr (D == 0) return c.st0;
        else if constexpr (D == 1) return c.st1;
        else if constexpr (D == 2) return c.st2;
        else if constexpr (D == 3) return c.st3;
        else if constexpr (D == 4) return c.st4;
        else if constexpr (D == 5) return c.st5;
        else if constexpr (D == 6) return c.st6;
        else return c.st7;
    }
    // The adds that follow leaf t: the I-th pops the pending node at height
    // SP - 1 - I (its left sibling at that moment).
    template <int SP, int I, int NM>
    __device__ __forceinline__ P unit_pops(CarryU &c, const P &x) {
        if constexpr (I == NM)
            return x;
        else
            return unit_pops<SP, I + 1, NM>(c, wpack(add(slot<SP - 1 - I>(c), x)));
    }
    // Leaf j of a pair (packed, in its layout): its adds, then it waits on the
    // stack, or it is a unit's root (the first unit's in r0, the second's left
    // in x).
    template <int J>
    __device__ __forceinline__ void unit_leaf(CarryU &c, P &x) {
        constexpr int t = J % TB;
        constexpr int sp = unit_sp(t), nm = unit_merges(t);
        const P y = unit_pops<sp, 0, nm>(c, x);
        if constexpr (t + 1 < TB) {
            slot<sp - nm>(c) = y;
            pin_p(slot<sp - nm>(c));
        } else if constexpr (J < TB) {
            c.r0 = y;
            pin_p(c.r0);
        } else {
            x = y;
        }
    }
    template <int U, int K>
    __device__ __forceinline__ void stageU(int t, CarryU &c) {
        const int s = TB * (t * G + U) + K;
        e.template begin<K & 1>(s);
        if constexpr (K == 0) {
            unit_leaf<2 * TB - 2>(c, c.cur0);
            P r1 = c.cur1;
            unit_leaf<2 * TB - 1>(c, r1);
            if constexpr (U == 0)
                climb_low<G - 1, 0>(wpack(add(c.r0, r1)), t > 0 ? t - 1 : 0);
            else
                climb_low<U - 1, 0>(wpack(add(c.r0, r1)), t);
        } else {
            unit_leaf<2 * K - 2>(c, c.cur0);
            unit_leaf<2 * K - 1>(c, c.cur1);
        }
        e.template read<1>();
        c.cur0 = e.template leaf<0, unit_swap((2 * K) % TB)>();
        c.cur1 = e.template leaf<1, unit_swap((2 * K + 1) % TB)>();
        pin_p(c.cur0);
        pin_p(c.cur1);
        if constexpr (K + 1 < TB)
            stageU<U, K + 1>(t, c);
        else if constexpr (U + 1 < G)
            stageU<U + 1, 0>(t, c);
    }
    __device__ __forceinline__ bool runU() {
        const int T = e.S / (TB * G);
        e.prologue();
        CarryU c;
        zero_p(c.cur0, c.cur1, c.r0, c.st0, c.st1, c.st2, c.st3, c.st4, c.st5, c.st6, c.st7);
        for (int t = 0; t < T; ++t)
            stageU<0, 0>(t, c);
        unit_leaf<2 * TB - 2>(c, c.cur0);
        P r1 = c.cur1;
        unit_leaf<2 * TB - 1>(c, r1);
        // one pair per group: the pair's node is the group root, which climbs
        // as a right child up to the root
        const F y = add(c.r0, r1);
        return finish_root(nup > 0 ? final_up<0>(wpack(y), y) : y);
    }

    template <class... Ps>
    __device__ __forceinline__ static void zero_p(Ps &...xs) {
        (zero_one(xs), ...);
    }
    __device__ __forceinline__ static void zero_one(P &x) {
#pragma unroll
        for (int a = 0; a < E::kFM; ++a)
#pragma unroll
            for (int b = 0; b < E::kFN; ++b)
                x.w[a][b] = u32x2{0u, 0u};
    }

    // Requires S = e.S = G * 2^nup (units of one leaf).  Computes the root
    // (unrounded fp32, in the layout of its parity) without storing it.
    __device__ __forceinline__ F run_root() {
        static_assert(TB == 1, "units of one leaf");
        const int T = e.S >> GL;
        e.prologue();
        P x0;
        P x1;
#pragma unroll
        for (int a = 0; a < E::kFM; ++a)
#pragma unroll
            for (int b = 0; b < E::kFN; ++b) {
                x0.w[a][b] = u32x2{0u, 0u};
                x1.w[a][b] = u32x2{0u, 0u};
            }
        for (int t = 0; t < T; ++t)
            stage<0>(t, x0, x1);
        return final_chain(wpack(add(x0, x1)));
    }

    // Requires S = e.S = TB * G * 2^nup.  Computes and stores the tile;
    // returns whether a root was non-finite.
    __device__ __forceinline__ bool run() {
        if constexpr (TB == 3)
            return run3();
        else if constexpr (TB == 5)
            return run5();
        else if constexpr (TB == 7)
            return run7();
        else if constexpr (TB > 7)
            return runU();
        else
            return finish_root(run_root());
    }
};


// Recomputes a tile with element-wise adds (exact IEEE behaviour for non-finite
// values; positions never move) and stores it.  Kept out of line so that its
// registers do not weigh on the main kernel's allocation: it runs only for
// tiles whose matrix-core tree produced a non-finite root.  Arguments of a
// called function arrive in vector registers, so the workgroup-uniform values
// are made scalar again for the staging code.
template <bool XK, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int TB, int GL,
          int RU, bool EPI>
__device__ __attribute__((noinline)) void wide_valu_tile(MfmaParams q, int tile_arg) {
    typedef WideEngine<XK, YK, OUT, FM, FN, WM, WN, NBUF> E;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    MfmaParams p = q;
    p.x = uniform_ptr(q.x);
    p.y = uniform_ptr(q.y);
    p.c = uniform_ptr(q.c);
    p.ldx = uniform64(q.ldx);
    p.ldy = uniform64(q.ldy);
    p.ldc = uniform64(q.ldc);
    p.I = __builtin_amdgcn_readfirstlane(q.I);
    p.J = __builtin_amdgcn_readfirstlane(q.J);
    p.R = __builtin_amdgcn_readfirstlane(q.R);
    p.L = __builtin_amdgcn_readfirstlane(q.L);
    p.tiles_j = __builtin_amdgcn_readfirstlane(q.tiles_j);
    p.levels = __builtin_amdgcn_readfirstlane(q.levels);
    const int tile = __builtin_amdgcn_readfirstlane(tile_arg);
    const int i0 = (tile / p.tiles_j) * E::BM;
    const int j0 = (tile % p.tiles_j) * E::BN;
    E e(p, EPI ? smem + kEpiLds : smem, p.levels > RU ? p.levels - RU : 0, i0, j0);
    WideTree<E, WideValuAdd, TB, GL, RU, EPI> valu(e, p, split_selector(threadIdx.x & 63), i0, j0,
                                                   false);
    valu.run();
}

// OCC: waves per SIMD the register allocation must allow (a 4-wave workgroup
// asks for 2 so that two workgroups share a compute unit).
// One output tile (tile index `tile` of the row-major tile grid of p).
template <bool XK, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int TB, int GL,
          int RU, bool EPI>
__device__ __forceinline__ void wide_tile(const MfmaParams &p, int tile) {
    typedef WideEngine<XK, YK, OUT, FM, FN, WM, WN, NBUF> E;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int i0 = (tile / p.tiles_j) * E::BM;
    const int j0 = (tile % p.tiles_j) * E::BN;

    E e(p, EPI ? smem + kEpiLds : smem, p.levels > RU ? p.levels - RU : 0, i0, j0);
    WideTree<E, WideMatrixAdd, TB, GL, RU, EPI> tree(e, p, split_selector(lane), i0, j0,
                                                 (tree_height_rt(p.L) & 1) != 0);
    // A non-finite root may have spilled NaN into the other sums of its
    // matrix-core add rows: such a tile is not stored but recomputed with
    // element-wise adds.
    if (tree.run())
        wide_valu_tile<XK, YK, OUT, FM, FN, WM, WN, NBUF, TB, GL, RU, EPI>(p, tile);
}

template <bool XK, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int TB, int GL,
          int RU, int OCC>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void mfma_wide_kernel(MfmaParams p) {
    // Tile order: columns in groups of four, the rows of a group's columns
    // before the next group, so the workgroups running at once share a few
    // Y panels (one HBM read of Y) and X stays in the caches.  Row by row, a
    // Y beyond the 256 MB Infinity Cache was read again for every row of
    // tiles (LM head, M = 4096, N = 151936: 530 TFLOP/s against 670).
    constexpr int G = 4;
    const int ti = gridDim.x / p.tiles_j;   // the grid is ti x tiles_j tiles
    const int g = blockIdx.x / (G * ti), u = blockIdx.x % (G * ti);
    const int tile = (u % ti) * p.tiles_j + g * G + u / ti;
    wide_tile<XK, YK, OUT, FM, FN, WM, WN, NBUF, TB, GL, RU, false>(p, tile);
}

// ---- K-split tiles (X K-major, bf16 or fp32 output, L a power of two): the
// workgroup holds KS = 2 or 4 wave groups of WM x WN waves, each with its own
// engine and stage buffers.  For L = 2^a the mid-split tree's nodes of depth
// log2 KS are the KS equal quarters (halves) of the leaves: group g evaluates
// the subtree over leaves g L/KS .. (g+1) L/KS - 1, which divides the chain
// of stages a tile waits for by KS.  The subtree roots meet in LDS and group 0
// performs the adds of the top log2 KS levels ((0 + 1) for KS = 2,
// (0 + 1) + (2 + 3) for KS = 4), then rounds and stores the tile.  All groups
// run the same number of stages, so every workgroup barrier is reached by all
// waves.  With matrix-core adds, a tile with a non-finite root returns true
// (not stored).  The tile's origin is (i0, j0); `lds` is the start of the
// groups' LDS.  EPI (grouped launches, bf16 out): group 0 also writes the
// per-token slots of the tile (store_staged), group 1 meets its barrier.
template <class Arith, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int GL, int RU,
          int KS, bool EPI = false>
__device__ __forceinline__ bool split_tile_at(const MfmaParams &p, int i0, int j0, char *lds) {
    typedef WideEngine<true, YK, OUT, FM, FN, WM, WN, NBUF> E;
    typedef typename E::P P;
    typedef typename E::F F;
    constexpr int NW = E::NW;
    static_assert(KS == 2 || KS == 4, "two or four wave groups");
    static_assert(OUT == OUT_BF16 || OUT == OUT_F32, "row-major output");
    static_assert(!EPI || (OUT == OUT_BF16 && KS == 2), "slots: bf16 tiles on two wave groups");
    char *const smem = lds;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = wave / NW, lw = wave % NW;
    const int wm = lw % WM, wn = lw / WM;
    const int parked = p.levels > RU ? p.levels - RU : 0;
    const int group_bytes = E::lds_bytes(parked);

    // this group's part of the reduction
    MfmaParams q = p;
    const int part = p.R / KS;
    q.R = part;
    q.L = p.L / KS;
    q.x = p.x + g * part;
    q.y = YK ? p.y + g * part : p.y + (int64_t)(g * part) * p.ldy;
    E e(q, smem + g * group_bytes, parked, i0, j0, g * 64 * NW);
    const bf16x8 sel = split_selector(lane);
    WideTree<E, Arith, 1, GL, RU, false> tree(e, q, sel, i0, j0, false);
    const P mine = wpack(tree.run_root());

    // Every wave is past its last stage (its copies and reads are complete):
    // groups 1 .. KS-1 hand their roots, rounded and packed, to group 0, each
    // through the start of its own LDS region.
    __syncthreads();
    const int slot = lw * 64 + lane;
    if (g > 0) {
        u32x2 *x = reinterpret_cast<u32x2 *>(smem + g * group_bytes) + slot;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                x[(a * FN + b) * NW * 64] = mine.w[a][b];
    }
    __syncthreads();
    auto root_of = [&](int h) {
        const u32x2 *x = reinterpret_cast<const u32x2 *>(smem + h * group_bytes) + slot;
        P r;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                r.w[a][b] = x[(a * FN + b) * NW * 64];
        return r;
    };

    // the top levels, left child first; the root's layout parity is that of
    // the whole tree's height
    const bool odd = Arith::kTransposes && (tree_height_rt(p.L) & 1) != 0;
    F root;
    bool nonfinite = false;
    char *staged = smem + parked * E::PARK_LEVEL;           // group 0's first stage buffer
    int *flags = reinterpret_cast<int *>(staged + E::BUF);  // its second
    if constexpr (EPI) {
        // staging, slots and store by group 0 (store_staged over its NW
        // waves); group 1 takes part in the one barrier, whose flags are
        // group 0's
        if (g == 0) {
            const F r = Arith::add(mine, root_of(1), sel);
            return store_staged<OUT, FM, FN, E::BM, E::BN, NW, true, true, Arith::kTransposes>(
                p, r, odd, i0, j0, wm, wn, lane, staged, flags);
        }
        if constexpr (Arith::kTransposes) {
            return publish_nonfinite<NW>(flags, false);
        } else {
            __syncthreads();
            return false;
        }
    }
    if (g == 0) {
        if constexpr (KS == 2) {
            root = Arith::add(mine, root_of(1), sel);
        } else {
            const P left = wpack(Arith::add(mine, root_of(1), sel));
            const P right = wpack(Arith::add(root_of(2), root_of(3), sel));
            root = Arith::add(left, right, sel);
        }
        if constexpr (OUT == OUT_F32) {
            if constexpr (Arith::kTransposes) {
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int b = 0; b < FN; ++b)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            nonfinite |= !(__builtin_fabsf(root.v[a][b][v]) <= 3.40282347e38f);
            }
        } else {
            nonfinite = odd ? stage_roots<false, true, FM, FN, E::BN, true>(root, wm, wn, lane, staged)
                            : stage_roots<false, false, FM, FN, E::BN, true>(root, wm, wn, lane, staged);
        }
    }
    if constexpr (Arith::kTransposes) {
        if (publish_nonfinite<KS * NW>(flags, nonfinite))
            return true;
    } else {
        __syncthreads();
    }
    if (g == 0) {
        if constexpr (OUT == OUT_F32)
            store_root<OUT>(p, root, odd, i0, j0, wm, wn, lane);
        else
            read_out_staged<E::BM, E::BN, NW, true>(p, staged, i0, j0, p.I - i0, p.J - j0, threadIdx.x);
    }
    return false;
}

template <class Arith, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int GL, int RU,
          int KS>
__device__ __forceinline__ bool split_tile(const MfmaParams &p, int tile) {
    typedef WideEngine<true, YK, OUT, FM, FN, WM, WN, NBUF> E;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    return split_tile_at<Arith, YK, OUT, FM, FN, WM, WN, NBUF, GL, RU, KS>(
        p, (tile / p.tiles_j) * E::BM, (tile % p.tiles_j) * E::BN, smem);
}

// The same tile with element-wise adds, for tiles whose matrix-core root was
// not finite (kept out of line, as wide_valu_tile).
template <bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int GL, int RU, int KS>
__device__ __attribute__((noinline)) void split_valu_tile(MfmaParams q, int tile_arg) {
    MfmaParams p = q;
    p.x = uniform_ptr(q.x);
    p.y = uniform_ptr(q.y);
    p.c = uniform_ptr(q.c);
    p.ldx = uniform64(q.ldx);
    p.ldy = uniform64(q.ldy);
    p.ldc = uniform64(q.ldc);
    p.I = __builtin_amdgcn_readfirstlane(q.I);
    p.J = __builtin_amdgcn_readfirstlane(q.J);
    p.R = __builtin_amdgcn_readfirstlane(q.R);
    p.L = __builtin_amdgcn_readfirstlane(q.L);
    p.tiles_j = __builtin_amdgcn_readfirstlane(q.tiles_j);
    p.levels = __builtin_amdgcn_readfirstlane(q.levels);
    p.cvec = __builtin_amdgcn_readfirstlane(q.cvec);
    split_tile<WideValuAdd, YK, OUT, FM, FN, WM, WN, NBUF, GL, RU, KS>(p, __builtin_amdgcn_readfirstlane(tile_arg));
}

// p.levels: the levels above the groups of stages of one wave group's subtree.
template <bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int GL, int RU, int KS, int OCC>
__global__ __launch_bounds__(64 * KS * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void mfma_wide_split_kernel(MfmaParams p) {
    // An MN-major Y ([R][J]) of 32-column tiles gives each tile half of every
    // 128-byte line of its panel: tiles 2u and 2u + 1 go to workgroups b and
    // b + 8 of a run of 16, which land on the same XCD (workgroup b runs on
    // XCD b mod 8), so the second half of each line is an L2 hit.  Workgroups
    // past the last whole run keep their own index.
    int tile = blockIdx.x;
    if (!YK && blockIdx.x < (gridDim.x & ~15u)) {
        const int b = blockIdx.x;
        tile = (b & ~15) + 2 * (b & 7) + ((b >> 3) & 1);
    }
    if (split_tile<WideMatrixAdd, YK, OUT, FM, FN, WM, WN, NBUF, GL, RU, KS>(p, tile))
        split_valu_tile<YK, OUT, FM, FN, WM, WN, NBUF, GL, RU, KS>(p, tile);
}

// ---- grouped launch (MoE grouped GEMM): the row-major X is cut into
// consecutive row groups, group e multiplied by its own Y operand
// y + e * y_stride; one launch covers the tiles of every group, group e owning
// tiles tile_start[e] .. tile_start[e+1]-1.  The same tile code runs on the
// group's rows, so each row gets the bits of an ungrouped product.
//
// Half-height tiles (tail balancing, tiles of 128 x 128 in units of one leaf):
// 64 x 128, four 64 x 32 waves per wave group, two wave groups splitting the
// tree at its root, each over half the stages, so a half takes about half a
// tile's time.  A half holds whole 128-column slot rows, so group 0 writes the
// slots as a whole tile does.
template <int GL, int RU>
__device__ __attribute__((noinline)) void grouped_half_valu(MfmaParams q, int i0, int j0) {
    extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
    MfmaParams p = q;
    p.x = uniform_ptr(q.x);
    p.y = uniform_ptr(q.y);
    p.c = uniform_ptr(q.c);
    p.ldx = uniform64(q.ldx);
    p.ldy = uniform64(q.ldy);
    p.ldc = uniform64(q.ldc);
    p.I = __builtin_amdgcn_readfirstlane(q.I);
    p.J = __builtin_amdgcn_readfirstlane(q.J);
    p.R = __builtin_amdgcn_readfirstlane(q.R);
    p.L = __builtin_amdgcn_readfirstlane(q.L);
    p.tiles_j = __builtin_amdgcn_readfirstlane(q.tiles_j);
    p.levels = __builtin_amdgcn_readfirstlane(q.levels);
    p.cvec = __builtin_amdgcn_readfirstlane(q.cvec);
    split_tile_at<WideValuAdd, false, OUT_BF16, 4, 2, 1, 4, 3, GL, RU, 2, true>(
        p, __builtin_amdgcn_readfirstlane(i0), __builtin_amdgcn_readfirstlane(j0), dyn_lds + kEpiLds);
}

template <int GL, int RU>
__device__ __forceinline__ void grouped_half_tile(MfmaParams q, int idx, int h, int levels) {
    extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
    const int i0 = (idx / q.tiles_j) * 128 + h * 64;
    const int j0 = (idx % q.tiles_j) * 128;
    if (i0 >= q.I)
        return;  // the lower half of a group's last row tile may hold no rows
    q.levels = levels;
    if (split_tile_at<WideMatrixAdd, false, OUT_BF16, 4, 2, 1, 4, 3, GL, RU, 2, true>(
            q, i0, j0, dyn_lds + kEpiLds))
        grouped_half_valu<GL, RU>(q, i0, j0);
}

template <int FM, int FN, int WM, int WN, int NBUF, int TB, int GL, int RU, int OCC>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void mfma_wide_grouped_kernel(MfmaParams p, GroupTable g) {
    const int b = blockIdx.x;
    const bool half = b >= g.split_from;
    const int t = half ? g.split_from + ((b - g.split_from) >> 1) : b;
    int lo = 0, hi = g.groups;  // the last group whose first tile is <= t
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (g.tile_start[mid] <= t)
            lo = mid;
        else
            hi = mid;
    }
    MfmaParams q = p;
    const int r0 = g.row_start[lo];
    q.x = p.x + (int64_t)r0 * p.ldx;
    q.y = p.y + (int64_t)lo * g.y_stride;
    q.c = static_cast<uint16_t *>(p.c) + (int64_t)r0 * p.ldc;
    q.I = g.rows[lo];
    if (threadIdx.x == 0) {  // visible to all waves after the first stage barrier
        extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
        EpiInfo *info = reinterpret_cast<EpiInfo *>(dyn_lds);
        info->g = g.g;
        info->slots = g.slots;
        info->ldg = g.ldg;
        info->slot_ld = g.slot_ld;
        info->r0 = r0;
    }
    if constexpr (TB == 1) {
        static_assert(FM * WM == 8 && FN * WN == 8 && WM * WN == 8, "halves of 128 x 128 tiles");
        if (half) {
            grouped_half_tile<GL, RU>(q, t - g.tile_start[lo], (b - g.split_from) & 1, g.split_levels);
            return;
        }
    }
    wide_tile<true, false, OUT_BF16, FM, FN, WM, WN, NBUF, TB, GL, RU, true>(q, t - g.tile_start[lo]);
}

}  // namespace detgemm
