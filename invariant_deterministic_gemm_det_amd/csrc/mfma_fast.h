// Fast path of the MFMA det_gemm kernel (same leaves, same tree, same bits as
// mfma_kernel.h), used when both operands are 16-byte aligned, the reduction
// length is a multiple of 64 and the leaf count is b * 2^a with b in {1, 3}.
//
// Differences from the general kernel, all in the data movement:
//   * operands go from global memory straight into LDS with
//     buffer_load_dwordx4 ... lds (each lane writes 16 bytes at M0 + 16*lane),
//     three stage buffers, loads issued two stages ahead, and no vector
//     registers or ds_write instructions carry them;
//   * the tree adds run one stage late (PipeTree below), between the fragment
//     reads and the leaf MFMAs of the next stage;
//   * a K-major operand tile is stored [row][64 reduction indices] with its
//     16-byte chunks XOR-swizzled by (row >> 1) & 7 and read with one
//     ds_read_b128 per MFMA fragment, as in the general kernel;
//   * an MN-major operand tile is stored in its natural layout [reduction
//     index][rows] (16-byte chunks XOR-swizzled per reduction index) and read
//     with two ds_read_b64_tr_b16 per fragment: in each 16-lane group, lane
//     4m + q addresses reduction index k0 + m, rows 4q .. 4q+3, and lane i of
//     the group receives rows i at indices k0 .. k0+3 -- half of the MFMA
//     operand of lane i;
//   * no per-chunk branches: rows past the end of an operand are clamped in
//     the precomputed source offsets.
#pragma once

#include "mfma_kernel.h"

namespace detgemm {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// XOR applied to the 16-byte chunk index of an MN-major tile row (one
// reduction index).  NC = chunks per row: 4 (64-byte rows, four rows per LDS
// bank sweep), 8 (128-byte rows, two rows per sweep) or 16 (256-byte rows).
// One transposed fragment read touches, per 32 lanes, the reduction rows
// r0 + {0..3, 8..11} (r0 a multiple of 4), each at the same aligned pair of
// chunks; the XOR (always even, so pairs stay pairs) sends those rows to
// disjoint banks.  With 64-byte rows, rows r0 .. r0+3 already fill one sweep
// with their pairs in disjoint banks, and rows r0+8 .. r0+11 take the other
// pair of each row.
template <int NC>
__device__ __forceinline__ int mn_key(int r) {
    if constexpr (NC >= 16)
        return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
    else if constexpr (NC == 8)
        return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
    else
        return 2 * ((r >> 3) & 1);
}

template <bool KMAJOR, int NR, int NW>
struct DirectStager {
    static constexpr int BYTES = NR * 128;   // one stage (64 reduction indices) of the tile
    static constexpr int INSTR = BYTES / 1024;
    static_assert(INSTR % NW == 0, "load instructions must split evenly over the waves");
    static constexpr int PER_WAVE = INSTR / NW;
    static constexpr int NC = NR / 8;        // 16-byte chunks per reduction row (MN-major)

    const uint16_t *tile_base;
    int64_t ld;
    int voff[PER_WAVE];
    int seg[PER_WAVE];  // LDS byte offset of the 1 KB segment this wave writes

    __device__ __forceinline__ void init(const uint16_t *base, int64_t ld_, int row0, int rows,
                                         int wave, int lane) {
        ld = ld_;
        tile_base = KMAJOR ? base + (int64_t)row0 * ld_ : base + row0;
        const int rows_left = rows - row0;
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int ins = q * NW + wave;
            seg[q] = ins * 1024;
            if (KMAJOR) {
                const int row = ins * 8 + (lane >> 3);
                const int lc = (lane & 7) ^ lds_key(row);
                const int rr = row < rows_left ? row : rows_left - 1;
                voff[q] = (int)((int64_t)rr * ld_ * 2) + lc * 16;
            } else {
                constexpr int RPI = 1024 / (NR * 2);  // reduction rows per instruction
                const int r = ins * RPI + lane / NC;
                const int lc = (lane % NC) ^ mn_key<NC>(r);
                int first = 8 * lc;                     // first operand row of the chunk
                if (first >= rows_left)
                    first = ((rows_left - 1) / 8) * 8;  // rows are a multiple of 8 here
                voff[q] = (int)((int64_t)r * ld_ * 2) + first * 2;
            }
        }
    }

    // Loads of stage s into the operand region `dst` (LDS byte pointer).  The
    // instruction is written out so that the compiler, which cannot tell these
    // LDS writes from the fragment reads of other buffers, does not wait for
    // them before every LDS read; the kernel waits for them itself.  An LDS DMA
    // that reads M0 needs one wait state after the scalar write of M0.
    __device__ __forceinline__ void issue(int s, char *dst) const {
        const uint16_t *sb = KMAJOR ? tile_base + s * 64 : tile_base + (int64_t)s * 64 * ld;
        const uint64_t a = reinterpret_cast<uint64_t>(sb);
        const u32x4 rs = {(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, 0xFFFFFFFFu, 0x00020000u};
        const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) char *)dst);
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q)
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :
                         : "s"(lds0 + seg[q]), "v"(voff[q]), "s"(rs)
                         : "memory", "m0");
    }
};

// Byte offsets (within an operand region) of one lane's fragment reads for the
// 16 operand rows starting at `rbase`, leaf h of the stage.
template <bool KMAJOR, int NR>
struct FragAddr {
    int off[2][2];  // [h][half]; K-major uses off[h][0] only

    __device__ __forceinline__ void init(int rbase, int lane) {
        const int i = lane & 15, G = lane >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (KMAJOR) {
                const int row = rbase + i;
                off[h][0] = row * 128 + (((4 * h + G) ^ lds_key(row)) << 4);
                off[h][1] = 0;
            } else {
                constexpr int NC = NR / 8;
                const int m = i >> 2, q = i & 3;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int r = 32 * h + 8 * G + 4 * half + m;   // reduction row
                    const int col = rbase + 4 * q;                 // first of 4 operand rows
                    const int lc = col >> 3;
                    off[h][half] = r * (NR * 2) + (((lc ^ mn_key<NC>(r)) << 4) | ((col & 7) * 2));
                }
            }
        }
    }

    __device__ __forceinline__ bf16x8 read(const char *region, int h) const {
        if (KMAJOR) {
            return *reinterpret_cast<const bf16x8 *>(region + off[h][0]);
        } else {
            const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(region + off[h][0]));
            const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(region + off[h][1]));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            return __builtin_bit_cast(bf16x8, v);
        }
    }
};

template <bool XK, bool YK, int FM, int FN, int WM, int WN>
struct FastEngine {
    static constexpr int NW = WM * WN;
    static constexpr int BM = 16 * FM * WM;
    static constexpr int BN = 16 * FN * WN;
    static constexpr int XB = BM * 128, YB = BN * 128;
    static constexpr int BUF = XB + YB;
    static constexpr int NBUF = 3;
    static constexpr int kFM = FM, kFN = FN;
    typedef Frag<FM, FN> F;

    // Upper tree levels parked in LDS: per level, each lane's packed node (8
    // bytes per 16x16 block), lanes adjacent so the accesses are conflict-free.
    static constexpr int PARK_FRAG = NW * 64 * 8;
    static constexpr int PARK_LEVEL = FM * FN * PARK_FRAG;
    static constexpr int REG_LEVELS = 1;  // levels kept in registers by the tree evaluator
    static constexpr int lds_bytes(int levels) {
        return NBUF * BUF + (levels > REG_LEVELS ? levels - REG_LEVELS : 0) * PARK_LEVEL;
    }

    const MfmaParams &p;
    char *smem;
    DirectStager<XK, BM, NW> sx;
    DirectStager<YK, BN, NW> sy;
    FragAddr<XK, BM> fx[FM];
    FragAddr<YK, BN> fy[FN];
    int park_off;
    int S;

    __device__ __forceinline__ FastEngine(const MfmaParams &p_, char *smem_, int i0, int j0)
        : p(p_), smem(smem_) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int wm = wave % WM, wn = wave / WM;
        sx.init(p.x, p.ldx, i0, p.I, wave, lane);
        sy.init(p.y, p.ldy, j0, p.J, wave, lane);
#pragma unroll
        for (int a = 0; a < FM; ++a)
            fx[a].init(wm * FM * 16 + a * 16, lane);
#pragma unroll
        for (int b = 0; b < FN; ++b)
            fy[b].init(wn * FN * 16 + b * 16, lane);
        S = p.R / 64;
        park_off = NBUF * BUF + threadIdx.x * 8;
    }

    static constexpr int LOADS = DirectStager<XK, BM, NW>::PER_WAVE + DirectStager<YK, BN, NW>::PER_WAVE;

    // MFMA operands of the current stage.
    bf16x8 fa[2][FM], fb[2][FN];  // [leaf][fragment]

    __device__ __forceinline__ void issue(int s) {
        char *buf = smem + (s % NBUF) * BUF;
        sx.issue(s, buf);
        sy.issue(s, buf + XB);
    }

    // Joins the workgroup once this wave's loads are done up to `keep` stages
    // of loads in flight; lgkmcnt(0) first retires this wave's LDS reads, so
    // after the barrier no wave still reads a buffer it has consumed.
    __device__ __forceinline__ void sync(int keep) {
        if (keep >= 1)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // Stages 0 and 1 in flight.
    __device__ __forceinline__ void prologue() {
        issue(0);
        if (S > 1)
            issue(1);
    }

    // Start of stage s: waits for this wave's loads of stage s (those of
    // stage s + 1 may stay in flight), joins the workgroup -- after which all
    // of stage s is in LDS and every wave is done reading stage s - 1 --,
    // refills the buffer of stage s - 1 with stage s + 2 and issues the
    // fragment reads of stage s.  The caller then runs the tree adds that the
    // previous stage made possible while the reads are in flight, and finally
    // the leaf MFMAs (leaves()).
    __device__ __forceinline__ void begin(int s) {
        sync(s + 1 < S ? 1 : 0);
        if (s + 2 < S)
            issue(s + 2);
        const char *buf = smem + (s % NBUF) * BUF;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int a = 0; a < FM; ++a)
                fa[h][a] = fx[a].read(buf, h);
#pragma unroll
            for (int b = 0; b < FN; ++b)
                fb[h][b] = fy[b].read(buf + XB, h);
        }
    }

    template <class P>
    __device__ __forceinline__ void park(int slot, const P &v) {
        char *base = smem + park_off + slot * PARK_LEVEL;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                *reinterpret_cast<uint2 *>(base + (a * FN + b) * PARK_FRAG) =
                    make_uint2(v.w[a][b][0], v.w[a][b][1]);
    }

    template <class P>
    __device__ __forceinline__ P unpark(int slot) const {
        const char *base = smem + park_off + slot * PARK_LEVEL;
        P v;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const uint2 w = *reinterpret_cast<const uint2 *>(base + (a * FN + b) * PARK_FRAG);
                v.w[a][b][0] = w.x;
                v.w[a][b][1] = w.y;
            }
        return v;
    }

    // The two leaves of the current stage.
    __device__ __forceinline__ void leaves(F &l0, F &l1) {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
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
    }
};

// ---------------------------------------------------------------- the tree
//
// A node kept for later use is stored rounded to bf16: per 16x16 block, the
// lane's four values as two packed pairs (v0, v1), (v2, v3).  Rounding a node
// early does not change the sum its parent forms, which rounds it anyway.
template <int FM, int FN>
struct Packed {
    uint32_t w[FM][FN][2];
};

template <int FM, int FN>
__device__ __forceinline__ Packed<FM, FN> pack(const Frag<FM, FN> &x) {
    Packed<FM, FN> o;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            o.w[a][b][0] = pair_bits(round_pair(x.v[a][b][0], x.v[a][b][1]));
            o.w[a][b][1] = pair_bits(round_pair(x.v[a][b][2], x.v[a][b][3]));
        }
    return o;
}

// B operand of the tree add on the matrix core, "split" pairing: output column
// 4g + v of a 16x16 block is the sum of the A-row entries k = 8g + v and
// k = 8g + 4 + v.  A lane's A operand is then (left child's four values, right
// child's four values), each child packed on its own, so a node is packed once
// however long it waits.  The sums land where the pairing of mfma_kernel.h puts
// them (block position (r, c) moves to (c, r)), and the arithmetic is the same:
// two exact products, every other product zero.  Lane 16g + j holds B rows
// 8g .. 8g+7 of column j.
__device__ __forceinline__ bf16x8 split_selector(int lane) {
    const int j = lane & 15, g = lane >> 4;
    u32x4 s = {0u, 0u, 0u, 0u};
    if ((j >> 2) == g) {
        const int v = j & 3;
        const uint32_t one = (v & 1) ? 0x3F800000u : 0x00003F80u;
        s[v >> 1] = one;
        s[2 + (v >> 1)] = one;
    }
    return __builtin_bit_cast(bf16x8, s);
}

// Tree adds on packed children, producing the parent's unrounded fp32 values.
struct SplitMatrixAdd {
    static constexpr bool kTransposes = true;
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> add(const Packed<FM, FN> &l,
                                                       const Packed<FM, FN> &r, bf16x8 sel) {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const u32x4 A = {l.w[a][b][0], l.w[a][b][1], r.w[a][b][0], r.w[a][b][1]};
                o.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A),
                                                                    sel, zero, 0, 0, 0);
            }
        return o;
    }
    // An add with a zero partner: same value, other layout parity.
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> flip(const Packed<FM, FN> &x, bf16x8 sel) {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const u32x4 A = {x.w[a][b][0], x.w[a][b][1], 0u, 0u};
                o.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A),
                                                                    sel, zero, 0, 0, 0);
            }
        return o;
    }
};

// The same adds element by element on the VALU (exact IEEE behaviour for
// non-finite values; positions never move).
struct SplitValuAdd {
    static constexpr bool kTransposes = false;
    __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> add(const Packed<FM, FN> &l,
                                                       const Packed<FM, FN> &r, bf16x8) {
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                o.v[a][b][0] = lo(l.w[a][b][0]) + lo(r.w[a][b][0]);
                o.v[a][b][1] = hi(l.w[a][b][0]) + hi(r.w[a][b][0]);
                o.v[a][b][2] = lo(l.w[a][b][1]) + lo(r.w[a][b][1]);
                o.v[a][b][3] = hi(l.w[a][b][1]) + hi(r.w[a][b][1]);
            }
        return o;
    }
    template <int FM, int FN>
    __device__ static __forceinline__ Frag<FM, FN> flip(const Packed<FM, FN> &x, bf16x8) {
        Frag<FM, FN> o;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                o.v[a][b][0] = lo(x.w[a][b][0]);
                o.v[a][b][1] = hi(x.w[a][b][0]);
                o.v[a][b][2] = lo(x.w[a][b][1]);
                o.v[a][b][3] = hi(x.w[a][b][1]);
            }
        return o;
    }
};

// Evaluates the whole tree for L = b * 2^a leaves, b in {1, 3}: blocks of 8
// leaves (b = 1) or 12 leaves (b = 3), each a fixed schedule of adds, then the
// levels above the blocks.  The adds that a stage's leaves make possible run in
// the next stage: those whose inputs are ready go between the fragment reads
// and the leaf MFMAs, those that need a result of the same stage go after the
// leaf MFMAs, so dependency chains overlap independent matrix work instead of
// stalling the wave.  The pending node of each upper level (at most one per
// level) waits packed: in registers for the lowest level, in LDS above.
template <class E, class Arith, int TB>
struct PipeTree {
    typedef typename E::F F;
    typedef Packed<E::kFM, E::kFN> P;
    E &e;
    const bf16x8 sel;
    const int levels;
    P park0;
    F root;

    __device__ __forceinline__ PipeTree(E &e_, bf16x8 sel_, int levels_)
        : e(e_), sel(sel_), levels(levels_) {}

    __device__ __forceinline__ F add(const F &l, const F &r) { return Arith::add(pack(l), pack(r), sel); }
    __device__ __forceinline__ F add(const P &l, const F &r) { return Arith::add(l, pack(r), sel); }
    __device__ __forceinline__ F flip(const F &x) { return Arith::flip(pack(x), sel); }

    // The root v of block `blk` climbs the levels above the blocks: it merges
    // with the pending node of each level whose bit in blk is set, and waits
    // at the first level whose bit is clear.  Level 0 (every other block) waits
    // in registers, the levels above in LDS.
    __device__ __forceinline__ void climb(F v, int blk) {
        if (levels == 0) {
            root = v;
            return;
        }
        if (!(blk & 1)) {
            park0 = pack(v);
            return;
        }
        v = add(park0, v);
        int h = 1;
        while (h < levels && ((blk >> h) & 1)) {
            v = Arith::add(e.template unpark<P>(h - 1), pack(v), sel);
            ++h;
        }
        if (h < levels)
            e.park(h - 1, pack(v));
        else
            root = v;
    }

    __device__ __forceinline__ void run(int nblk) {
        if constexpr (TB == 1)
            run8(nblk);
        else
            run12(nblk);
    }

    // 8 leaves in stages A..D: ((l0 l1)(l2 l3))((l4 l5)(l6 l7)).  The first
    // block is peeled off so that no value of the loop body is conditionally
    // defined (which would keep it alive across iterations).
    __device__ __forceinline__ void run8(int nblk) {
        F l6, l7, d45;  // carried into the next block
        P n03p;
        {
            F l0, l1, l2, l3, l4, l5;
            e.begin(0);
            e.leaves(l0, l1);
            e.begin(1);
            const F d01 = add(l0, l1);
            e.leaves(l2, l3);
            block8_cd(2, d01, l2, l3, l4, l5, l6, l7, d45, n03p);
        }
        for (int blk = 1; blk < nblk; ++blk) {
            const int s0 = blk * 4;
            F l0, l1, l2, l3, l4, l5;
            e.begin(s0);                        // A
            const F d67 = add(l6, l7);
            e.leaves(l0, l1);
            const F n47 = add(d45, d67);
            e.begin(s0 + 1);                    // B
            const F d01 = add(l0, l1);
            const F top = add(n03p, n47);
            e.leaves(l2, l3);
            climb(top, blk - 1);
            block8_cd(s0 + 2, d01, l2, l3, l4, l5, l6, l7, d45, n03p);
        }
        const F d67 = add(l6, l7);
        const F n47 = add(d45, d67);
        climb(add(n03p, n47), nblk - 1);
    }

    // Stages C and D of an 8-leaf block.
    __device__ __forceinline__ void block8_cd(int s, const F &d01, const F &l2, const F &l3, F &l4,
                                              F &l5, F &l6, F &l7, F &d45, P &n03p) {
        e.begin(s);                             // C
        const F d23 = add(l2, l3);
        e.leaves(l4, l5);
        const F n03 = add(d01, d23);
        e.begin(s + 1);                         // D
        n03p = pack(n03);
        d45 = add(l4, l5);
        e.leaves(l6, l7);
    }

    // 12 leaves in stages S0..S5: (l0 (l1 l2))(l3 (l4 l5)) | (l6 (l7 l8))(l9 (l10 l11)).
    // A single leaf meets a two-leaf node, one level taller, through a flip.
    __device__ __forceinline__ void run12(int nblk) {
        F l9, l10, l11, n69;  // carried into the next block
        P n06p;
        {
            F l0, l1, l2, l3;
            e.begin(0);
            e.leaves(l0, l1);
            e.begin(1);
            const F f0 = flip(l0);
            e.leaves(l2, l3);
            block12_rest(2, f0, l1, l2, l3, l9, l10, l11, n69, n06p);
        }
        for (int blk = 1; blk < nblk; ++blk) {
            const int s0 = blk * 6;
            F l0, l1, l2, l3;
            e.begin(s0);                        // S0
            const F t10 = add(l10, l11);
            const F g9 = flip(l9);
            e.leaves(l0, l1);
            const F n612 = add(n69, add(g9, t10));
            e.begin(s0 + 1);                    // S1
            const F f0 = flip(l0);
            const F top = add(n06p, n612);
            e.leaves(l2, l3);
            climb(top, blk - 1);
            block12_rest(s0 + 2, f0, l1, l2, l3, l9, l10, l11, n69, n06p);
        }
        const F t10 = add(l10, l11);
        const F g9 = flip(l9);
        const F n612 = add(n69, add(g9, t10));
        climb(add(n06p, n612), nblk - 1);
    }

    // Stages S2..S5 of a 12-leaf block.
    __device__ __forceinline__ void block12_rest(int s, const F &f0, const F &l1, const F &l2,
                                                 const F &l3, F &l9, F &l10, F &l11, F &n69,
                                                 P &n06p) {
        F l4, l5, l6, l7, l8;
        e.begin(s);                             // S2
        const F t1 = add(l1, l2);
        e.leaves(l4, l5);
        const F n03 = add(f0, t1);
        e.begin(s + 1);                         // S3
        const F t4 = add(l4, l5);
        const F f3 = flip(l3);
        e.leaves(l6, l7);
        const F n06 = add(n03, add(f3, t4));
        e.begin(s + 2);                         // S4
        n06p = pack(n06);
        const F f6 = flip(l6);
        e.leaves(l8, l9);
        e.begin(s + 3);                         // S5
        const F t7 = add(l7, l8);
        e.leaves(l10, l11);
        n69 = add(f6, t7);
    }
};

template <bool XK, bool YK, int OUT, int TB, int TK, int FM, int FN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void mfma_fast_kernel(MfmaParams p) {
    typedef FastEngine<XK, YK, FM, FN, WM, WN> E;
    typedef typename E::F F;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int tile = blockIdx.x;
    const int i0 = (tile / p.tiles_j) * E::BM;
    const int j0 = (tile % p.tiles_j) * E::BN;

    E e(p, smem, i0, j0);
    const bf16x8 sel = split_selector(lane);
    const int nblk = p.L / (TB << TK);
    e.prologue();
    PipeTree<E, SplitMatrixAdd, TB> tree(e, sel, p.levels);
    tree.run(nblk);
    bool nonfinite = false;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                nonfinite |= !(__builtin_fabsf(tree.root.v[a][b][v]) <= 3.40282347e38f);
    // A non-finite root may have spilled NaN into the other sums of its
    // matrix-core add rows: recompute such a tile with element-wise adds.
    if (__syncthreads_or(nonfinite)) {
        e.prologue();
        PipeTree<E, SplitValuAdd, TB> valu(e, sel, p.levels);
        valu.run(nblk);
        store_root<OUT>(p, valu.root, false, i0, j0, wm, wn, lane);
    } else {
        store_root<OUT>(p, tree.root, (tree_height_rt(p.L) & 1) != 0, i0, j0, wm, wn, lane);
    }
}

}  // namespace detgemm
