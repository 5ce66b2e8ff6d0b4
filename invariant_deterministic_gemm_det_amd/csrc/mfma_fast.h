// Fast path of the MFMA det_gemm kernel (same leaves, same tree, same bits as
// mfma_kernel.h), used when both operands are 16-byte aligned, the reduction
// length is a multiple of 64 and the leaf count is b * 2^a with b in {1, 3}.
//
// Differences from the general kernel, all in the data movement:
//   * operands go from global memory straight into LDS with
//     buffer_load_dwordx4 ... lds (each lane writes 16 bytes at M0 + 16*lane),
//     three stage buffers deep, and no vector registers or ds_write
//     instructions carry them;
//   * software pipelining: the fragment reads of stage s + 1 are issued before
//     the MFMAs of stage s, and a buffer is refilled (stage s + 3) as soon as
//     its operands are in registers;
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
// reduction index).  NC = chunks per row: 8 (128-byte rows, two rows per LDS
// bank sweep) or 16 (256-byte rows).  One transposed fragment read touches, per
// 32 lanes, the reduction rows r0 + {0..3, 8..11} (r0 a multiple of 4), each at
// the same aligned pair of chunks; the XOR (always even, so pairs stay pairs)
// sends those rows to disjoint banks.
template <int NC>
__device__ __forceinline__ int mn_key(int r) {
    if constexpr (NC >= 16)
        return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
    else
        return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
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
    static constexpr int PARK_FRAG = NW * 64 * 8;
    static constexpr int PARK_LEVEL = FM * FN * PARK_FRAG;
    typedef Frag<FM, FN> F;

    static constexpr int lds_bytes(int levels) { return NBUF * BUF + levels * PARK_LEVEL; }

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
        park_off = NBUF * BUF + (wave * 64 + lane) * 8;
        S = p.R / 64;
    }

    static constexpr int LOADS = DirectStager<XK, BM, NW>::PER_WAVE + DirectStager<YK, BN, NW>::PER_WAVE;

    // MFMA operands of two stages: set s & 1 holds stage s while stage s + 1
    // is read into the other set.
    bf16x8 fa[2][2][FM], fb[2][2][FN];  // [set][leaf][fragment]

    __device__ __forceinline__ void issue(int s) {
        char *buf = smem + (s % NBUF) * BUF;
        sx.issue(s, buf);
        sy.issue(s, buf + XB);
    }

    template <int SET>
    __device__ __forceinline__ void read_frags(int s) {
        const char *buf = smem + (s % NBUF) * BUF;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int a = 0; a < FM; ++a)
                fa[SET][h][a] = fx[a].read(buf, h);
#pragma unroll
            for (int b = 0; b < FN; ++b)
                fb[SET][h][b] = fy[b].read(buf + XB, h);
        }
    }

    // Joins the workgroup once this wave's loads are done up to `keep` stages
    // of loads in flight; lgkmcnt(0) first retires this wave's LDS reads, so
    // after the barrier no wave still reads a buffer it has consumed.
    __device__ __forceinline__ void sync(int keep) {
        if (keep >= 2)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS) : "memory");
        else if (keep == 1)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // Stages 0, 1, 2 in flight; stage 0 in LDS and read into set 0.
    __device__ __forceinline__ void prologue() {
        issue(0);
        if (S > 1)
            issue(1);
        if (S > 2)
            issue(2);
        sync(S - 1);
        read_frags<0>(0);
    }

    // Both leaves of stage s (operands in set PAR = s & 1).  Before its MFMAs:
    // waits for stage s + 1 to land (stage s + 2 may stay in flight), joins
    // the workgroup, refills the buffer of stage s -- whose operands are
    // already in registers -- with stage s + 3, and starts reading stage s + 1
    // into the other set, so those LDS reads overlap this stage's MFMAs.
    //
    // The reads are issued even after the last stage (from a buffer no load
    // targets any more; the values are never used): with them on every path,
    // the compiler's wait before this stage's MFMAs only needs the older reads
    // of set PAR, instead of draining the ones just issued.
    template <int PAR>
    __device__ __forceinline__ void stage(int s, F &l0, F &l1) {
        sync(s + 2 < S ? 1 : 0);
        if (s + 3 < S)
            issue(s + 3);
        read_frags<PAR ^ 1>(s + 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                l0.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[PAR][0][a], fb[PAR][0][b],
                                                                     zero, 0, 0, 0);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                l1.v[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[PAR][1][a], fb[PAR][1][b],
                                                                     zero, 0, 0, 0);
    }

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
    const bf16x8 sel = add_selector(lane);
    F root;
    e.prologue();
    run_blocks<E, TB << TK, MatrixAdd>(e, p, sel, root);
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
}

}  // namespace detgemm
