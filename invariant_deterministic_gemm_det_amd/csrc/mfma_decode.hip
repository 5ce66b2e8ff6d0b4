// Decode-shaped forward products: at most 128 rows of X (one token, or a small
// batch of them, against a weight matrix).  Same leaves, same tree, same bits
// as every other det_gemm kernel; only the work split differs.
//
// The contract (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
// (det_gemm)", sections on the leaf product-sum and the mid-split reduction
// tree) forbids splitting the reduction across workgroups, and a product of a
// few rows has only N / 16 output blocks per 16 rows: 384 at N = 6144, too few
// to keep 256 compute units streaming the weights if each block walks the
// whole reduction alone.  Here the tree itself supplies the parallelism inside
// a workgroup:
//   * a workgroup owns an M x 16 CB output tile: all M rows (staged as 1, 2, 4
//     or 8 blocks of 16 rows: M <= 16, 32, 64 or 128; 32-column tiles take at
//     most 64 rows, 64-column tiles at most 16) and 16, 32 or 64 columns, one
//     MFMA per row block and column block with its own tree state.  It has
//     W = 8 or 16 waves; wave w evaluates the subtree rooted at node w of
//     depth log2(W) of the mid-split tree over the L leaves (L >= W, so every
//     such node holds at least one leaf), a contiguous range of about L / W
//     leaves;
//   * a wave walks its leaves in ascending order with the streaming post-order
//     (after leaf t, as many adds as there are inner nodes whose range ends at
//     t + 1), pending left siblings in registers;
//   * the W subtree roots meet in LDS and the first waves (one per 16 x 16
//     block) add them in the order of the top log2(W) levels.
// A leaf is the same v_mfma_f32_16x16x32_bf16 with the same lane assignment as
// in the other kernels (lane l: X row l % 16 and Y column l % 16 at reduction
// indices 8(l / 16) .. +7).  Inside a wave's subtree a tree add is the
// selector MFMA of the wide kernel (a leaf at odd depth is computed with
// swapped operands, so both children of every add share a layout); the top
// levels use the element-wise VALU add; a tile whose root is not finite is
// recomputed with element-wise adds throughout.  Both adds give the exactly
// rounded bf16 sum, so the bits are those of every other configuration.
//
// Data movement, per wave and without workgroup barriers: a private ring of
// NB unit slots in LDS (a unit: one leaf, or two leaves of a K-major Y),
// filled by buffer_load_dwordx4 ... lds (16 bytes per lane at M0 + 16 * lane)
// NB - 1 units ahead, drained with s_waitcnt vmcnt.
//   * Y, reduction index contiguous (the weight stored [N][K]), two-leaf
//     units (even L): 128-byte rows (one whole cache line per column), chunk c
//     of row r at c ^ ((r >> 1) & 7); one-leaf units: 64-byte rows, chunk c of
//     row r at c ^ ((r >> 2) & 3).  Either way the 16 rows of one
//     quarter-wave's ds_read_b128 land on all 64 banks.
//   * Y, column index contiguous (the weight stored [K][N]): 32 indices x 16 CB
//     columns.  16 columns: 32-byte rows, rows with bit 3 set swap 128-byte
//     halves; 32 columns: 64-byte rows, rows with bit 3 set swap 32-byte
//     halves; 64 columns: 128-byte rows, 16-byte chunks XORed as in the
//     direct-to-LDS kernel.  Each way the two 16-lane groups of a half-wave
//     ds_read_b64_tr_b16 (indices r0 .. r0+3 and r0+8 .. r0+11) use disjoint
//     banks.
//   * X: the MP rows the product needs (MP = 1 for a single row, else 16, 32,
//     64 or 128, rows past the last clamped to it) in the K-major layout of
//     the unit.
// A compute unit serves these copies at a bounded rate of cache-line requests,
// so wider tiles (more of each requested line used) stream faster and narrower
// ones reach more compute units; the host picks the width from the tile count.
// Workgroup b runs on XCD b mod 8; consecutive tiles go to the same XCD, so the
// workgroups that share a 128-byte line of a [K][N] weight share that XCD's L2.
#include "mfma_launch.h"

namespace detgemm {

namespace {

// CB column blocks of 16 per workgroup (a tile of 16 * CB columns), MP staged
// rows of X (1, 16, 32, 64 or 128: MR = 1, 2, 4 or 8 blocks of 16), UL leaves
// per copy unit (2: a K-major Y read as whole 128-byte lines, two leaves of
// each column), W waves (one subtree each: depth 3 or 4).
template <int MP, int CB, int UL, int W>
struct DecodeShape {
    static constexpr int MR = MP >= 16 ? MP / 16 : 1;
    static constexpr int Y_BYTES = CB * 1024 * UL;
    static constexpr int SLOT = Y_BYTES + MP * 64 * UL;   // Y tile, then the X blocks
    // Ring slots per wave.  Measured: deeper rings do not help (the limit is
    // how the copies meet the memory system, not the bytes in flight), while
    // two workgroups per compute unit do: 4 slots for 16- and 32-column
    // tiles, 2 for 64-column ones and for the larger two-leaf units; with 16
    // waves, as many as the LDS holds (at least 2).
    static constexpr int NB0 = UL == 2 ? ((CB == 1 && MP == 1) ? 4 : 2) : (CB == 4 ? 2 : 4);
    static constexpr int NB = (NB0 > 2 && W * NB0 * SLOT > 160 * 1024) ? NB0 / 2 : NB0;
    static constexpr int AHEAD = NB - 1;                  // units in flight per wave
    static constexpr int OPS = UL == 2 ? 2 * CB + (MP == 1 ? 1 : 2 * MR) : CB + MR;  // copies per unit
    static constexpr int WAVE_BYTES = NB * SLOT;
    static constexpr int LDS = W * WAVE_BYTES;
    static constexpr int BPW = (MR * CB + W - 1) / W;      // output blocks per wave at the end
    static constexpr bool kFits = NB >= 2 && LDS <= 160 * 1024 && WAVE_BYTES >= MR * CB * 1024;
    // Waves per SIMD the register allocation must allow: two workgroups per
    // compute unit when their rings fit the LDS twice, and at most four.
    static constexpr int OCC = (W / 4) * (2 * LDS <= 160 * 1024 ? 2 : 1) < 4 ? (W / 4) * (2 * LDS <= 160 * 1024 ? 2 : 1) : 4;
};

__device__ __forceinline__ int kt_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }
__device__ __forceinline__ int nt_row(int r) { return (r * 32) ^ (((r >> 3) & 1) << 7); }
// K-major two-leaf tiles (128-byte rows: 64 reduction indices): chunk c of row
// r at c ^ ((r >> 1) & 7), the layout of the direct-to-LDS kernel; the 16 rows
// of one quarter-wave's ds_read_b128 land on all 64 banks.
__device__ __forceinline__ int kt128(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
// 128-byte rows (64 columns): chunk c of row r at c ^ key8(r); one half-wave's
// transposed read (rows r0 .. r0+3 and r0+8 .. r0+11, one aligned chunk pair
// each) then covers disjoint banks.
__device__ __forceinline__ int key8(int r) { return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)); }

__device__ __forceinline__ u32x4 rsrc_at(const void *base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const u32x4 rs = {(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, 0xFFFFFFFFu, 0x00020000u};
    return rs;
}

// One 1 KB (or, with fewer active lanes, smaller) LDS DMA.  Waits for the
// wave's outstanding LDS reads first: the slot being refilled was read by the
// previous unit.  One wait state separates the M0 write from the load.  NT:
// a non-temporal load (weights that do not stay in the caches).
template <bool NT = false>
__device__ __forceinline__ void dma16(uint32_t lds, int voff, u32x4 rs) {
    if constexpr (NT)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     :
                     : "s"(lds), "v"(voff), "s"(rs)
                     : "memory", "m0");
    else
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(lds), "v"(voff), "s"(rs)
                     : "memory", "m0");
}

// The pending left siblings of one 16 x 16 block of a wave: one 16-dword
// register vector indexed by the wave-uniform depth, which the compiler reads
// and writes with GPR indexing (no branches, no per-lane scratch array).  A
// node waits rounded to bf16 (two packed pairs): its parent's add rounds it to
// bf16 anyway, so storing it rounded changes nothing and halves the registers.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 pack_node(f32x4 v) {
    const u32x2 o = {pair_bits(round_pair(v[0], v[1])), pair_bits(round_pair(v[2], v[3]))};
    return o;
}

__device__ __forceinline__ f32x4 unpack_node(u32x2 h) {
    const f32x4 o = {__uint_as_float(h[0] << 16), __uint_as_float(h[0] & 0xFFFF0000u),
                     __uint_as_float(h[1] << 16), __uint_as_float(h[1] & 0xFFFF0000u)};
    return o;
}

struct NodeStack {
    typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
    u32x16 v;   // pair d in elements 2d, 2d + 1; d is wave-uniform
    __device__ __forceinline__ f32x4 get(int d) const {
        const u32x2 h = {v[2 * d], v[2 * d + 1]};
        return unpack_node(h);
    }
    __device__ __forceinline__ u32x2 raw(int d) const {
        const u32x2 h = {v[2 * d], v[2 * d + 1]};
        return h;
    }
    __device__ __forceinline__ void put(int d, f32x4 x) {
        const u32x2 h = pack_node(x);
        v[2 * d] = h[0];
        v[2 * d + 1] = h[1];
    }
};

// Root of the W subtree roots in the order of the top log2(W) levels.
template <int LO, int HI>
__device__ __forceinline__ f32x4 top_levels(const f32x4 *r) {
    if constexpr (HI - LO == 1)
        return r[LO];
    else
        return merge4(top_levels<LO, (LO + HI) / 2>(r), top_levels<(LO + HI) / 2, HI>(r));
}

// Where leaf t of the mid-split tree over [0, n) stands: the number of inner
// nodes whose range ends at it (the adds that follow it in post-order) and
// the parity of its depth (root: depth 0).
struct LeafPlan {
    int merges;
    int odd;
};

__device__ __forceinline__ LeafPlan leaf_plan(int t, int n) {
    int lo = 0, hi = n, merges = 0, depth = 0;
    while (hi - lo > 1) {
        if (hi == t + 1)
            ++merges;
        const int mid = lo + (hi - lo) / 2;
        if (t < mid)
            hi = mid;
        else
            lo = mid;
        ++depth;
    }
    return LeafPlan{merges, depth & 1};
}

// Register budget: 128 VGPRs when four waves share a SIMD (two 8-wave
// workgroups or one 16-wave workgroup per compute unit), else 256.
template <bool YK, int OUT, int MP, int CB, int UL, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(DecodeShape<MP, CB, UL, W>::OCC,
                                                                       DecodeShape<MP, CB, UL, W>::OCC)))
void mfma_decode_kernel(MfmaParams p) {
    static_assert(UL == 1 || YK, "two-leaf units only for a K-major Y");
    static_assert(W == 8 || W == 16, "subtrees of depth 3 or 4");
    typedef DecodeShape<MP, CB, UL, W> S;
    static_assert(S::kFits, "the rings fit the LDS");
    constexpr int MR = S::MR;
    typedef Frag<(MP >= 16 ? MP / 16 : 1), CB> F;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // Tile of this workgroup: XCD x = b mod 8 owns a contiguous run of tiles.
    const int nb = p.tiles_j, b = blockIdx.x;
    const int x = b & 7, q8 = nb >> 3, rem = nb & 7;
    const int tile = x * q8 + (x < rem ? x : rem) + (b >> 3);
    const int j0 = tile * 16 * CB;

    // Leaf range of this wave: node `wave` at depth log2(W) of the mid-split
    // tree.
    int lo = 0, hi = p.L;
#pragma unroll
    for (int bit = (W == 16 ? 3 : W == 8 ? 2 : 1); bit >= 0; --bit) {
        const int mid = lo + (hi - lo) / 2;
        if ((wave >> bit) & 1)
            lo = mid;
        else
            hi = mid;
    }
    const int n = hi - lo;

    // Copy units of this wave: the units holding leaves lo .. hi-1 (with
    // two-leaf units the first and last may hold a neighbour's leaf, which is
    // read and skipped).
    const int ulo = lo / UL, nunits = (hi + UL - 1) / UL - ulo;

    // Per-lane source offsets (bytes) of the copies of a unit; the unit's base
    // address moves in the scalar resource.
    int yoff[CB * UL];
    int xoff2[MR][2] = {};
    const uint16_t *ybase;
    if (UL == 2) {
        // copy 2q + s: columns 16q + 8s .. +7 of the tile, 128 bytes each
        const int cp = lane & 7;
#pragma unroll
        for (int q = 0; q < CB; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 8 * h + (lane >> 3);            // column within the block
                const int c = cp ^ ((row >> 1) & 7);
                const int col = j0 + 16 * q + row < p.J ? j0 + 16 * q + row : p.J - 1;
                yoff[q * UL + h] = (int)(((int64_t)(col - j0) * p.ldy + 8 * c) * 2);
            }
        ybase = p.y + (int64_t)j0 * p.ldy;
#pragma unroll
        for (int a = 0; a < MR; ++a)
#pragma unroll
            for (int h = 0; h < 2; ++h) {   // X rows 16a + 8h .. +7, or lanes 0..7 of row 0
                const int row = MP == 1 ? 0 : 8 * h + (lane >> 3);
                const int c = MP == 1 ? lane : (cp ^ ((row >> 1) & 7));
                const int rr = 16 * a + row < p.I ? 16 * a + row : p.I - 1;
                xoff2[a][h] = (int)(((int64_t)rr * p.ldx + 8 * c) * 2);
            }
    } else if (YK) {
        // copy q: columns 16q .. 16q+15 of the tile, K-major slot layout
        const int r = lane >> 2, c = (lane & 3) ^ ((r >> 2) & 3);
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int col = j0 + 16 * q + r < p.J ? j0 + 16 * q + r : p.J - 1;
            yoff[q] = (int)(((int64_t)(col - j0) * p.ldy + 8 * c) * 2);
        }
        ybase = p.y + (int64_t)j0 * p.ldy;
    } else if (CB == 1) {
        const int P = 16 * lane;
        const int qq = P ^ (((P >> 8) & 1) << 7);
        const int r = qq >> 5, c = (qq >> 4) & 1;
        int col = j0 + 8 * c;
        if (col >= p.J)
            col = p.J - 8;  // J is a multiple of 8 on this path
        yoff[0] = (int)(((int64_t)r * p.ldy + (col - j0)) * 2);
        ybase = p.y + j0;
    } else if (CB == 2) {
        // copy q: reduction rows 16q .. 16q+15, 64 bytes each
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int r = 16 * q + (lane >> 2), c16 = lane & 3;
            int col = j0 + 16 * ((c16 >> 1) ^ ((r >> 3) & 1)) + 8 * (c16 & 1);
            if (col >= p.J)
                col = p.J - 8;
            yoff[q] = (int)(((int64_t)r * p.ldy + (col - j0)) * 2);
        }
        ybase = p.y + j0;
    } else {
        // copy q: reduction rows 8q .. 8q+7, 128 bytes each
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int r = 8 * q + (lane >> 3), c = (lane & 7) ^ key8(r);
            int col = j0 + 8 * c;
            if (col >= p.J)
                col = p.J - 8;
            yoff[q] = (int)(((int64_t)r * p.ldy + (col - j0)) * 2);
        }
        ybase = p.y + j0;
    }
    int xoff[MR];
#pragma unroll
    for (int a = 0; a < MR; ++a) {   // X rows 16a .. 16a+15
        const int r = lane >> 2, c = (lane & 3) ^ ((r >> 2) & 3);
        const int row = 16 * a + r < p.I ? 16 * a + r : p.I - 1;
        xoff[a] = (int)(((int64_t)row * p.ldx + 8 * c) * 2);
    }
    const int64_t ystep = YK ? 32 * UL : (int64_t)32 * p.ldy;  // elements per unit

    // Fragment read offsets within a slot.
    const int i16 = lane & 15, G = lane >> 4;
    const int xrd = S::Y_BYTES + kt_off(MP == 1 ? 0 : i16, G);
    int yrd[CB][2];
#pragma unroll
    for (int q = 0; q < CB; ++q) {
        if (YK) {
            yrd[q][0] = q * 1024 + kt_off(i16, G);
            yrd[q][1] = 0;
        } else if (CB == 1) {
            const int m = i16 >> 2, qq = i16 & 3;
            yrd[q][0] = nt_row(8 * G + m) + 8 * qq;
            yrd[q][1] = nt_row(8 * G + 4 + m) + 8 * qq;
        } else if (CB == 2) {
            const int m = i16 >> 2, qq = i16 & 3;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 8 * G + 4 * h + m;
                yrd[q][h] = r * 64 + ((q ^ ((r >> 3) & 1)) << 5) + 8 * qq;
            }
        } else {
            const int m = i16 >> 2, col = 16 * q + 4 * (i16 & 3), lc = col >> 3;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 8 * G + 4 * h + m;
                yrd[q][h] = r * 128 + (((lc ^ key8(r)) << 4) | ((col & 7) * 2));
            }
        }
    }

    int xp[2], yp[CB][2];   // two-leaf units: leaf h of the unit
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        xp[h] = S::Y_BYTES + (MP == 1 ? (4 * h + G) * 16 : kt128(i16, 4 * h + G));
#pragma unroll
        for (int q = 0; q < CB; ++q)
            yp[q][h] = q * 2048 + kt128(i16, 4 * h + G);
    }

    char *ring = smem + wave * S::WAVE_BYTES;
    const uint32_t ring_lds =
        (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char *)ring);

    const bool ynt = __builtin_amdgcn_readfirstlane(p.ynt) != 0;
    auto ycopy = [&](uint32_t lds, int voff, u32x4 rs) {
        if (ynt)
            dma16<true>(lds, voff, rs);
        else
            dma16<false>(lds, voff, rs);
    };
    auto issue = [&](int u) {  // local unit u into slot u % NB
        const int unit = ulo + u;
        const uint32_t slot = ring_lds + (uint32_t)((u % S::NB) * S::SLOT);
        const u32x4 rs = rsrc_at(ybase + (int64_t)unit * ystep);
        const u32x4 xs = rsrc_at(p.x + (int64_t)unit * 32 * UL);
        if (UL == 2) {
#pragma unroll
            for (int e = 0; e < 2 * CB; ++e)
                ycopy(slot + e * 1024, yoff[e], rs);
            if (MP == 1) {
                if (lane < 8)
                    dma16(slot + S::Y_BYTES, xoff2[0][0], xs);
            } else {
#pragma unroll
                for (int a = 0; a < MR; ++a) {
                    dma16(slot + S::Y_BYTES + a * 2048, xoff2[a][0], xs);
                    dma16(slot + S::Y_BYTES + a * 2048 + 1024, xoff2[a][1], xs);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < CB; ++q)
                ycopy(slot + q * 1024, yoff[q], rs);
            if (MP == 1) {
                if (lane < 4)
                    dma16(slot + S::Y_BYTES, xoff[0], xs);
            } else {
#pragma unroll
                for (int a = 0; a < MR; ++a)
                    dma16(slot + S::Y_BYTES + a * 1024, xoff[a], xs);
            }
        }
    };

    // The wave's subtree, in ascending leaf order.  Matrix-core adds (MA):
    // a tree add is the selector MFMA of the wide kernel, whose result lands
    // transposed; a leaf at odd depth below the wave's root is computed with
    // swapped operands (the same products and sums, transposed), so that the
    // two children of every add share a layout and the wave's root comes out
    // in the plain layout.  Element-wise adds (not MA): merge4, positions
    // never move.
    const bf16x8 sel = split_selector(lane);
    auto subtree = [&](auto matrix_add) {
        constexpr bool MA = decltype(matrix_add)::value;
        const int pre = nunits < S::AHEAD ? nunits : S::AHEAD;
        for (int u = 0; u < pre; ++u)
            issue(u);

        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        NodeStack st[MR][CB];
#pragma unroll
        for (int a = 0; a < MR; ++a)
#pragma unroll
            for (int q = 0; q < CB; ++q)
                st[a][q].v = 0u;
        int sp = 0;
        for (int u = 0; u < nunits; ++u) {
            if (u + S::AHEAD < nunits) {
                issue(u + S::AHEAD);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::OPS * S::AHEAD) : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            const char *slot = ring + (u % S::NB) * S::SLOT;
#pragma unroll
            for (int h = 0; h < UL; ++h) {
                const int t = (ulo + u) * UL + h - lo;   // local leaf
                if (t < 0 || t >= n)
                    continue;                            // a neighbour's leaf of a two-leaf unit
                const LeafPlan lp = leaf_plan(t, n);
                bf16x8 fx[MR];
#pragma unroll
                for (int a = 0; a < MR; ++a)
                    fx[a] = *reinterpret_cast<const bf16x8 *>(slot + (UL == 2 ? xp[h] + a * 2048 : xrd + a * 1024));
                bf16x8 fy[CB];
#pragma unroll
                for (int q = 0; q < CB; ++q) {
                    if (UL == 2) {
                        fy[q] = *reinterpret_cast<const bf16x8 *>(slot + yp[q][h]);
                    } else if (YK) {
                        fy[q] = *reinterpret_cast<const bf16x8 *>(slot + yrd[q][0]);
                    } else {
                        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(slot + yrd[q][0]));
                        const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(slot + yrd[q][1]));
                        typedef short s16x8 __attribute__((ext_vector_type(8)));
                        const s16x8 v = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
                        fy[q] = __builtin_bit_cast(bf16x8, v);
                    }
                }
                F cur;
                if (MA && lp.odd) {
#pragma unroll
                    for (int q = 0; q < CB; ++q)
#pragma unroll
                        for (int a = 0; a < MR; ++a)
                            cur.v[a][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fy[q], fx[a], zero, 0, 0, 0);
                } else {
#pragma unroll
                    for (int q = 0; q < CB; ++q)
#pragma unroll
                        for (int a = 0; a < MR; ++a)
                            cur.v[a][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[a], fy[q], zero, 0, 0, 0);
                }
                for (int k = 0; k < lp.merges; ++k) {
                    --sp;
#pragma unroll
                    for (int a = 0; a < MR; ++a)
#pragma unroll
                        for (int q = 0; q < CB; ++q) {
                            if constexpr (MA) {
                                const u32x4 A = __builtin_shufflevector(st[a][q].raw(sp), pack_node(cur.v[a][q]),
                                                                        0, 1, 2, 3);
                                cur.v[a][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, A), sel, zero, 0, 0, 0);
                            } else {
                                cur.v[a][q] = merge4(st[a][q].get(sp), cur.v[a][q]);
                            }
                        }
                }
                if (t + 1 < n) {
#pragma unroll
                    for (int a = 0; a < MR; ++a)
#pragma unroll
                        for (int q = 0; q < CB; ++q)
                            st[a][q].put(sp, cur.v[a][q]);
                    ++sp;
                } else {
                    // The wave's root goes to the start of its own ring: its
                    // copies are complete (the last unit waited for all of
                    // them) and nothing reads the ring after this leaf.
#pragma unroll
                    for (int a = 0; a < MR; ++a)
#pragma unroll
                        for (int q = 0; q < CB; ++q)
                            *reinterpret_cast<f32x4 *>(ring + ((a * CB + q) * 64 + lane) * 16) = cur.v[a][q];
                }
            }
        }
    };

    // The W subtree roots meet in LDS, each in its wave's own ring; wave w
    // adds the roots of blocks b = w, w + W, ... (b = row block * CB + column
    // block) in the order of the top levels, with element-wise adds.
    constexpr int BPW = S::BPW;
    f32x4 top[BPW];
    auto meet = [&]() {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BPW; ++k) {
            const int b = wave + k * W;
            top[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (b < MR * CB) {
                f32x4 r[W];
#pragma unroll
                for (int w = 0; w < W; ++w)
                    r[w] = *reinterpret_cast<const f32x4 *>(smem + w * S::WAVE_BYTES + (b * 64 + lane) * 16);
                top[k] = top_levels<0, W>(r);
            }
        }
    };

    subtree(std::true_type{});
    meet();
    // A non-finite value in a matrix-core add spreads NaN over the other sums
    // of its row, and every non-finite node leaves a non-finite root: a tile
    // with a non-finite root is recomputed with element-wise adds (exact IEEE
    // behaviour).  The flags are one dword per wave at the start of the LDS,
    // written once every root has been read.
    bool bad = false;
#pragma unroll
    for (int k = 0; k < BPW; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            bad |= !(__builtin_fabsf(top[k][v]) <= 3.40282347e38f);
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    __syncthreads();
    int *flags = reinterpret_cast<int *>(smem);
    if (lane == 0)
        flags[wave] = wave_bad ? 1 : 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < W; w += 4) {
        const uint4 f = *reinterpret_cast<const uint4 *>(flags + w);
        any |= (int)(f.x | f.y | f.z | f.w);
    }
    if (any) {
        __syncthreads();   // every wave has read the flags before the rings refill
        subtree(std::false_type{});
        meet();
    }

    // Lane 16g + c holds rows 4g .. 4g+3 of column c of the block.  A zero
    // root is stored as +0.
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
        const int b = wave + k * W;
        if (b >= MR * CB)
            break;
        const uint32_t lo2 = pair_bits(round_pair(top[k][0], top[k][1]));
        const uint32_t hi2 = pair_bits(round_pair(top[k][2], top[k][3]));
        const uint16_t v4[4] = {(uint16_t)lo2, (uint16_t)(lo2 >> 16), (uint16_t)hi2,
                                (uint16_t)(hi2 >> 16)};
        const int j = j0 + 16 * (b % CB) + i16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * (b / CB) + 4 * G + v;
            const uint16_t h = (v4[v] & 0x7FFF) ? v4[v] : (uint16_t)0;
            if (i < p.I && j < p.J) {
                if (OUT == OUT_BF16)
                    static_cast<uint16_t *>(p.c)[(int64_t)i * p.ldc + j] = h;
                else
                    static_cast<float *>(p.c)[(int64_t)i * p.ldc + j] = __uint_as_float((uint32_t)h << 16);
            }
        }
    }
}

template <bool YK, int OUT, int MP, int CB, int UL, int W>
hipError_t launch_decode_one(const MfmaParams &p, hipStream_t st) {
    typedef DecodeShape<MP, CB, UL, W> S;
    const void *fn = reinterpret_cast<const void *>(&mfma_decode_kernel<YK, OUT, MP, CB, UL, W>);
    static int max_dynamic = -1;
    if (max_dynamic < 0) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
        if (e != hipSuccess)
            return e;
        max_dynamic = S::LDS;
    }
    const int64_t tiles = (p.J + 16 * CB - 1) / (16 * CB);
    MfmaParams q = p;
    q.tiles_j = (int32_t)tiles;
    hipLaunchKernelGGL((mfma_decode_kernel<YK, OUT, MP, CB, UL, W>), dim3((unsigned)tiles),
                       dim3(64 * W), S::LDS, st, q);
    return hipGetLastError();
}

// When the tiles make at most one round over the 256 compute units, the
// chain of leaves of each wave sets the time: 16 waves (subtrees of depth 4,
// half the leaves each) when there are at least 16 leaves and the rings fit.
template <bool YK, int OUT, int MP, int CB, int UL>
hipError_t launch_decode_waves(const MfmaParams &p, hipStream_t st) {
    if constexpr (CB <= 2 && DecodeShape<MP, CB, UL, 16>::kFits) {
        const int64_t tiles = (p.J + 16 * CB - 1) / (16 * CB);
        if (p.L >= 16 && tiles <= 256)
            return launch_decode_one<YK, OUT, MP, CB, UL, 16>(p, st);
    }
    return launch_decode_one<YK, OUT, MP, CB, UL, 8>(p, st);
}

// A K-major Y with an even leaf count is copied in two-leaf units (whole
// 128-byte lines of each column), on 16- and 32-column tiles (64-column
// tiles would not fit the unit's registers) when the rings fit the LDS.
template <bool YK, int OUT, int MP, int CB>
hipError_t launch_decode_units(const MfmaParams &p, hipStream_t st) {
    if constexpr (YK && CB <= 2 && DecodeShape<MP, CB, 2, 8>::kFits) {
        if (p.L % 2 == 0)
            return launch_decode_waves<YK, OUT, MP, CB, 2>(p, st);
    }
    return launch_decode_waves<YK, OUT, MP, CB, 1>(p, st);
}

template <bool YK, int OUT, int CB>
hipError_t launch_decode_rows(const MfmaParams &p, hipStream_t st) {
    if (p.I == 1)
        return launch_decode_units<YK, OUT, 1, CB>(p, st);
    if (p.I <= 16)
        return launch_decode_units<YK, OUT, 16, CB>(p, st);
    if constexpr (CB <= 2) {   // 17 to 32 rows: two row blocks
        if (p.I <= 32)
            return launch_decode_units<YK, OUT, 32, CB>(p, st);
    }
    if constexpr (CB <= 2) {   // 33 to 64 rows: four row blocks on 16- and 32-column tiles
        if (p.I <= 64)
            return launch_decode_units<YK, OUT, 64, CB>(p, st);
    }
    if constexpr (CB == 1)     // 65 to 128 rows: eight row blocks on 16-column tiles
        return launch_decode_units<YK, OUT, 128, CB>(p, st);
    return hipErrorInvalidValue;
}

template <bool YK, int OUT>
hipError_t launch_decode_cols(const MfmaParams &p, int cb, hipStream_t st) {
    if (cb == 4)
        return launch_decode_rows<YK, OUT, 4>(p, st);
    return cb == 2 ? launch_decode_rows<YK, OUT, 2>(p, st) : launch_decode_rows<YK, OUT, 1>(p, st);
}

}  // namespace

hipError_t launch_decode(const MfmaParams &p, bool yk, int out, int cb, hipStream_t st) {
    if (yk)
        return out == OUT_BF16 ? launch_decode_cols<true, OUT_BF16>(p, cb, st)
                               : launch_decode_cols<true, OUT_F32>(p, cb, st);
    return out == OUT_BF16 ? launch_decode_cols<false, OUT_BF16>(p, cb, st)
                           : launch_decode_cols<false, OUT_F32>(p, cb, st);
}

}  // namespace detgemm
