// Host-side launch helpers for the MFMA kernel: one function per operand layout
// and output mode, each defined in its own translation unit (mfma_*.hip) so the
// kernel instances compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "mfma_wide.h"

namespace detgemm {

constexpr int kLdsMax = 160 * 1024;  // LDS per workgroup on gfx950

enum KernelKind { KIND_GENERAL = 0, KIND_FAST = 1, KIND_WIDE = 2, KIND_DECODE = 3 };

// Tile configurations.  Every one computes identical bits (same leaf
// instruction, same lane assignment, same tree); they differ in tile shape and
// data movement only.
//   0: 128 x 64 tile, 8 waves of 32 x 32, general kernel (mfma_kernel.h)
//   1:  16 x 128 tile, 4 waves of 16 x 32   (few rows)
//   2:  64 x 64 tile, 4 waves of 32 x 32    (deep LDS stacks)
//   3: configuration 0 on the direct-to-LDS kernel (mfma_fast.h)
//   4: configuration 2 on the direct-to-LDS kernel
//   5: 128 x 128 tile, 8 waves of 64 x 32, wide kernel (mfma_wide.h), 2 stage
//      buffers, groups of 16 stages, power-of-two leaf counts
//   6: 128 x 64 tile, 4 waves of 64 x 32, wide kernel, 2 stage buffers (two
//      workgroups per compute unit)
//   7: configuration 5 for leaf counts 3 * 2^a (units of three leaves), groups
//      of 4 six-leaf nodes
//   8, 9: configurations 5 and 7 with three stage buffers and early copies
//  10: at most 16 rows of X: one 16 x 16 output block per workgroup, the
//      reduction split over 8 waves along the subtrees of depth 3
//      (mfma_decode.hip)
//  11: configuration 10 with 16 x 64 output tiles
//  12: configuration 10 with 16 x 32 output tiles
struct TileCfg {
    int fm, fn, wm, wn;
    int kind;
    int nbuf, gl, ru;  // wide kernel: stage buffers, static group levels, register levels
    int tb;            // wide kernel: leaves per unit (1 or odd)
    int ks;            // wide kernel: wave groups splitting the tree at its root (0 or 1: none, 2)
    int bm() const { return 16 * fm * wm; }
    int bn() const { return 16 * fn * wn; }
    int nw() const { return wm * wn; }
    bool fast() const { return kind != KIND_GENERAL; }
    // Must match Engine::lds_bytes / FastEngine::lds_bytes / WideEngine::lds_bytes.
    // `levels`: for the general and fast kernels the levels above the 8- or
    // 12-leaf blocks; for the wide kernel the levels above the groups of 2^gl
    // stages.
    int lds_bytes(int levels) const {
        const int park = fm * fn * nw() * 64 * 8;
        if (kind == KIND_WIDE)
            return (ks > 1 ? ks : 1) * (nbuf * (bm() + bn()) * 128 + (levels > ru ? levels - ru : 0) * park);
        const int parked = kind == KIND_FAST ? (levels > 1 ? levels - 1 : 0) : levels;
        return (kind == KIND_FAST ? 3 : 2) * (bm() + bn()) * 128 + parked * park;
    }
};
constexpr TileCfg kTileCfgs[] = {
    {2, 2, 4, 2, KIND_GENERAL, 0, 0, 0, 1}, {1, 2, 1, 4, KIND_GENERAL, 0, 0, 0, 1},
    {2, 2, 2, 2, KIND_GENERAL, 0, 0, 0, 1}, {2, 2, 4, 2, KIND_FAST, 0, 0, 0, 1},
    {2, 2, 2, 2, KIND_FAST, 0, 0, 0, 1},    {4, 2, 2, 4, KIND_WIDE, 2, 4, 1, 1},
    {4, 2, 2, 2, KIND_WIDE, 2, 3, 1, 1},    {4, 2, 2, 4, KIND_WIDE, 2, 2, 1, 3},
    {4, 2, 2, 4, KIND_WIDE, 3, 4, 1, 1},    {4, 2, 2, 4, KIND_WIDE, 3, 2, 1, 3},
    {1, 1, 1, 1, KIND_DECODE, 0, 0, 0, 1},  {1, 4, 1, 1, KIND_DECODE, 0, 0, 0, 1},
    {1, 2, 1, 1, KIND_DECODE, 0, 0, 0, 1},  {2, 2, 4, 1, KIND_WIDE, 4, 3, 2, 1, 2},
    {2, 1, 2, 2, KIND_WIDE, 6, 3, 2, 1, 2},  {2, 1, 2, 2, KIND_WIDE, 3, 3, 2, 1, 4},
    {2, 2, 2, 2, KIND_WIDE, 2, 3, 2, 1, 4}, {4, 2, 2, 4, KIND_WIDE, 2, 4, 2, 1},
    {4, 2, 2, 4, KIND_WIDE, 3, 3, 1, 5},    {4, 2, 2, 4, KIND_WIDE, 3, 2, 1, 7},
    {4, 2, 2, 4, KIND_WIDE, 2, 2, 1, 7},    {4, 2, 2, 4, KIND_WIDE, 3, 0, 1, 43},
    {4, 2, 2, 4, KIND_WIDE, 3, 0, 1, 27},   {4, 2, 2, 4, KIND_WIDE, 2, 0, 1, 27},
    {4, 2, 2, 4, KIND_WIDE, 3, 0, 1, 37},   {4, 2, 2, 4, KIND_WIDE, 3, 0, 1, 11},
    {4, 2, 2, 4, KIND_WIDE, 2, 0, 1, 17},   {4, 2, 2, 4, KIND_WIDE, 3, 0, 1, 19},
    {4, 2, 2, 4, KIND_WIDE, 2, 0, 1, 25},   {4, 2, 2, 4, KIND_WIDE, 3, 0, 1, 35}};
constexpr int kNumTileCfgs = 30;

struct TreeSel {
    int mode;  // TREE_BLOCK or TREE_STACK
    int tb;    // block base size b of the fast and general kernels (1 or 3)
    int tk;    // block = b * 2^tk leaves: 8 for b = 1, 12 for b = 3
};

// Launches one kernel instance.  The dynamic LDS limit of each instance is
// raised once to what its static LDS leaves of the 160 KB; a request beyond it
// returns hipErrorInvalidConfiguration without launching.
template <bool FAST, bool XK, bool YK, int OUT, int TREE, int TB, int TK, int FM, int FN, int WM,
          int WN>
hipError_t launch_one(const MfmaParams &p, int64_t tiles, hipStream_t st) {
    typedef typename std::conditional<FAST, FastEngine<XK, YK, FM, FN, WM, WN>,
                                      Engine<XK, YK, FM, FN, WM, WN>>::type E;
    void (*kernel)(MfmaParams);
    if constexpr (FAST)
        kernel = &mfma_fast_kernel<XK, YK, OUT, TB, TK, FM, FN, WM, WN>;
    else
        kernel = &mfma_kernel<XK, YK, OUT, TREE, TB, TK, FM, FN, WM, WN>;
    const void *fn = reinterpret_cast<const void *>(kernel);
    static int max_dynamic = -1;
    if (max_dynamic < 0) {
        hipFuncAttributes attr;
        hipError_t e = hipFuncGetAttributes(&attr, fn);
        if (e != hipSuccess)
            return e;
        const int room = kLdsMax - (int)attr.sharedSizeBytes;
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, room);
        if (e != hipSuccess)
            return e;
        max_dynamic = room;
    }
    const int lds = E::lds_bytes(p.levels);
    if (lds > max_dynamic)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kernel, dim3((unsigned)tiles), dim3(64 * WM * WN), lds, st, p);
    return hipGetLastError();
}

// Wide kernel: power-of-two leaf counts only (checked by the caller), never the
// leaf dump; p.levels holds the levels above the groups of 2^GL stages.
template <bool XK, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int TB, int GL,
          int RU, int OCC>
hipError_t launch_wide(const MfmaParams &p, int64_t tiles, hipStream_t st) {
    if constexpr (OUT == OUT_LEAVES) {
        return hipErrorInvalidValue;
    } else {
        typedef WideEngine<XK, YK, OUT, FM, FN, WM, WN, NBUF> E;
        void (*kernel)(MfmaParams) = &mfma_wide_kernel<XK, YK, OUT, FM, FN, WM, WN, NBUF, TB, GL, RU, OCC>;
        const void *fn = reinterpret_cast<const void *>(kernel);
        static int max_dynamic = -1;
        if (max_dynamic < 0) {
            hipFuncAttributes attr;
            hipError_t e = hipFuncGetAttributes(&attr, fn);
            if (e != hipSuccess)
                return e;
            const int room = kLdsMax - (int)attr.sharedSizeBytes;
            e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, room);
            if (e != hipSuccess)
                return e;
            max_dynamic = room;
        }
        const int lds = E::lds_bytes(p.levels > RU ? p.levels - RU : 0);
        if (lds > max_dynamic)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kernel, dim3((unsigned)tiles), dim3(64 * WM * WN), lds, st, p);
        return hipGetLastError();
    }
}

// K-split wide kernel (X K-major, row-major bf16 or fp32 output): KS wave
// groups per workgroup, p.levels counted in one group's subtree.
template <bool XK, bool YK, int OUT, int FM, int FN, int WM, int WN, int NBUF, int GL, int RU, int KS,
          int OCC>
hipError_t launch_wide_split(const MfmaParams &p, int64_t tiles, hipStream_t st) {
    if constexpr (!XK || (OUT != OUT_BF16 && OUT != OUT_F32)) {
        return hipErrorInvalidValue;
    } else {
        typedef WideEngine<true, YK, OUT, FM, FN, WM, WN, NBUF> E;
        void (*kernel)(MfmaParams) = &mfma_wide_split_kernel<YK, OUT, FM, FN, WM, WN, NBUF, GL, RU, KS, OCC>;
        const void *fn = reinterpret_cast<const void *>(kernel);
        static int max_dynamic = -1;
        if (max_dynamic < 0) {
            hipFuncAttributes attr;
            hipError_t e = hipFuncGetAttributes(&attr, fn);
            if (e != hipSuccess)
                return e;
            const int room = kLdsMax - (int)attr.sharedSizeBytes;
            e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, room);
            if (e != hipSuccess)
                return e;
            max_dynamic = room;
        }
        const int lds = KS * E::lds_bytes(p.levels > RU ? p.levels - RU : 0);
        if (lds > max_dynamic)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kernel, dim3((unsigned)tiles), dim3(64 * KS * WM * WN), lds, st, p);
        return hipGetLastError();
    }
}

// Grouped wide kernel (forward layout, bf16 out): one launch over the tiles of
// every row group of `g`; its LDS starts with the epilogue header (kEpiLds).
template <int FM, int FN, int WM, int WN, int NBUF, int TB, int GL, int RU, int OCC>
hipError_t launch_wide_grouped(const MfmaParams &p, const GroupTable &g, int64_t tiles,
                               hipStream_t st) {
    typedef WideEngine<true, false, OUT_BF16, FM, FN, WM, WN, NBUF> E;
    void (*kernel)(MfmaParams, GroupTable) =
        &mfma_wide_grouped_kernel<FM, FN, WM, WN, NBUF, TB, GL, RU, OCC>;
    const void *fn = reinterpret_cast<const void *>(kernel);
    static int max_dynamic = -1;
    if (max_dynamic < 0) {
        hipFuncAttributes attr;
        hipError_t e = hipFuncGetAttributes(&attr, fn);
        if (e != hipSuccess)
            return e;
        const int room = kLdsMax - (int)attr.sharedSizeBytes;
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, room);
        if (e != hipSuccess)
            return e;
        max_dynamic = room;
    }
    int lds = kEpiLds + E::lds_bytes(p.levels > RU ? p.levels - RU : 0);
    int64_t blocks = tiles;
    if (g.split_from < tiles) {
        // half-height tail tiles: two wave groups of four 64 x 32 waves
        typedef WideEngine<true, false, OUT_BF16, 4, 2, 1, 4, 3> H;
        if (TB != 1 || g.split_from < 0)
            return hipErrorInvalidValue;
        const int half = kEpiLds + 2 * H::lds_bytes(g.split_levels > RU ? g.split_levels - RU : 0);
        lds = half > lds ? half : lds;
        blocks = tiles + (tiles - g.split_from);
    }
    if (lds > max_dynamic)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * WM * WN), lds, st, p, g);
    return hipGetLastError();
}

template <bool FAST, bool XK, bool YK, int OUT, int FM, int FN, int WM, int WN>
hipError_t launch_trees(const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st) {
    if constexpr (FAST) {
        // block trees only, never the leaf dump (checked by the caller)
        if constexpr (OUT != OUT_LEAVES) {
            if (t.mode == TREE_BLOCK && t.tb == 1 && t.tk == 3)
                return launch_one<true, XK, YK, OUT, TREE_BLOCK, 1, 3, FM, FN, WM, WN>(p, tiles, st);
            if (t.mode == TREE_BLOCK && t.tb == 3 && t.tk == 2)
                return launch_one<true, XK, YK, OUT, TREE_BLOCK, 3, 2, FM, FN, WM, WN>(p, tiles, st);
        }
        return hipErrorInvalidValue;
    } else if constexpr (OUT == OUT_LEAVES) {
        return launch_one<false, XK, YK, OUT, TREE_STACK, 1, 0, FM, FN, WM, WN>(p, tiles, st);
    } else {
        if (t.mode == TREE_BLOCK) {
            if (t.tb == 1 && t.tk == 3)
                return launch_one<false, XK, YK, OUT, TREE_BLOCK, 1, 3, FM, FN, WM, WN>(p, tiles, st);
            if (t.tb == 3 && t.tk == 2)
                return launch_one<false, XK, YK, OUT, TREE_BLOCK, 3, 2, FM, FN, WM, WN>(p, tiles, st);
            return hipErrorInvalidValue;
        }
        return launch_one<false, XK, YK, OUT, TREE_STACK, 1, 0, FM, FN, WM, WN>(p, tiles, st);
    }
}

template <bool XK, bool YK, int OUT>
hipError_t launch_layout(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles,
                         hipStream_t st) {
    switch (cfg) {
    case 0:
        return launch_trees<false, XK, YK, OUT, 2, 2, 4, 2>(t, p, tiles, st);
    case 1:
        return launch_trees<false, XK, YK, OUT, 1, 2, 1, 4>(t, p, tiles, st);
    case 2:
        return launch_trees<false, XK, YK, OUT, 2, 2, 2, 2>(t, p, tiles, st);
    case 3:
        return launch_trees<true, XK, YK, OUT, 2, 2, 4, 2>(t, p, tiles, st);
    case 4:
        return launch_trees<true, XK, YK, OUT, 2, 2, 2, 2>(t, p, tiles, st);
    case 5:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 2, 1, 4, 1, 2>(p, tiles, st);
    case 6:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 2, 2, 1, 3, 1, 2>(p, tiles, st);
    case 7:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 2, 3, 2, 1, 2>(p, tiles, st);
    case 8:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 1, 4, 1, 2>(p, tiles, st);
    case 9:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 3, 2, 1, 2>(p, tiles, st);
    // 128x128 for trees deeper than configurations 5 and 8 park in the LDS
    // (1024 leaves): a second level of pending nodes in registers
    case 17:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 2, 1, 4, 2, 2>(p, tiles, st);
    // L = 5 * 2^a (K = 5120, 10240, 20480): units of five leaves, five stages
    // per pair of units
    case 18:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 5, 3, 1, 2>(p, tiles, st);
    // L = 7 * 2^a (K = 7168, 14336, 28672): units of seven leaves, seven
    // stages per pair of units; two stage buffers where the parked levels of
    // the deepest trees (L = 896) leave no room for three
    case 19:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 7, 2, 1, 2>(p, tiles, st);
    case 20:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 2, 7, 2, 1, 2>(p, tiles, st);
    // L = 43 * 2^a (K = 11008, 22016) and 27 * 2^a (K = 13824, 27648): the
    // unit trees walked with a stack of static register slots
    case 21:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 43, 0, 1, 2>(p, tiles, st);
    case 22:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 27, 0, 1, 2>(p, tiles, st);
    // 27-leaf units on two stage buffers, for the parked levels of L = 864
    // (K = 27648); 37-leaf units (K = 18944, L = 592)
    case 23:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 2, 27, 0, 1, 2>(p, tiles, st);
    case 24:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 37, 0, 1, 2>(p, tiles, st);
    // more odd unit sizes of common reduction lengths: 11 (K = 2816, 5632),
    // 17 (17408), 19 (4864, 9728), 25 (25600), 35 (8960); 17 and 25 on two
    // stage buffers, whose LDS holds the parked levels of L = 544 and 800
    case 25:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 11, 0, 1, 2>(p, tiles, st);
    case 26:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 2, 17, 0, 1, 2>(p, tiles, st);
    case 27:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 19, 0, 1, 2>(p, tiles, st);
    case 28:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 2, 25, 0, 1, 2>(p, tiles, st);
    case 29:
        return launch_wide<XK, YK, OUT, 4, 2, 2, 4, 3, 35, 0, 1, 2>(p, tiles, st);
    // Narrow tiles for 33 to 128 rows (X K-major, row-major output), the tree
    // split over wave groups (the stages per tile divided by their number):
    // 128x32 on 2 x 4 waves of 2 x 2 blocks with four stage buffers per group,
    // 64x32 on 2 x 4 waves of 2 x 1 blocks with six, and 64x32 on 4 x 4 waves
    // (four waves per SIMD) with three; 64x64 on 4 x 4 waves of 2 x 2 blocks
    // with two.
    case 13:
        return launch_wide_split<XK, YK, OUT, 2, 2, 4, 1, 4, 3, 2, 2, 2>(p, tiles, st);
    case 14:
        return launch_wide_split<XK, YK, OUT, 2, 1, 2, 2, 6, 3, 2, 2, 2>(p, tiles, st);
    case 15:
        return launch_wide_split<XK, YK, OUT, 2, 1, 2, 2, 3, 3, 2, 4, 4>(p, tiles, st);
    case 16:
        return launch_wide_split<XK, YK, OUT, 2, 2, 2, 2, 2, 3, 2, 4, 4>(p, tiles, st);
    default:
        return hipErrorInvalidValue;
    }
}

// Defined in mfma_<layout>.hip.
hipError_t launch_fwd_bf16(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st);
hipError_t launch_fwd_f32(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st);
hipError_t launch_kk_bf16(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st);
hipError_t launch_nn_bf16(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st);
hipError_t launch_nn_bf16t(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st);
hipError_t launch_leaves(int cfg, const TreeSel &t, const MfmaParams &p, int64_t tiles, hipStream_t st);
// Configurations 10, 11 and 12 (X K-major, at most 16 rows, bf16 or fp32
// output, cb = column blocks of 16 per workgroup: 1, 4 or 2); defined in
// mfma_decode.hip.
hipError_t launch_decode(const MfmaParams &p, bool yk, int out, int cb, hipStream_t st);
// Grouped forward (wide configurations 5, 7, 8, 9 only); defined in mfma_moe.hip.
hipError_t launch_moe_grouped(int cfg, const MfmaParams &p, const GroupTable &g, int64_t tiles,
                              hipStream_t st);

}  // namespace detgemm
