// C-ABI of the det_gemm library (declared in include/det_gemm.h): argument
// validation, the mapping of the six operations onto one contraction
// X(i, r) . Y(j, r), and kernel selection.
//
// Operation roles (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
// (det_gemm)", section "Ascend NPU backend", first bullet: backward reuses the
// forward kernel on transposed operands; db_transposed writes [N,K]):
//   op                  out[i][j]   X(i, r)        Y(j, r)        R
//   fwd, fwd_fp32       C[m][n]     A[m][k]  (K)   B[k][n]  (MN)  K
//   fwd_rhs_transposed  C[m][n]     A[m][k]  (K)   Bt[n][k] (K)   K
//   da                  dA[m][k]    dC[m][n] (K)   B[k][n]  (K)   N
//   db                  dB[k][n]    A[m][k]  (MN)  dC[m][n] (MN)  M
//   db_transposed       dBt[n][k] = the db value at (k, n), stored transposed
// (K) = the reduction index is contiguous in memory, (MN) = the row index is.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <vector>

#include "det_attention.h"
#include "det_gemm.h"
#include "det_moe.h"
#include "mfma_launch.h"
#include "strict_kernel.h"
#include "device_check.h"

using namespace detgemm;

namespace {

constexpr int64_t kMaxLd = DET_GEMM_MAX_LD;   // keeps buffer offsets of a tile below 2^31
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

enum Op { OP_FWD, OP_RHS_T, OP_FWD_F32, OP_DA, OP_DB, OP_DB_T, OP_LEAVES };

struct Mat {
    const void *p;
    int64_t rows, cols, ld;
    int elem;
};

struct Problem {
    const uint16_t *x;
    int64_t ldx;
    bool xk;
    const uint16_t *y;
    int64_t ldy;
    bool yk;
    void *c;
    int64_t ldc;
    int out;
    int64_t I, J, R;
};

bool mat_ok(const Mat &m) {
    if (m.rows == 0 || m.cols == 0)
        return true;
    if (!m.p || m.ld < m.cols || m.ld < 1 || m.ld > kMaxLd)
        return false;
    return true;
}

void mat_range(const Mat &m, uintptr_t &lo, uintptr_t &hi) {
    lo = reinterpret_cast<uintptr_t>(m.p);
    hi = lo + (uintptr_t)(((m.rows - 1) * m.ld + m.cols) * m.elem);
}

bool overlaps(const Mat &a, const Mat &b) {
    if (a.rows == 0 || a.cols == 0 || b.rows == 0 || b.cols == 0)
        return false;
    uintptr_t alo, ahi, blo, bhi;
    mat_range(a, alo, ahi);
    mat_range(b, blo, bhi);
    return alo < bhi && blo < ahi;
}

int g_force_config = -1;  // tile configuration pinned for inspection, -1 = automatic

}  // namespace

namespace detgemm {

// Once per device: the kernels are built for gfx950 only.
std::atomic<int> g_device_ok[64];

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return DET_GEMM_EHIP;
    if (dev < 0 || dev >= 64)
        return DET_GEMM_EHIP;
    int state = g_device_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return DET_GEMM_EHIP;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_ok[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? DET_GEMM_OK : DET_GEMM_EHIP;
}

// Compute units of the current device (read once per device); 0 if unknown.
std::atomic<int> g_device_cus[64];
int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int n = g_device_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0)
            n = 0;
        g_device_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace detgemm

namespace {

// ---- tree selection.  L = b * 2^a with b odd.  For b in {1, 3} the tree is a
// perfect binary tree of depth a - k over identical blocks of b * 2^k leaves,
// reduced by the static block evaluator; otherwise the LDS-stack walk is used.
TreeSel pick_tree(int L, int &levels) {
    int a = 0;
    while (((L >> a) & 1) == 0)
        ++a;
    const int b = L >> a;
    if (b == 1 && a >= 3) {
        levels = a - 3;
        return {TREE_BLOCK, 1, 3};
    }
    if (b == 3 && a >= 2) {
        levels = a - 2;
        return {TREE_BLOCK, 3, 2};
    }
    // Deepest LDS stack of the streaming post-order walk over [0, L).
    int top = 0, deepest = 0;
    for (int t = 0; t < L; ++t) {
        int lo = 0, hi = L, merges = 0;
        while (hi - lo > 1) {
            if (hi == t + 1)
                ++merges;
            const int mid = lo + (hi - lo) / 2;
            if (t < mid)
                hi = mid;
            else
                lo = mid;
        }
        top -= merges;
        if (t + 1 < L)
            ++top;
        deepest = top > deepest ? top : deepest;
    }
    levels = deepest;
    return {TREE_STACK, 1, 0};
}

bool aligned16(const void *p, int64_t ld) {
    return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && (ld % 8) == 0;
}

// The direct-to-LDS kernels take whole 64-index stages, 16-byte aligned rows
// and, for an operand whose row index is contiguous, whole 8-row chunks.
bool staged_ok(const Problem &pr) {
    return pr.out != OUT_LEAVES && pr.R % 64 == 0 && aligned16(pr.x, pr.ldx) &&
           aligned16(pr.y, pr.ldy) && (pr.xk || pr.I % 8 == 0) && (pr.yk || pr.J % 8 == 0);
}

bool fast_ok(const Problem &pr, const TreeSel &t) { return t.mode == TREE_BLOCK && staged_ok(pr); }

// The wide kernel: the fast kernel's operand conditions and a leaf count
// L = 2 * tb * 2^k (tb = 1, 3, 5, 7, 11, 17, 19, 25, 27, 35, 37 or 43: the mid-split tree is the perfect tree
// over units of tb leaves) with at least one group of 2^gl nodes of 2 * tb leaves
// (with exactly one group, the group root is the root); a tree split at its
// root over two or four wave groups needs units of one leaf, a K-major X, a
// row-major output and a group of stages in each part.  `up` receives the
// levels above the groups (of one part for a split tree).
bool wide_ok(const Problem &pr, const TreeSel &t, const TileCfg &c, int &up) {
    const int64_t L = (pr.R + 31) / 32;
    const bool split = c.ks > 1;
    if (!staged_ok(pr) || L % (2 * c.tb) != 0 ||
        (split && (!pr.xk || c.tb != 1 || pr.out == OUT_BF16_T)))
        return false;
    const int64_t S = L / (2 * c.tb), G = int64_t(1) << c.gl;  // nodes of 2 * tb leaves
    const int64_t SG = split ? S / c.ks : S;                   // stages of one wave group
    if ((S & (S - 1)) != 0 || SG < G)
        return false;
    up = 0;
    while ((G << up) < SG)
        ++up;
    return c.lds_bytes(up) <= kLdsMax;  // the wide kernels use no static LDS
}

// The decode kernels (configurations 10 to 12): X K-major with at most 128
// rows (at most 64 on 32-column tiles, 16 on 64-column tiles), bf16 or fp32
// output, whole leaves, at
// least 8 and at most 1024 of them (one leaf or more per wave, at most 8
// pending left siblings per wave), 16-byte aligned rows and, for a [K][N]
// operand Y, whole 8-column chunks.
bool decode_ok(const Problem &pr) {
    const int64_t L = pr.R / 32;
    return pr.xk && (pr.out == OUT_BF16 || pr.out == OUT_F32) && pr.I >= 1 && pr.I <= 128 &&
           pr.R % 32 == 0 && L >= 8 && L <= 1024 && aligned16(pr.x, pr.ldx) &&
           aligned16(pr.y, pr.ldy) && (pr.yk || pr.J % 8 == 0);
}

// Selection (measured on MI355X; every configuration gives the same bits).
// At most 16 rows: the decode kernel, whose workgroups split the reduction
// along the tree.  Wider tiles read more of each cache line they request (a
// compute unit keeps a bounded number of line requests in flight), narrower
// ones spread over more compute units: 64 columns once there are more than
// 128 such tiles, 32 columns above 128 such tiles, else 16 (M = 1, K = 4096:
// N = 6144 13.9 us on 32 columns, 19.9 on 16; N = 11008 17.5 us on 64
// columns, 23.9 on 32; N = 151936 215 us on 64 columns, 246 on 32;
// K = 32768, N = 4096 85 us on 16 columns, 94 on 32).  A K-major Y with an
// even leaf count is read in whole lines at any width and stays on 16 or 32
// columns (N = 151936: 202 us on 32 columns, 242 on 64).  17 to 64 rows: the
// decode kernel stages 2 to 4 blocks of 16 rows per tile and re-reads X once
// per tile, so it wins while the 32-column tiles times the row blocks stay
// under about 1400 (M = 32, K = 4096, N = 6144: 16.7 us instead of 40 on the
// wide kernel; N = 18432: 46 us instead of 51), or 600 for 65 to 128 rows on
// 16-column tiles (M = 128, N = 2048: 20 us; N = 6144: 48 us instead of 40 on
// the wide kernel).  Before those, 33 to 128 rows go to the 32-column wide
// tiles with the tree split at its root over two wave groups, 64x32 while
// they fit one round over the compute units (K = 4096: M = 128, N = 2048
// 17 us instead of 20 on the decode kernel; M = 64, N = 6144 19 us instead of
// 21), else 128x32 (M = 128, N = 6144: 24 us instead of 40 on the wide
// kernel); up to 64 rows the decode kernel keeps at most 128 and more than
// 192 column tiles (M = 64, N = 2048: 13 us, 17 on 64x32; N = 8192: 22.5 us,
// 23.3 on 64x32).  A K-major Y (whole 128-byte lines
// per column and stage) takes 64x32 tiles on four wave groups instead, at
// any column count that fits one round (M = 64, N = 6144: 14.1 us instead of
// 16.3; M = 128, N = 2048: 12.9 instead of 15.8), as do 17 to 32 rows of it
// with 129 to 256 column tiles (M = 32, N = 6144: 13.6 us instead of 15.0 on
// the decode kernel; at most 16 rows, or at most 128 column tiles, the decode
// kernel stays faster), and 65 to 128 rows of a
// [K][N] weight with 129 to 256 column tiles take 64x64 tiles on four wave
// groups, whose weight copies are whole lines (M = 128, N = 6144: 22.8 us
// instead of 24.1 on 128x32; N = 8192: 23.0 instead of 25.8).  First of all,
// 17 to 64 rows (33 to 64 of a K-major Y) with 129 to 256 column tiles of 64
// take 64x64 tiles on four wave groups (K = 4096, N = 9216 .. 16384: 23 to
// 27 us instead of 30 to 40; more tiles than one round lost with the weight
// in HBM).  A [K][N] Y on 32-column split tiles reads half lines, whose other
// halves the split kernel's XCD pairing turns into L2 hits, so it takes the
// 64x32 tiles at 129 to 256 column tiles too (M = 48, N = 8192: 17.7 us
// instead of 22.5 on the decode kernel), and above 192 of them from 17 rows
// on four wave groups (M = 32: 16.5 instead of 17.0).  Otherwise the
// wide kernel
// (N = 28672: 54 us instead of 65 at M = 32, 54 instead of 83 at M = 64),
// on 128x128 tiles above 128 column tiles (N = 18432, M = 64: 51 us, 55 on
// 128x64).  Otherwise 128x128 wide tiles when they make at least two waves
// of workgroups over the 256 compute units (M = 2048, N = 4096, K = 4096:
// 539 TFLOP/s instead of 473 on 128x64), else the 128x64 wide kernel, two
// workgroups per compute unit, which keeps more units busy on small and
// mid-size products (M = 1024 at K = 4096, N = 6144: 94 us instead of 111 us)
// -- but from 256 leaves its parked tree levels leave LDS for one workgroup
// per unit, and beyond one round of its tiles the 128x128 tiles win (K = 8192,
// M = 1024, N = 4096: 553 TFLOP/s instead of 388).
int pick_config(const Problem &pr, const TreeSel &t, int levels) {
    if (g_force_config >= 0)
        return g_force_config;
    int up = 0;
    if (decode_ok(pr)) {
        const int64_t t32 = (pr.J + 31) / 32, blocks = (pr.I + 15) / 16;
        // 17 to 64 rows (33 to 64 of a K-major Y) with 129 to 256 tiles of
        // 64x64: those tiles on four wave groups, one round over the compute
        // units
        const int64_t t64x64 = (pr.J + 63) / 64;
        if (pr.I > (pr.yk ? 32 : 16) && pr.I <= 64 && t64x64 > 128 && t64x64 <= 256 &&
            wide_ok(pr, t, kTileCfgs[16], up))
            return 16;
        // 33 to 128 rows: the narrow wide tiles that split the tree over
        // wave groups, while their tiles make at most one round over the
        // compute units (and, up to 64 rows of a [K][N] weight, while the
        // decode kernel has 129 to 192 column tiles)
        // 17 to 32 rows of a K-major Y with 129 to 256 column tiles: the
        // 64x32 tiles on four wave groups (the decode kernel's two row blocks
        // wait on longer chains)
        if (pr.I > 16 && pr.I <= 32 && t32 > (pr.yk ? 128 : 192) && t32 <= 256 &&
            wide_ok(pr, t, kTileCfgs[15], up))
            return 15;
        if (pr.I > 32) {
            const int64_t t64 = (pr.I + 63) / 64 * t32, t128 = (pr.I + 127) / 128 * t32;
            if (pr.yk && t64 <= 256 && wide_ok(pr, t, kTileCfgs[15], up))
                return 15;
            if (t64 <= 256 && (pr.I > 64 || t32 > 128) && wide_ok(pr, t, kTileCfgs[14], up))
                return 14;
            // 65 to 128 rows of a [K][N] weight with 129 to 256 column tiles:
            // 64x64 tiles on four wave groups read whole 128-byte weight lines
            if (pr.I > 64 && !pr.yk && t32 > 128 && t32 <= 256 &&
                (pr.I + 63) / 64 * ((pr.J + 63) / 64) <= 256 && wide_ok(pr, t, kTileCfgs[16], up))
                return 16;
            if (pr.I > 64 && t128 <= 256 && wide_ok(pr, t, kTileCfgs[13], up))
                return 13;
        }
        const bool line_units = pr.yk && (pr.R / 32) % 2 == 0;  // two-leaf copies read whole lines
        // A K-major weight read in whole lines keeps up to 32 rows on the
        // decode kernel at any width (its copies of a weight larger than the
        // Infinity Cache are non-temporal): N = 151936, M = 32: 279 us
        // instead of 306 on the wide kernel; N = 40960, M = 17: 73 instead
        // of 109; N = 28672: equal.
        const bool decode_lines = line_units && pr.I <= 32;
        if (!decode_lines &&
            ((pr.I > 16 && t32 * blocks > 1400) || (pr.I > 64 && t32 * blocks > 600))) {
            const int first = (pr.J + 127) / 128 > 128 ? 8 : 6;
            for (int c : {first, first == 8 ? 6 : 8})
                if (wide_ok(pr, t, kTileCfgs[c], up))
                    return c;
        }
        if (pr.I > 64)
            return 10;  // eight row blocks: 16-column tiles only
        if (!line_units && pr.I <= 16 && (pr.J + 63) / 64 > 128)
            return 11;
        return t32 > 128 ? 12 : 10;
    }
    const int64_t t128 = ((pr.I + 127) / 128) * ((pr.J + 127) / 128);
    if (t128 >= 2 * 256)
        for (int c : {8, 5, 9, 7, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29})  // three stage buffers with early copies if the LDS holds them
            if (wide_ok(pr, t, kTileCfgs[c], up))
                return c;
    // 128x64 tiles while they fit one round, or two workgroups per compute
    // unit: from 256 leaves their parked tree levels leave LDS for one, and
    // four waves per unit ran 30 % below the 128x128 tiles
    if (wide_ok(pr, t, kTileCfgs[6], up) &&
        (2 * t128 <= 256 || 2 * kTileCfgs[6].lds_bytes(up) <= kLdsMax))
        return 6;
    // deeper trees than configurations 5 and 8 hold: 128x128 tiles with a
    // second register level (K = 32768, M = 2048, N = 4096: 420 TFLOP/s
    // instead of 355 on 128x64; at 512 leaves and fewer it loses to them)
    for (int c : {8, 5, 9, 7, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29})
        if (wide_ok(pr, t, kTileCfgs[c], up))
            return c;
    if (wide_ok(pr, t, kTileCfgs[6], up))
        return 6;
    if (pr.I <= 16)
        return 1;
    // 8-wave 128x64 tiles for blocks of 8 leaves; the 4-wave 64x64 tile (twice
    // the registers per wave) for blocks of 12 and for the LDS stack.
    const bool wide = t.mode == TREE_BLOCK && t.tb == 1;
    if (fast_ok(pr, t)) {
        if (wide && kTileCfgs[3].lds_bytes(levels) <= kLdsMax - 1024)
            return 3;
        if (kTileCfgs[4].lds_bytes(levels) <= kLdsMax - 1024)
            return 4;
    }
    if (wide && kTileCfgs[0].lds_bytes(levels) <= kLdsMax - 1024)
        return 0;
    return 2;
}

int run_mfma(const Problem &pr, hipStream_t st) {
    MfmaParams p;
    std::memset(&p, 0, sizeof p);
    p.x = pr.x;
    p.ldx = pr.ldx;
    p.y = pr.y;
    p.ldy = pr.ldy;
    p.c = pr.c;
    p.ldc = pr.ldc;
    p.I = (int32_t)pr.I;
    p.J = (int32_t)pr.J;
    p.R = (int32_t)pr.R;
    p.L = (int32_t)((pr.R + 31) / 32);
    int levels = 0;
    const TreeSel tree = pick_tree(p.L, levels);
    p.levels = levels;
    const int cfg = pick_config(pr, tree, levels);
    const TileCfg &c = kTileCfgs[cfg];
    if (c.kind == KIND_DECODE) {
        if (!decode_ok(pr) || (c.fn == 4 && pr.I > 16) || (c.fn == 2 && pr.I > 64))
            return DET_GEMM_EINVAL;  // a forced decode configuration this problem does not fit
        if ((pr.J + 15) / 16 > kMaxDim)
            return DET_GEMM_EINVAL;
        // A weight larger than the 256 MB Infinity Cache cannot stay there
        // from one call to the next: its copies are non-temporal when each
        // workgroup reads whole cache lines of it (a K-major Y, or 64-column
        // tiles of a [K][N] Y).  Measured on the LM head (K = 4096,
        // N = 151936): 188 us instead of 213 at M = 1.  A weight the cache
        // holds keeps its copies cacheable (QKV, [K][N]: 13.7 us instead of
        // 18.0).  Bits do not depend on it.
        p.ynt = (pr.yk || c.fn == 4) && pr.J * pr.R * 2 > (int64_t(256) << 20) ? 1 : 0;
        const hipError_t e = launch_decode(p, pr.yk, pr.out, c.fn, st);
        return e == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
    }
    if (c.kind == KIND_WIDE) {
        int up = 0;
        if (!wide_ok(pr, tree, c, up))
            return DET_GEMM_EINVAL;  // a forced wide configuration this problem does not fit
        p.levels = up;
    } else if (c.fast() && !fast_ok(pr, tree)) {
        return DET_GEMM_EINVAL;  // a forced fast configuration this problem does not fit
    }
    const int64_t tiles_i = (pr.I + c.bm() - 1) / c.bm();
    const int64_t tiles_j = (pr.J + c.bn() - 1) / c.bn();
    if (tiles_i * tiles_j > kMaxDim)
        return DET_GEMM_EINVAL;
    p.tiles_j = (int32_t)tiles_j;
    p.xvec = aligned16(pr.x, pr.ldx);
    p.yvec = aligned16(pr.y, pr.ldy);
    p.cvec = pr.out != OUT_F32 && aligned16(pr.c, pr.ldc);
    const int64_t tiles = tiles_i * tiles_j;

    hipError_t e;
    if (pr.out == OUT_LEAVES) {
        p.levels = 0;
        e = launch_leaves(cfg, tree, p, tiles, st);
    } else if (pr.xk && !pr.yk && pr.out == OUT_BF16)
        e = launch_fwd_bf16(cfg, tree, p, tiles, st);
    else if (pr.xk && !pr.yk && pr.out == OUT_F32)
        e = launch_fwd_f32(cfg, tree, p, tiles, st);
    else if (pr.xk && pr.yk && pr.out == OUT_BF16)
        e = launch_kk_bf16(cfg, tree, p, tiles, st);
    else if (!pr.xk && !pr.yk && pr.out == OUT_BF16)
        e = launch_nn_bf16(cfg, tree, p, tiles, st);
    else if (!pr.xk && !pr.yk && pr.out == OUT_BF16_T)
        e = launch_nn_bf16t(cfg, tree, p, tiles, st);
    else
        return DET_GEMM_EINVAL;
    if (e == hipErrorInvalidConfiguration)
        return DET_GEMM_EINVAL;  // a forced configuration without LDS room for this tree
    return e == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

int run_strict(const Problem &pr, hipStream_t st) {
    StrictParams p;
    p.x = pr.x;
    p.sxi = pr.xk ? pr.ldx : 1;
    p.sxr = pr.xk ? 1 : pr.ldx;
    p.y = pr.y;
    p.syj = pr.yk ? pr.ldy : 1;
    p.syr = pr.yk ? 1 : pr.ldy;
    p.c = pr.c;
    if (pr.out == OUT_BF16_T) {
        p.sci = 1;
        p.scj = pr.ldc;
    } else {
        p.sci = pr.ldc;
        p.scj = 1;
    }
    p.I = pr.I;
    p.J = pr.J;
    p.R = pr.R;
    p.L = (int32_t)((pr.R + 31) / 32);
    const int64_t ti = (pr.I + kStrictTile - 1) / kStrictTile;
    const int64_t tj = (pr.J + kStrictTile - 1) / kStrictTile;
    if (ti * tj > kMaxDim || tj > kMaxDim)
        return DET_GEMM_EINVAL;
    p.tiles_j = (int32_t)tj;
    const dim3 grid((unsigned)(ti * tj)), block(256);
    if (pr.out == OUT_F32)
        hipLaunchKernelGGL(strict_kernel<true>, grid, block, 0, st, p);
    else
        hipLaunchKernelGGL(strict_kernel<false>, grid, block, 0, st, p);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

// Validates the operands of `op` and builds the contraction.  Returns
// DET_GEMM_OK with *empty set when there is nothing to do.
int build(Op op, const void *P, int64_t ldp, const void *Q, int64_t ldq, void *Out, int64_t ldo,
          int64_t M, int64_t N, int64_t K, Problem &pr, bool &empty) {
    empty = false;
    if (M < 0 || N < 0 || K < 0)
        return DET_GEMM_EINVAL;
    Mat in1, in2, out;
    const uint16_t *p16 = static_cast<const uint16_t *>(P);
    const uint16_t *q16 = static_cast<const uint16_t *>(Q);
    switch (op) {
    case OP_FWD:
    case OP_FWD_F32:
    case OP_LEAVES:
        in1 = {P, M, K, ldp, 2};
        in2 = {Q, K, N, ldq, 2};
        out = {Out, M, op == OP_LEAVES ? N * ((K + 31) / 32) : N,
               op == OP_LEAVES ? N * ((K + 31) / 32) : ldo, op == OP_FWD_F32 ? 4 : 2};
        pr = {p16, ldp, true, q16, ldq, false, Out, ldo,
              op == OP_FWD ? OUT_BF16 : (op == OP_FWD_F32 ? OUT_F32 : OUT_LEAVES), M, N, K};
        break;
    case OP_RHS_T:
        in1 = {P, M, K, ldp, 2};
        in2 = {Q, N, K, ldq, 2};
        out = {Out, M, N, ldo, 2};
        pr = {p16, ldp, true, q16, ldq, true, Out, ldo, OUT_BF16, M, N, K};
        break;
    case OP_DA:  // P = dC [M,N], Q = B [K,N], Out = dA [M,K]
        in1 = {P, M, N, ldp, 2};
        in2 = {Q, K, N, ldq, 2};
        out = {Out, M, K, ldo, 2};
        pr = {p16, ldp, true, q16, ldq, true, Out, ldo, OUT_BF16, M, K, N};
        break;
    case OP_DB:    // P = A [M,K], Q = dC [M,N], Out = dB [K,N]
    case OP_DB_T:  // Out = dBt [N,K]
        in1 = {P, M, K, ldp, 2};
        in2 = {Q, M, N, ldq, 2};
        out = op == OP_DB ? Mat{Out, K, N, ldo, 2} : Mat{Out, N, K, ldo, 2};
        pr = {p16, ldp, false, q16, ldq, false, Out, ldo, op == OP_DB ? OUT_BF16 : OUT_BF16_T,
              K, N, M};
        break;
    }
    if (pr.I == 0 || pr.J == 0) {
        empty = true;
        return DET_GEMM_OK;
    }
    if (pr.R == 0 || pr.R > DET_GEMM_MAX_REDUCTION)
        return DET_GEMM_EKCAP;
    if (pr.I > kMaxDim || pr.J > kMaxDim)
        return DET_GEMM_EINVAL;
    if (!mat_ok(in1) || !mat_ok(in2) || !mat_ok(out))
        return DET_GEMM_EINVAL;
    if (overlaps(out, in1) || overlaps(out, in2))
        return DET_GEMM_EINVAL;
    return DET_GEMM_OK;
}

int entry(Op op, bool strict, const void *P, int64_t ldp, const void *Q, int64_t ldq, void *Out,
          int64_t ldo, int64_t M, int64_t N, int64_t K, void *stream) {
    Problem pr;
    bool empty;
    const int rc = build(op, P, ldp, Q, ldq, Out, ldo, M, N, K, pr, empty);
    if (rc != DET_GEMM_OK || empty)
        return rc;
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return strict ? run_strict(pr, st) : run_mfma(pr, st);
}

// ---- element-wise inspection kernels
__global__ void debug_round_kernel(const float *x, uint16_t *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        out[i] = (uint16_t)pair_bits(round_pair(x[i], 0.0f));
}

__global__ void debug_add_kernel(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const float l = __uint_as_float((uint32_t)a[i] << 16);
        const float r = __uint_as_float((uint32_t)b[i] << 16);
        out[i] = (uint16_t)pair_bits(round_pair(merge(l, r), 0.0f));
    }
}

// Issue-rate probe (inspection): the instruction mix of one pipeline stage of
// the 128x128 wide kernel without any memory traffic.  Per wave and
// iteration, four rounds of 8 independent v_mfma_f32_16x16x32_bf16 whose
// results are each rounded to bf16 by two v_cvt_pk_bf16_f32 and fed back as
// the next round's A operand (a tree add consumes its children rounded):
// 32 MFMAs and 64 conversions, the per-stage counts of a wave of that kernel.
// MODE 0: the MFMAs alone (accumulating chains); 1: both, dependent as above.
// 512 threads per workgroup (two waves per SIMD, as the wide kernel).  Values
// stay bounded (B holds 1/32); each thread writes one float of `sink`.
template <int MODE>
__global__ __launch_bounds__(512) void issue_probe_kernel(float *sink, int iters) {
    const int lane = threadIdx.x & 63;
    const uint32_t one32 = 0x3D003D00u;  // bf16 1/32, twice
    const u32x4 bw = {one32, one32, one32, one32};
    const bf16x8 B = __builtin_bit_cast(bf16x8, bw);
    const u32x4 bw1 = {one32, 0u, one32, 0u};   // a second weight: different products
    const bf16x8 B1 = __builtin_bit_cast(bf16x8, bw1);
    u32x4 A[8];
    f32x4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t w = 0x3F803F80u + (uint32_t)((lane + k) & 7);
        A[k] = u32x4{w, w, w, w};
        acc[k] = f32x4{1.0f + k, 1.0f, 1.0f, (float)lane};
    }
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (MODE == 0) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[k]), B,
                                                                     acc[k], 0, 0, 0);
            } else {
                // A of MFMAs 2q and 2q + 1: the rounded results of the previous
                // round's MFMAs 2q and 2q + 1 (as a tree add's two children)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[k >> 1]),
                                                                     (k & 1) ? B1 : B, zero, 0, 0, 0);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    A[q] = u32x4{pair_bits(round_pair(acc[2 * q][0], acc[2 * q][1])),
                                 pair_bits(round_pair(acc[2 * q][2], acc[2 * q][3])),
                                 pair_bits(round_pair(acc[2 * q + 1][0], acc[2 * q + 1][1])),
                                 pair_bits(round_pair(acc[2 * q + 1][2], acc[2 * q + 1][3]))};
            }
        }
    }
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3] + __uint_as_float(A[k][0] & 0x3FFFFFFFu);
    sink[(int64_t)blockIdx.x * 512 + threadIdx.x] = v;
}

// The tree add as the matrix-core kernels run it.  Blocks of 256 pairs, one
// wave per block: pair k of a block sits at block position (k / 16, k % 16) of
// both children, i.e. in the lane and register where an MFMA result holds that
// position (lane 16g + c, register v for position (4g + v, c)); the two
// children are added by one v_mfma_f32_16x16x32_bf16 against a 0/1 selector,
// exactly the code of the tree steps:
//   selector 0: WideMatrixAdd with split_selector (the wide and direct-to-LDS
//               kernels: each child packed on its own),
//   selector 1: MatrixAdd with add_selector (the general kernel: the children
//               packed pairwise by v_cvt_pk).
// The add moves each sum to the lane and register that the transposed (odd
// parity) layout uses for the same block position, which is how the store
// reads it back.  A block with a non-finite sum is redone with element-wise
// fp32 adds (positions unchanged), as a tile with a non-finite root is.  The
// result is rounded to bf16 by v_cvt_pk, as a node is before its parent's add.
__global__ __launch_bounds__(256) void debug_matrix_add_kernel(const uint16_t *a, const uint16_t *b,
                                                               uint16_t *out, int64_t n,
                                                               int selector) {
    const int lane = threadIdx.x & 63;
    const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 256;
    if (base >= n)
        return;  // the whole wave
    const int g = lane >> 4, c = lane & 15;
    uint32_t av[4], bv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t i = base + (4 * g + v) * 16 + c;
        av[v] = i < n ? a[i] : 0u;
        bv[v] = i < n ? b[i] : 0u;
    }
    WPacked<1, 1> l, r;
    l.w[0][0] = u32x2{av[0] | (av[1] << 16), av[2] | (av[3] << 16)};
    r.w[0][0] = u32x2{bv[0] | (bv[1] << 16), bv[2] | (bv[3] << 16)};
    Frag<1, 1> s;
    if (selector == 0) {
        s = WideMatrixAdd::add<1, 1>(l, r, split_selector(lane));
    } else {
        Frag<1, 1> lf, rf;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            lf.v[0][0][v] = __uint_as_float(av[v] << 16);
            rf.v[0][0][v] = __uint_as_float(bv[v] << 16);
        }
        s = MatrixAdd::merge<1, 1>(lf, rf, add_selector(lane));
    }
    bool bad = false;
#pragma unroll
    for (int v = 0; v < 4; ++v)
        bad |= !(__builtin_fabsf(s.v[0][0][v]) <= 3.40282347e38f);
    const bool redo = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (redo)
        s = WideValuAdd::add<1, 1>(l, r, bf16x8{});
    const WPacked<1, 1> q = wpack(s);
    const uint32_t w[2] = {q.w[0][0].x, q.w[0][0].y};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        // odd parity: lane (g, c) register v holds position (c, 4g + v);
        // element-wise adds keep the even parity (4g + v, c)
        const int k = redo ? (4 * g + v) * 16 + c : c * 16 + 4 * g + v;
        if (base + k < n)
            out[base + k] = (uint16_t)(w[v >> 1] >> (16 * (v & 1)));
    }
}

// ---- combination of K-shard partials: each thread takes 8 consecutive
// columns of one row (16-byte loads when aligned) and evaluates the mid-split
// tree over the parts, unrolled at compile time for each part count.
struct Parts {
    const uint16_t *p[DET_GEMM_MAX_PARTS];
};

template <int LO, int HI>
__device__ __forceinline__ float tree_of_parts(const float (&v)[DET_GEMM_MAX_PARTS]) {
    if constexpr (HI - LO == 1) {
        return v[LO];
    } else {
        constexpr int MID = LO + (HI - LO) / 2;
        const float l = tree_of_parts<LO, MID>(v), r = tree_of_parts<MID, HI>(v);
        // the bf16 add: fp32 sum of the two bf16 values, rounded to bf16 (kept in fp32)
        const uint32_t b = pair_bits(round_pair(merge(l, r), 0.0f)) & 0xFFFFu;
        return __uint_as_float(b << 16);
    }
}

template <int NP>
__global__ __launch_bounds__(256) void shard_reduce_kernel(Parts parts, int64_t ldp, uint16_t *out,
                                                           int64_t ldo, int64_t M, int64_t N,
                                                           int64_t chunks_per_row, bool vec) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= M * chunks_per_row)
        return;
    const int64_t r = q / chunks_per_row, c0 = (q % chunks_per_row) * 8;
    const int n = N - c0 < 8 ? (int)(N - c0) : 8;
    uint16_t vals[NP][8];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const uint16_t *src = parts.p[k] + r * ldp + c0;
        if (vec && n == 8) {
            // each part and the output are touched once: non-temporal
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
            const uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vals[k][e] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
        } else {
            for (int e = 0; e < 8; ++e)
                vals[k][e] = e < n ? src[e] : (uint16_t)0;
        }
    }
    uint16_t res[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float v[DET_GEMM_MAX_PARTS];
#pragma unroll
        for (int k = 0; k < DET_GEMM_MAX_PARTS; ++k)
            v[k] = k < NP ? __uint_as_float((uint32_t)vals[k < NP ? k : 0][e] << 16) : 0.0f;
        res[e] = (uint16_t)(__float_as_uint(tree_of_parts<0, NP>(v)) >> 16);
    }
    uint16_t *dst = out + r * ldo + c0;
    if (vec && n == 8) {
        const u32x4 o = {res[0] | ((uint32_t)res[1] << 16), res[2] | ((uint32_t)res[3] << 16),
                         res[4] | ((uint32_t)res[5] << 16), res[6] | ((uint32_t)res[7] << 16)};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(dst));
    } else {
        for (int e = 0; e < n; ++e)
            dst[e] = res[e];
    }
}

template <int NP>
hipError_t launch_shard_reduce(const Parts &parts, int64_t ldp, uint16_t *out, int64_t ldo,
                               int64_t M, int64_t N, bool vec, hipStream_t st) {
    const int64_t cpr = (N + 7) / 8, blocks = (M * cpr + 255) / 256;
    hipLaunchKernelGGL(shard_reduce_kernel<NP>, dim3((unsigned)blocks), dim3(256), 0, st, parts,
                       ldp, out, ldo, M, N, cpr, vec);
    return hipGetLastError();
}

template <int NP>
hipError_t dispatch_shard_reduce(int n, const Parts &parts, int64_t ldp, uint16_t *out,
                                 int64_t ldo, int64_t M, int64_t N, bool vec, hipStream_t st) {
    if constexpr (NP > DET_GEMM_MAX_PARTS) {
        return hipErrorInvalidValue;
    } else {
        if (n == NP)
            return launch_shard_reduce<NP>(parts, ldp, out, ldo, M, N, vec, st);
        return dispatch_shard_reduce<NP + 1>(n, parts, ldp, out, ldo, M, N, vec, st);
    }
}

}  // namespace

extern "C" {

int det_gemm_shard_reduce(const det_bf16 *const *parts, int64_t nparts, int64_t ldp,
                          det_bf16 *out, int64_t ldo, int64_t M, int64_t N, void *stream) {
    if (M < 0 || N < 0 || nparts < 1 || nparts > DET_GEMM_MAX_PARTS || !parts)
        return DET_GEMM_EINVAL;
    if (M == 0 || N == 0)
        return DET_GEMM_OK;
    if (M > kMaxDim || N > kMaxDim || (M * ((N + 7) / 8) + 255) / 256 > kMaxDim)
        return DET_GEMM_EINVAL;
    const Mat om{out, M, N, ldo, 2};
    if (!mat_ok(om))
        return DET_GEMM_EINVAL;
    Parts ps;
    std::memset(&ps, 0, sizeof ps);
    bool vec = aligned16(out, ldo);
    for (int64_t k = 0; k < nparts; ++k) {
        const Mat pm{parts[k], M, N, ldp, 2};
        if (!mat_ok(pm) || overlaps(om, pm))
            return DET_GEMM_EINVAL;
        ps.p[k] = parts[k];
        vec = vec && aligned16(parts[k], ldp);
    }
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    const hipError_t e = dispatch_shard_reduce<1>((int)nparts, ps, ldp, out, ldo, M, N, vec,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

int det_gemm_fwd(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb, det_bf16 *C,
                 int64_t ldc, int64_t M, int64_t N, int64_t K, void *stream) {
    return entry(OP_FWD, false, A, lda, B, ldb, C, ldc, M, N, K, stream);
}

int det_gemm_fwd_rhs_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *Bt, int64_t ldbt,
                                det_bf16 *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                void *stream) {
    return entry(OP_RHS_T, false, A, lda, Bt, ldbt, C, ldc, M, N, K, stream);
}

int det_gemm_fwd_fp32(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb, float *C,
                      int64_t ldc, int64_t M, int64_t N, int64_t K, void *stream) {
    return entry(OP_FWD_F32, false, A, lda, B, ldb, C, ldc, M, N, K, stream);
}

int det_gemm_da(const det_bf16 *dC, int64_t lddc, const det_bf16 *B, int64_t ldb, det_bf16 *dA,
                int64_t ldda, int64_t M, int64_t N, int64_t K, void *stream) {
    return entry(OP_DA, false, dC, lddc, B, ldb, dA, ldda, M, N, K, stream);
}

int det_gemm_db(const det_bf16 *A, int64_t lda, const det_bf16 *dC, int64_t lddc, det_bf16 *dB,
                int64_t lddb, int64_t M, int64_t N, int64_t K, void *stream) {
    return entry(OP_DB, false, A, lda, dC, lddc, dB, lddb, M, N, K, stream);
}

int det_gemm_db_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *dC, int64_t lddc,
                           det_bf16 *dBt, int64_t lddbt, int64_t M, int64_t N, int64_t K,
                           void *stream) {
    return entry(OP_DB_T, false, A, lda, dC, lddc, dBt, lddbt, M, N, K, stream);
}

int det_gemm_strict_fwd(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                        det_bf16 *C, int64_t ldc, int64_t M, int64_t N, int64_t K, void *stream) {
    return entry(OP_FWD, true, A, lda, B, ldb, C, ldc, M, N, K, stream);
}

int det_gemm_strict_fwd_rhs_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *Bt,
                                       int64_t ldbt, det_bf16 *C, int64_t ldc, int64_t M,
                                       int64_t N, int64_t K, void *stream) {
    return entry(OP_RHS_T, true, A, lda, Bt, ldbt, C, ldc, M, N, K, stream);
}

int det_gemm_strict_fwd_fp32(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                             float *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             void *stream) {
    return entry(OP_FWD_F32, true, A, lda, B, ldb, C, ldc, M, N, K, stream);
}

int det_gemm_strict_da(const det_bf16 *dC, int64_t lddc, const det_bf16 *B, int64_t ldb,
                       det_bf16 *dA, int64_t ldda, int64_t M, int64_t N, int64_t K,
                       void *stream) {
    return entry(OP_DA, true, dC, lddc, B, ldb, dA, ldda, M, N, K, stream);
}

int det_gemm_strict_db(const det_bf16 *A, int64_t lda, const det_bf16 *dC, int64_t lddc,
                       det_bf16 *dB, int64_t lddb, int64_t M, int64_t N, int64_t K,
                       void *stream) {
    return entry(OP_DB, true, A, lda, dC, lddc, dB, lddb, M, N, K, stream);
}

int det_gemm_strict_db_transposed(const det_bf16 *A, int64_t lda, const det_bf16 *dC,
                                  int64_t lddc, det_bf16 *dBt, int64_t lddbt, int64_t M,
                                  int64_t N, int64_t K, void *stream) {
    return entry(OP_DB_T, true, A, lda, dC, lddc, dBt, lddbt, M, N, K, stream);
}

int det_gemm_debug_leaves(const det_bf16 *A, int64_t lda, const det_bf16 *B, int64_t ldb,
                          det_bf16 *leaves, int64_t M, int64_t N, int64_t K, void *stream) {
    return entry(OP_LEAVES, false, A, lda, B, ldb, leaves, 0, M, N, K, stream);
}

int det_gemm_debug_round(const float *x, det_bf16 *out, int64_t n, void *stream) {
    if (n < 0)
        return DET_GEMM_EINVAL;
    if (n == 0)
        return DET_GEMM_OK;
    if (!x || !out)
        return DET_GEMM_EINVAL;
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > kMaxDim)
        return DET_GEMM_EINVAL;
    hipLaunchKernelGGL(debug_round_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), x, out, n);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

int det_gemm_debug_add(const det_bf16 *a, const det_bf16 *b, det_bf16 *out, int64_t n,
                       void *stream) {
    if (n < 0)
        return DET_GEMM_EINVAL;
    if (n == 0)
        return DET_GEMM_OK;
    if (!a || !b || !out)
        return DET_GEMM_EINVAL;
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > kMaxDim)
        return DET_GEMM_EINVAL;
    hipLaunchKernelGGL(debug_add_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a, b, out, n);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

int det_gemm_debug_matrix_add(const det_bf16 *a, const det_bf16 *b, det_bf16 *out, int64_t n,
                              int selector, void *stream) {
    if (n < 0 || (selector != 0 && selector != 1))
        return DET_GEMM_EINVAL;
    if (n == 0)
        return DET_GEMM_OK;
    if (!a || !b || !out)
        return DET_GEMM_EINVAL;
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    const int64_t blocks = (n + 1023) / 1024;  // 4 waves of 256 pairs
    if (blocks > kMaxDim)
        return DET_GEMM_EINVAL;
    hipLaunchKernelGGL(debug_matrix_add_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a, b, out, n, selector);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

int det_gemm_debug_issue_probe(int mode, int iters, int workgroups, float *sink, void *stream) {
    if (mode < 0 || mode > 1 || iters < 1 || workgroups < 1 || !sink)
        return DET_GEMM_EINVAL;
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (mode == 0)
        hipLaunchKernelGGL(issue_probe_kernel<0>, dim3((unsigned)workgroups), dim3(512), 0, st, sink, iters);
    else
        hipLaunchKernelGGL(issue_probe_kernel<1>, dim3((unsigned)workgroups), dim3(512), 0, st, sink, iters);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

int det_gemm_debug_force_config(int config) {
    if (config < -1 || config >= kNumTileCfgs)
        return DET_GEMM_EINVAL;
    g_force_config = config;
    return kNumTileCfgs;
}

int det_gemm_debug_config(int op, const void *P, int64_t ldp, const void *Q, int64_t ldq,
                          const void *Out, int64_t ldo, int64_t M, int64_t N, int64_t K) {
    if (op < OP_FWD || op > OP_DB_T)
        return DET_GEMM_EINVAL;
    Problem pr;
    bool empty;
    const int rc = build(static_cast<Op>(op), P, ldp, Q, ldq, const_cast<void *>(Out), ldo, M, N,
                         K, pr, empty);
    if (rc != DET_GEMM_OK)
        return rc;
    if (empty)
        return DET_GEMM_EINVAL;  // nothing is launched, so no configuration runs
    int levels = 0;
    const TreeSel tree = pick_tree((int32_t)((pr.R + 31) / 32), levels);
    return pick_config(pr, tree, levels);
}

const char *det_gemm_status_string(int status) {
    switch (status) {
    case DET_GEMM_OK:
        return "success";
    case DET_GEMM_EINVAL:
        return "invalid argument (null pointer, negative size, leading dimension, overlap)";
    case DET_GEMM_EKCAP:
        return "reduction length must be in [1, 32768]";
    case DET_GEMM_EHIP:
        return "HIP runtime error or no gfx950 device";
    case DET_ATTN_ESCRATCH:
        return "problem needs more scratch than the library's fixed device array holds";
    default:
        return "unknown status";
    }
}

}  // extern "C"

// ==== MoE grouped GEMM with the per-token slot epilogue (det_moe.h) ====
namespace {

constexpr int kCombineDepth = 24;  // pending left subtrees of a slot tree, J < 2^23

// Slots as a kernel of their own (when the grouped GEMM does not write them):
// block (rows 16*bx .. 16*bx+15, slot by), one wave per row.
__global__ __launch_bounds__(256) void moe_slot_kernel(const uint16_t *y, int64_t ldy,
                                                       const uint16_t *g, int64_t ldg,
                                                       float *slots, int64_t slot_ld, int T,
                                                       int N) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = blockIdx.y;
    const int c = j * kSlot + 2 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = blockIdx.x * 16 + wave * 4 + q;
        if (r >= T)
            break;
        const uint16_t *yr = y + (int64_t)r * ldy, *gr = g + (int64_t)r * ldg;
        float p0 = 0.0f, p1 = 0.0f;
        if (c < N)
            p0 = bf16_value(yr[c]) * bf16_value(gr[c]);
        if (c + 1 < N)
            p1 = bf16_value(yr[c + 1]) * bf16_value(gr[c + 1]);
        const float v = slot_tree(p0, p1);
        if (lane == 0)
            slots[(int64_t)j * slot_ld + r] = v;
    }
}

// dprob[r]: the mid-split tree of fp32 adds over the J slots of row r, one
// thread per row, as a post-order walk over the slots in ascending order with
// a stack of pending left subtrees (in LDS, one column per thread): after slot
// t, every inner node whose range ends at t is closed by adding its left
// subtree (popped) to the running node.
// The slots are loaded 32 at a time ahead of their tree steps.
constexpr int kCombineThreads = 64, kCombineChunk = 32;

__global__ __launch_bounds__(kCombineThreads) void moe_combine_kernel(const float *slots,
                                                                      int64_t slot_ld,
                                                                      float *dprob, int T, int J) {
    __shared__ float stack[kCombineDepth][kCombineThreads];
    const int r = blockIdx.x * kCombineThreads + threadIdx.x;
    if (r >= T)
        return;
    if (J == 0) {
        dprob[r] = 0.0f;
        return;
    }
    int sp = 0;
    for (int t0 = 0; t0 < J; t0 += kCombineChunk) {
        float v[kCombineChunk];
#pragma unroll
        for (int q = 0; q < kCombineChunk; ++q)
            v[q] = t0 + q < J ? slots[(int64_t)(t0 + q) * slot_ld + r] : 0.0f;
#pragma unroll
        for (int q = 0; q < kCombineChunk; ++q) {
            if (t0 + q >= J)
                break;
            float x = v[q];
            for (int m = merges_after(t0 + q, J); m > 0; --m)
                x = stack[--sp][threadIdx.x] + x;
            stack[sp++][threadIdx.x] = x;
        }
    }
    dprob[r] = stack[0][threadIdx.x];
}

int launch_slots(const uint16_t *Y, int64_t ldy, const uint16_t *G, int64_t ldg, float *slots,
                 int64_t slot_ld, int64_t T, int64_t J, int64_t N, hipStream_t st) {
    if (J == 0)
        return DET_GEMM_OK;
    hipLaunchKernelGGL(moe_slot_kernel, dim3((unsigned)((T + 15) / 16), (unsigned)J), dim3(256),
                       0, st, Y, ldy, G, ldg, slots, slot_ld, (int)T, (int)N);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

int moe_entry(const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw, int64_t w_stride,
              const int64_t *off, int64_t E, const uint16_t *G, int64_t ldg, uint16_t *Y,
              int64_t ldy, float *slots, int64_t slot_ld, float *dprob, int64_t T, int64_t N,
              int64_t K, hipStream_t st) {
    if (T < 0 || N < 0 || K < 0 || E < 1 || E > DET_MOE_MAX_EXPERTS || !off)
        return DET_GEMM_EINVAL;
    if (off[0] != 0 || off[E] != T)
        return DET_GEMM_EINVAL;
    for (int64_t e = 0; e < E; ++e)
        if (off[e + 1] < off[e])
            return DET_GEMM_EINVAL;
    if (T == 0)
        return DET_GEMM_OK;
    if (K == 0 || K > DET_GEMM_MAX_REDUCTION)
        return DET_GEMM_EKCAP;
    const int64_t J = (N + kSlot - 1) / kSlot;
    if (T > kMaxDim || N > kMaxDim || J > 65535 || !dprob || slot_ld < T || slot_ld > kMaxDim ||
        (J > 0 && !slots) || w_stride < 0)
        return DET_GEMM_EINVAL;
    const Mat x{X, T, K, ldx, 2}, gm{G, T, N, ldg, 2}, ym{Y, T, N, ldy, 2};
    const Mat sm{slots, J, T, slot_ld, 4}, dm{dprob, 1, T, T, 4};
    // the weights as one range: E matrices [K,N] w_stride apart
    const Mat wm{W, K, N, ldw, 2};
    if (!mat_ok(x) || !mat_ok(gm) || !mat_ok(ym) || !mat_ok(wm) || !mat_ok(sm) || !mat_ok(dm))
        return DET_GEMM_EINVAL;
    if (N > 0 && (w_stride > (kMaxDim << 8) / E))
        return DET_GEMM_EINVAL;
    const Mat wall{W, 1, N > 0 ? (E - 1) * w_stride + (K - 1) * ldw + N : 0, 1, 2};
    const Mat *outs[3] = {&ym, &sm, &dm};
    const Mat *ins[3] = {&x, &gm, &wall};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 3; ++b)
            if (overlaps(*outs[a], *ins[b]))
                return DET_GEMM_EINVAL;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(*outs[a], *outs[b]))
                return DET_GEMM_EINVAL;
    }
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    const int64_t blocks = (T + kCombineThreads - 1) / kCombineThreads;
    if (N > 0) {
        // the grouped wide kernel when the shape allows it, else one product per expert
        Problem base{X, ldx, true, W, ldw, false, Y, ldy, OUT_BF16, T, N, K};
        const int L = (int)((K + 31) / 32);
        int levels = 0;
        const TreeSel tree = pick_tree(L, levels);
        int cfg = -1, up = 0;
        if (g_force_config >= 0) {
            if (kTileCfgs[g_force_config].kind == KIND_WIDE) {
                if (kTileCfgs[g_force_config].bn() != kSlot ||
                    !wide_ok(base, tree, kTileCfgs[g_force_config], up))
                    return DET_GEMM_EINVAL;
                cfg = g_force_config;
            }
        } else {
            for (int c : {8, 5, 9, 7})
                if (wide_ok(base, tree, kTileCfgs[c], up) &&
                    kTileCfgs[c].lds_bytes(up) + kEpiLds <= kLdsMax) {
                    cfg = c;
                    break;
                }
        }
        // the grouped kernel's LDS also holds the epilogue header
        if (cfg >= 0 && kTileCfgs[cfg].lds_bytes(up) + kEpiLds > kLdsMax) {
            if (g_force_config >= 0)
                return DET_GEMM_EINVAL;
            cfg = -1;
        }
        bool fused = false;
        if (cfg >= 0) {
            GroupTable g;
            std::memset(&g, 0, sizeof g);
            const int64_t tiles_j = (N + kTileCfgs[cfg].bn() - 1) / kTileCfgs[cfg].bn();
            int64_t tiles = 0;
            g.groups = (int32_t)E;
            for (int64_t e = 0; e < E; ++e) {
                const int64_t rows = off[e + 1] - off[e];
                g.tile_start[e] = (int32_t)tiles;
                g.row_start[e] = (int32_t)off[e];
                g.rows[e] = (int32_t)rows;
                tiles += (rows + kTileCfgs[cfg].bm() - 1) / kTileCfgs[cfg].bm() * tiles_j;
                if (tiles > kMaxDim)
                    return DET_GEMM_EINVAL;
            }
            g.tile_start[E] = (int32_t)tiles;
            g.y_stride = w_stride;
            // Tail balancing: one workgroup of these tiles fills a compute
            // unit, so when the last round would keep at most half of the
            // units busy, its tiles run as two half-height tiles each (the
            // tree split over two wave groups, half the stages each): every
            // unit then ends after about the same share of the work.  Bits do
            // not depend on the tile shape.
            g.split_from = (int32_t)tiles;
            g.split_levels = 0;
            if (kTileCfgs[cfg].tb == 1) {
                const int64_t cus = device_cus();
                const int64_t r = cus > 0 ? tiles % cus : 0;
                const TileCfg h{4, 2, 1, 4, KIND_WIDE, 3, kTileCfgs[cfg].gl, kTileCfgs[cfg].ru, 1, 2};
                int uph = 0;
                if (tiles > cus && r > 0 && 2 * r <= cus && wide_ok(base, tree, h, uph) &&
                    h.lds_bytes(uph) + kEpiLds <= kLdsMax) {
                    g.split_from = (int32_t)(tiles - r);
                    g.split_levels = uph;
                }
            }
            MfmaParams p;
            std::memset(&p, 0, sizeof p);
            p.x = X;
            p.ldx = ldx;
            p.y = W;
            p.ldy = ldw;
            p.c = Y;
            p.ldc = ldy;
            p.I = 0;  // per group
            p.J = (int32_t)N;
            p.R = (int32_t)K;
            p.L = L;
            p.tiles_j = (int32_t)tiles_j;
            p.levels = up;
            p.xvec = aligned16(X, ldx);
            p.yvec = aligned16(W, ldw) && (w_stride % 8) == 0;
            p.cvec = aligned16(Y, ldy);
            fused = aligned16(G, ldg);
            if (fused) {
                g.g = G;
                g.ldg = ldg;
                g.slots = slots;
                g.slot_ld = slot_ld;
            }
            const hipError_t e = launch_moe_grouped(cfg, p, g, tiles, st);
            if (e == hipErrorInvalidConfiguration)
                return DET_GEMM_EINVAL;
            if (e != hipSuccess)
                return DET_GEMM_EHIP;
        } else {
            for (int64_t e = 0; e < E; ++e) {
                if (off[e + 1] == off[e])
                    continue;
                Problem pr = base;
                pr.x = X + off[e] * ldx;
                pr.y = W + e * w_stride;
                pr.c = Y + off[e] * ldy;
                pr.I = off[e + 1] - off[e];
                const int rc = run_mfma(pr, st);
                if (rc != DET_GEMM_OK)
                    return rc;
            }
        }
        if (!fused) {
            const int rc = launch_slots(Y, ldy, G, ldg, slots, slot_ld, T, J, N, st);
            if (rc != DET_GEMM_OK)
                return rc;
        }
    }
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, st, slots,
                       slot_ld, dprob, (int)T, (int)J);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

}  // namespace

extern "C" {

int det_moe_fwd_dprob(const det_bf16 *X, int64_t ldx, const det_bf16 *W, int64_t ldw,
                      int64_t w_stride, const int64_t *offsets, int64_t E, const det_bf16 *G,
                      int64_t ldg, det_bf16 *Y, int64_t ldy, float *slots, int64_t slot_ld,
                      float *dprob, int64_t T, int64_t N, int64_t K, void *stream) {
    return moe_entry(X, ldx, W, ldw, w_stride, offsets, E, G, ldg, Y, ldy, slots, slot_ld, dprob,
                     T, N, K, static_cast<hipStream_t>(stream));
}

int det_moe_debug_slots(const det_bf16 *Y, int64_t ldy, const det_bf16 *G, int64_t ldg,
                        float *slots, int64_t slot_ld, int64_t T, int64_t N, void *stream) {
    if (T < 0 || N < 0)
        return DET_GEMM_EINVAL;
    const int64_t J = (N + kSlot - 1) / kSlot;
    if (T == 0 || J == 0)
        return DET_GEMM_OK;
    if (T > kMaxDim || J > 65535 || slot_ld < T || !slots)
        return DET_GEMM_EINVAL;
    const Mat ym{Y, T, N, ldy, 2}, gm{G, T, N, ldg, 2}, sm{slots, J, T, slot_ld, 4};
    if (!mat_ok(ym) || !mat_ok(gm) || !mat_ok(sm) || overlaps(sm, ym) || overlaps(sm, gm))
        return DET_GEMM_EINVAL;
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    return launch_slots(Y, ldy, G, ldg, slots, slot_ld, T, J, N, static_cast<hipStream_t>(stream));
}

}  // extern "C"
