// Strict-order det_gemm kernel: every leaf is summed by a scalar fp32 fused
// multiply-add chain in ascending reduction index, exactly as the leaf is
// defined (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
// (det_gemm)", section "Ascend NPU backend": 32-element leaves accumulated in
// fp32 in ascending order, rounded once to bf16 round-to-nearest-even, merged by
// the mid-split tree of bf16 adds).  A bf16 product is exact in fp32, so
// fma(x, y, s) rounds exactly like s + x*y.  Slow by design: it exists to be
// bit-exact to the CPU definition.
//
// One 256-thread workgroup owns a 16x16 output tile; thread (ty, tx) owns output
// (i0+ty, j0+tx) and walks all leaves of its reduction in order.  The leaf tiles
// of both operands are staged through LDS with scalar loads, so any operand
// layout (any pair of strides) is handled by the same code.  The tree is
// evaluated in streaming post-order: after leaf l the kernel performs as many
// merges as there are inner nodes whose leaf range ends at l+1, popping the two
// most recent values from a per-thread stack kept in LDS.
#pragma once

#include "bf16_device.h"

namespace detgemm {

struct StrictParams {
    const uint16_t *x;   // X(i, r) = x[i*sxi + r*sxr]
    int64_t sxi, sxr;
    const uint16_t *y;   // Y(j, r) = y[j*syj + r*syr]
    int64_t syj, syr;
    void *c;             // out(i, j) at c[i*sci + j*scj] (elements)
    int64_t sci, scj;
    int64_t I, J, R;
    int32_t L;
    int32_t tiles_j;
};

constexpr int kStrictTile = 16;
constexpr int kStrictStack = 12;   // ceil(log2 1024) + 2 entries suffice

__device__ __forceinline__ float strict_widen(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// Round to nearest, ties to even, on the bit pattern; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t strict_round(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t strict_add(uint16_t a, uint16_t b) {
    return strict_round(__fadd_rn(strict_widen(a), strict_widen(b)));
}

// Number of inner nodes of the mid-split tree over [0, L) whose leaf range ends
// at leaf l (i.e. hi == l + 1): walk from the root down to leaf l.
__device__ __forceinline__ int strict_merges_after(int l, int L) {
    int lo = 0, hi = L, count = 0;
    while (hi - lo > 1) {
        if (hi == l + 1)
            ++count;
        int mid = lo + (hi - lo) / 2;
        if (l < mid)
            hi = mid;
        else
            lo = mid;
    }
    return count;
}

template <bool OUT_F32>
__global__ __launch_bounds__(256) void strict_kernel(StrictParams p) {
    __shared__ float xs[kStrictTile][33];
    __shared__ float ys[kStrictTile][33];
    __shared__ uint16_t stack[kStrictStack][256];

    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int64_t tile = blockIdx.x;
    const int64_t i0 = (tile / p.tiles_j) * kStrictTile;
    const int64_t j0 = (tile % p.tiles_j) * kStrictTile;

    int top = 0;  // stack size
    for (int l = 0; l < p.L; ++l) {
        const int64_t r0 = (int64_t)l * 32;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + 256 * q;
            const int row = e >> 5, rr = e & 31;
            const int64_t r = r0 + rr;
            const int64_t gi = i0 + row, gj = j0 + row;
            xs[row][rr] = (gi < p.I && r < p.R) ? strict_widen(p.x[gi * p.sxi + r * p.sxr]) : 0.0f;
            ys[row][rr] = (gj < p.J && r < p.R) ? strict_widen(p.y[gj * p.syj + r * p.syr]) : 0.0f;
        }
        __syncthreads();
        float s = 0.0f;
        for (int k = 0; k < 32; ++k)
            s = __builtin_fmaf(xs[ty][k], ys[tx][k], s);
        __syncthreads();

        uint16_t node = strict_round(s);
        const int merges = strict_merges_after(l, p.L);
        for (int m = 0; m < merges; ++m) {
            --top;
            node = strict_add(stack[top][tid], node);
        }
        stack[top][tid] = node;
        ++top;
    }

    const int64_t i = i0 + ty, j = j0 + tx;
    if (i < p.I && j < p.J) {
        const uint16_t root = stack[0][tid];
        const int64_t off = i * p.sci + j * p.scj;
        if (OUT_F32)
            static_cast<float *>(p.c)[off] = strict_widen(root);
        else
            static_cast<uint16_t *>(p.c)[off] = root;
    }
}

}  // namespace detgemm
