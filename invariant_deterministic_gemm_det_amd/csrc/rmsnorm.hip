// Batch-invariant RMSNorm (declared in include/det_norm.h).
//
// Summary page of "Defeating Nondeterminism in LLM Inference", section on
// batch-invariant kernel design, RMSNorm: each row is reduced by one
// workgroup with one fixed strategy, never split across workgroups.
//
// One workgroup of 256 threads per row; thread t is lane t of the definition:
// it reads its 8-element chunks t, t + 256, ... with 16-byte loads, sums their
// squares in ascending order, and keeps up to four chunks in registers for the
// output pass (rows of up to 8192 elements are read from HBM once).  The
// 256 lane sums meet in the pairwise tree: six shuffle levels inside each
// wave, then (wave 0 + wave 1) + (wave 2 + wave 3).  Square root and division
// are rounded to nearest as the definition requires (the runtime's fp32
// square root and division are not guaranteed to be): a candidate from fp64,
// moved to the fp32 neighbour while that is closer, decided exactly in fp64.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bf16_device.h"
#include "det_norm.h"
#include "device_check.h"

using namespace detgemm;

namespace {

constexpr int kLanes = 256;
constexpr int kChunk = 8;
constexpr int kKeep = 4;

__device__ __forceinline__ float bf(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Chunk c of a row (elements 8c .. 8c+7; past H: +0), as 4 words of bf16 pairs.
template <bool VEC>
__device__ __forceinline__ uint4 load_chunk(const uint16_t *row, int c, int H) {
    if (VEC && 8 * c + 8 <= H)
        return *reinterpret_cast<const uint4 *>(row + 8 * c);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < 8 && 8 * c + e < H; ++e)
        w[e >> 1] |= (uint32_t)row[8 * c + e] << (16 * (e & 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool VEC>
__device__ __forceinline__ void store_chunk(uint16_t *row, int c, int H, uint4 v) {
    if (VEC && 8 * c + 8 <= H) {
        *reinterpret_cast<uint4 *>(row + 8 * c) = v;
        return;
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    for (int e = 0; e < 8 && 8 * c + e < H; ++e)
        row[8 * c + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
}

__device__ __forceinline__ float chunk_sumsq(float p, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = bf((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        p = __fadd_rn(p, __fmul_rn(x, x));
    }
    return p;
}

__device__ __forceinline__ uint4 chunk_out(uint4 xv, uint4 wv, float rs) {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = __fmul_rn(__fmul_rn(bf(xw[k] & 0xFFFFu), rs), bf(ww[k] & 0xFFFFu));
        const float b = __fmul_rn(__fmul_rn(bf(xw[k] >> 16), rs), bf(ww[k] >> 16));
        o[k] = pair_bits(round_pair(a, b));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float next_up(float q) { return __uint_as_float(__float_as_uint(q) + 1u); }
__device__ __forceinline__ float next_down(float q) { return __uint_as_float(__float_as_uint(q) - 1u); }

__device__ __forceinline__ bool positive_finite(float q) { return q > 0.0f && q <= 3.40282347e38f; }

// fp32 square root rounded to nearest.  For a positive finite fp32 q, the
// half-way points m to its neighbours have at most 26 significant bits, so m*m
// is exact in fp64 and s < m*m decides on which side of m the root lies (the
// root of an fp32 value never falls on a half-way point).
__device__ __forceinline__ float sqrt_rn(float s) {
    float q = (float)__builtin_sqrt((double)s);
    for (int it = 0; it < 2 && positive_finite(q); ++it) {
        const double lo = 0.5 * ((double)q + (double)next_down(q));
        const double hi = 0.5 * ((double)q + (double)next_up(q));
        if ((double)s < lo * lo)
            q = next_down(q);
        else if ((double)s > hi * hi)
            q = next_up(q);
        else
            break;
    }
    return q;
}

// fp32 quotient a / b rounded to nearest, for a >= 0 and b > 0 with b an fp32
// value and the half-way products m*b exact in fp64 (m: 26 bits, b: 24 bits);
// a quotient of fp32 values never falls on a half-way point.
__device__ __forceinline__ float div_rn(float a, float b) {
    float q = (float)((double)a / (double)b);
    for (int it = 0; it < 2 && positive_finite(q); ++it) {
        const double lo = 0.5 * ((double)q + (double)next_down(q));
        const double hi = 0.5 * ((double)q + (double)next_up(q));
        if (lo * (double)b > (double)a)
            q = next_down(q);
        else if (hi * (double)b < (double)a)
            q = next_up(q);
        else
            break;
    }
    return q;
}

template <bool VEC>
__global__ __launch_bounds__(kLanes) void rmsnorm_kernel(const uint16_t *x, int64_t ldx,
                                                         const uint16_t *w, float eps, uint16_t *y,
                                                         int64_t ldy, float *rstd, int H) {
    __shared__ float part[kLanes / 64];
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const uint16_t *xr = x + r * ldx;
    const int chunks = (H + kChunk - 1) / kChunk;
    uint4 keep[kKeep];
    float p = 0.0f;
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
        const int c = t + k * kLanes;
        keep[k] = c < chunks ? load_chunk<VEC>(xr, c, H) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kKeep; ++k)
        p = chunk_sumsq(p, keep[k]);  // zero chunks add +0: no change
    for (int c = t + kKeep * kLanes; c < chunks; c += kLanes)
        p = chunk_sumsq(p, load_chunk<VEC>(xr, c, H));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        p = __fadd_rn(p, __shfl_xor(p, m, 64));
    if ((t & 63) == 0)
        part[t >> 6] = p;
    __syncthreads();
    const float ss = __fadd_rn(__fadd_rn(part[0], part[1]), __fadd_rn(part[2], part[3]));
    const float rs = div_rn(1.0f, sqrt_rn(__fadd_rn(div_rn(ss, (float)H), eps)));
    if (t == 0 && rstd)
        rstd[r] = rs;
    uint16_t *yr = y + r * ldy;
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
        const int c = t + k * kLanes;
        if (c < chunks)
            store_chunk<VEC>(yr, c, H, chunk_out(keep[k], load_chunk<VEC>(w, c, H), rs));
    }
    for (int c = t + kKeep * kLanes; c < chunks; c += kLanes)
        store_chunk<VEC>(yr, c, H, chunk_out(load_chunk<VEC>(xr, c, H), load_chunk<VEC>(w, c, H), rs));
}

bool aligned16(const void *p, int64_t ld) {
    return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && ld % 8 == 0;
}

bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
    if (na <= 0 || nb <= 0)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

extern "C" int det_rmsnorm(const det_bf16 *x, int64_t ldx, const det_bf16 *w, float eps,
                           det_bf16 *y, int64_t ldy, float *rstd, int64_t R, int64_t H,
                           void *stream) {
    if (R < 0 || H < 1 || H > DET_NORM_MAX_H)
        return DET_GEMM_EINVAL;
    if (R == 0)
        return DET_GEMM_OK;
    if (!x || !w || !y || R > 0x7FFFFFFF || (R > 1 && (ldx < H || ldy < H)))
        return DET_GEMM_EINVAL;
    const int64_t xb = ((R - 1) * (R > 1 ? ldx : 0) + H) * 2, yb = ((R - 1) * (R > 1 ? ldy : 0) + H) * 2;
    if (overlap(y, yb, x, xb) || overlap(y, yb, w, H * 2) ||
        (rstd && (overlap(rstd, R * 4, x, xb) || overlap(rstd, R * 4, w, H * 2) ||
                  overlap(rstd, R * 4, y, yb))))
        return DET_GEMM_EINVAL;
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec = aligned16(x, R > 1 ? ldx : 8) && aligned16(y, R > 1 ? ldy : 8) &&
                     aligned16(w, 8);
    if (vec)
        hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3((unsigned)R), dim3(kLanes), 0, st, x, ldx, w,
                           eps, y, ldy, rstd, (int)H);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3((unsigned)R), dim3(kLanes), 0, st, x, ldx,
                           w, eps, y, ldy, rstd, (int)H);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}
