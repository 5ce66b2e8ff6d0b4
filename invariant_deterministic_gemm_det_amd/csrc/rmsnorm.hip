// Batch-invariant RMSNorm (declared in include/det_norm.h).
//
// Summary page of "Defeating Nondeterminism in LLM Inference", section on
// batch-invariant kernel design, RMSNorm: each row is reduced by one
// workgroup with one fixed strategy, never split across workgroups.
//
// The sum of squares is the mid-split tree of fp32 adds over the row's H
// squares.  One workgroup of 256 threads per row evaluates it from the nodes
// of depth 8: thread t takes node t (bits of t from the top: 0 = left child),
// a contiguous range of about H / 256 elements, and evaluates that subtree
// itself; the 256 node sums then meet in the top 8 levels, six shuffle levels
// inside each wave and (wave 0 + wave 1) + (wave 2 + wave 3).  A node of one
// element has no children, so for H < 256 some positions of depth 8 are empty
// and a parent with an empty right child is its left child.
//   * H = 256 * M with M in the instantiated set: every node holds exactly M
//     elements, [M t, M t + M); the thread loads them with the widest aligned
//     loads, evaluates the subtree at compile time in registers, and writes
//     its own outputs from the kept values (the row is read from HBM once).
//   * any other H: each thread walks its range in ascending order with the
//     streaming post-order of the mid-split tree (a stack of pending left
//     subtrees in LDS), then the output pass reads the row again in 16-byte
//     chunks.
// Square root and division are rounded to nearest as the definition requires
// (the runtime's fp32 square root and division are not guaranteed to be): a
// candidate from fp64, moved to the fp32 neighbour while that is closer,
// decided exactly in fp64.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bf16_device.h"
#include "det_norm.h"
#include "device_check.h"

using namespace detgemm;

namespace {

constexpr int kLanes = 256;
constexpr int kChunk = 8;
constexpr int kStack = 16;   // pending left subtrees of a node's walk: ranges below 2^15

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

__device__ __forceinline__ float square(uint32_t bits16) {
    const float x = bf(bits16);
    return __fmul_rn(x, x);
}

// Mid-split tree of fp32 adds over the compile-time range s[LO, HI).
template <int LO, int HI, int M>
__device__ __forceinline__ float tree_sum(const float (&s)[M]) {
    if constexpr (HI - LO == 1) {
        return s[LO];
    } else {
        constexpr int MID = LO + (HI - LO) / 2;
        return __fadd_rn(tree_sum<LO, MID>(s), tree_sum<MID, HI>(s));
    }
}

// The top 8 levels over the 256 node sums (one per thread) and the row's
// rstd; `empty`: this thread's position of depth 8 holds no node (H < 256).
// Both threads of a pair compute the same parent (fp32 addition commutes).
__device__ __forceinline__ float row_rstd(float p, bool empty, int H, float eps) {
    __shared__ float part[kLanes / 64];
    __shared__ int part_empty[kLanes / 64];
    const int t = threadIdx.x;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float q = __shfl_xor(p, m, 64);
        const bool qe = __shfl_xor(empty ? 1 : 0, m, 64) != 0;
        p = empty ? q : (qe ? p : __fadd_rn(p, q));
        empty = empty && qe;
    }
    if ((t & 63) == 0) {
        part[t >> 6] = p;
        part_empty[t >> 6] = empty ? 1 : 0;
    }
    __syncthreads();
    const auto join = [](float a, bool ae, float b, bool be, bool &e) {
        e = ae && be;
        return ae ? b : (be ? a : __fadd_rn(a, b));
    };
    bool e01, e23, e;
    const float s01 = join(part[0], part_empty[0] != 0, part[1], part_empty[1] != 0, e01);
    const float s23 = join(part[2], part_empty[2] != 0, part[3], part_empty[3] != 0, e23);
    const float ss = join(s01, e01, s23, e23, e);
    return div_rn(1.0f, sqrt_rn(__fadd_rn(div_rn(ss, (float)H), eps)));
}

// H = 256 * M.  G: elements per load (8, 4, 2 or 1; VEC false: 1).
template <int M, bool VEC>
__global__ __launch_bounds__(kLanes) void rmsnorm_fixed_kernel(const uint16_t *x, int64_t ldx,
                                                               const uint16_t *w, float eps,
                                                               uint16_t *y, int64_t ldy,
                                                               float *rstd) {
    constexpr int G = !VEC ? 1 : (M % 8 == 0 ? 8 : (M % 4 == 0 ? 4 : (M % 2 == 0 ? 2 : 1)));
    constexpr int H = kLanes * M;
    const int64_t r = blockIdx.x;
    const int i0 = M * threadIdx.x;
    const uint16_t *xr = x + r * ldx + i0;
    uint32_t xv[(M + 1) / 2];  // the thread's elements, two per word
#pragma unroll
    for (int k = 0; k < M; k += G) {
        if constexpr (G == 8) {
            const uint4 q = *reinterpret_cast<const uint4 *>(xr + k);
            xv[k / 2] = q.x, xv[k / 2 + 1] = q.y, xv[k / 2 + 2] = q.z, xv[k / 2 + 3] = q.w;
        } else if constexpr (G == 4) {
            const uint2 q = *reinterpret_cast<const uint2 *>(xr + k);
            xv[k / 2] = q.x, xv[k / 2 + 1] = q.y;
        } else if constexpr (G == 2) {
            xv[k / 2] = *reinterpret_cast<const uint32_t *>(xr + k);
        } else {
            const uint32_t h = xr[k];
            xv[k / 2] = (k & 1) ? (xv[k / 2] | (h << 16)) : h;
        }
    }
    float sq[M];
#pragma unroll
    for (int k = 0; k < M; ++k)
        sq[k] = square((xv[k / 2] >> (16 * (k & 1))) & 0xFFFFu);
    const float rs = row_rstd(tree_sum<0, M>(sq), false, H, eps);
    if (threadIdx.x == 0 && rstd)
        rstd[r] = rs;
    const uint16_t *wr = w + i0;
    uint16_t *yr = y + r * ldy + i0;
    if constexpr (G >= 2) {
        // G elements of w in, G of y out per access, like the loads of x
#pragma unroll
        for (int k = 0; k < M; k += G) {
            uint32_t wk[G / 2], o[G / 2];
            if constexpr (G == 8) {
                const uint4 q = *reinterpret_cast<const uint4 *>(wr + k);
                wk[0] = q.x, wk[1] = q.y, wk[2] = q.z, wk[3] = q.w;
            } else if constexpr (G == 4) {
                const uint2 q = *reinterpret_cast<const uint2 *>(wr + k);
                wk[0] = q.x, wk[1] = q.y;
            } else {
                wk[0] = *reinterpret_cast<const uint32_t *>(wr + k);
            }
#pragma unroll
            for (int h = 0; h < G / 2; ++h) {
                const uint32_t xk = xv[k / 2 + h];
                const float a = __fmul_rn(__fmul_rn(bf(xk & 0xFFFFu), rs), bf(wk[h] & 0xFFFFu));
                const float b = __fmul_rn(__fmul_rn(bf(xk >> 16), rs), bf(wk[h] >> 16));
                o[h] = pair_bits(round_pair(a, b));
            }
            if constexpr (G == 8)
                *reinterpret_cast<uint4 *>(yr + k) = make_uint4(o[0], o[1], o[2], o[3]);
            else if constexpr (G == 4)
                *reinterpret_cast<uint2 *>(yr + k) = make_uint2(o[0], o[1]);
            else
                *reinterpret_cast<uint32_t *>(yr + k) = o[0];
        }
    } else {
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const float xk = bf((xv[k / 2] >> (16 * (k & 1))) & 0xFFFFu);
            const float v = __fmul_rn(__fmul_rn(xk, rs), bf(wr[k]));
            yr[k] = (uint16_t)pair_bits(round_pair(v, 0.0f));
        }
    }
}

// Number of inner nodes of the mid-split tree over [0, n) whose range ends
// at i + 1: the adds that follow leaf i in the post-order walk.
__device__ __forceinline__ int merges_after(int i, int n) {
    int lo = 0, hi = n, count = 0;
    while (hi - lo > 1) {
        if (hi == i + 1)
            ++count;
        const int mid = lo + (hi - lo) / 2;
        if (i < mid)
            hi = mid;
        else
            lo = mid;
    }
    return count;
}

// Any H: node ranges from the splits, subtrees by the streaming walk.
template <bool VEC>
__global__ __launch_bounds__(kLanes) void rmsnorm_any_kernel(const uint16_t *x, int64_t ldx,
                                                             const uint16_t *w, float eps,
                                                             uint16_t *y, int64_t ldy,
                                                             float *rstd, int H) {
    __shared__ float stack[kStack][kLanes];
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const uint16_t *xr = x + r * ldx;
    // node t of depth 8: take the left (bit 0) or right (bit 1) child 8 times
    int lo = 0, hi = H;
    bool empty = false;
#pragma unroll
    for (int d = 7; d >= 0; --d) {
        const int bit = (t >> d) & 1;
        if (hi - lo >= 2) {
            const int mid = lo + (hi - lo) / 2;
            if (bit)
                lo = mid;
            else
                hi = mid;
        } else if (bit) {
            empty = true;  // a leaf has no right child
        }
    }
    float p = 0.0f;
    if (!empty) {
        const int n = hi - lo;
        int sp = 0;
        for (int i = 0; i < n; ++i) {
            float v = square(xr[lo + i]);
            for (int m = merges_after(i, n); m > 0; --m)
                v = __fadd_rn(stack[--sp][t], v);
            stack[sp++][t] = v;
        }
        p = stack[0][t];
    }
    const float rs = row_rstd(p, empty, H, eps);
    if (t == 0 && rstd)
        rstd[r] = rs;
    uint16_t *yr = y + r * ldy;
    const int chunks = (H + kChunk - 1) / kChunk;
    for (int c = t; c < chunks; c += kLanes)
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

// The node sizes M (H = 256 * M) with a compile-time kernel: model widths
// from 256 to 16384 that are multiples of 256 * 4, and the small ones.
template <int... Ms>
struct MList {};
using kFixedList = MList<1, 2, 4, 8, 12, 16, 20, 24, 28, 32, 40, 48, 56, 64>;
constexpr kFixedList kFixed{};

// Whether the row base and leading dimension allow loads of G elements.
bool aligned_to(const void *p, int64_t ld, int64_t R, int G) {
    return (reinterpret_cast<uintptr_t>(p) % (2 * G)) == 0 && (R <= 1 || ld % G == 0);
}

template <int M>
void launch_m(const uint16_t *x, int64_t ldx, const uint16_t *w, float eps, uint16_t *y,
              int64_t ldy, float *rstd, int64_t R, hipStream_t st) {
    constexpr int G = M % 8 == 0 ? 8 : (M % 4 == 0 ? 4 : (M % 2 == 0 ? 2 : 1));
    const bool vec = aligned_to(x, ldx, R, G) && aligned_to(y, ldy, R, G) && aligned_to(w, 0, 1, G);
    if (vec)
        hipLaunchKernelGGL((rmsnorm_fixed_kernel<M, true>), dim3((unsigned)R), dim3(kLanes), 0, st, x,
                           ldx, w, eps, y, ldy, rstd);
    else
        hipLaunchKernelGGL((rmsnorm_fixed_kernel<M, false>), dim3((unsigned)R), dim3(kLanes), 0, st, x,
                           ldx, w, eps, y, ldy, rstd);
}

template <int... Ms>
bool launch_fixed(MList<Ms...>, int M, const uint16_t *x, int64_t ldx, const uint16_t *w,
                  float eps, uint16_t *y, int64_t ldy, float *rstd, int64_t R, hipStream_t st) {
    bool done = false;
    ((M == Ms && !done ? (launch_m<Ms>(x, ldx, w, eps, y, ldy, rstd, R, st), done = true) : false), ...);
    return done;
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
    const dim3 grid((unsigned)R), block(kLanes);
    if (H % kLanes == 0 && launch_fixed(kFixed, (int)(H / kLanes), x, ldx, w, eps, y, ldy, rstd, R, st))
        return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
    const bool vec = aligned16(x, R > 1 ? ldx : 8) && aligned16(y, R > 1 ? ldy : 8) &&
                     aligned16(w, 8);
    if (vec)
        hipLaunchKernelGGL(rmsnorm_any_kernel<true>, grid, block, 0, st, x, ldx, w, eps, y, ldy, rstd,
                           (int)H);
    else
        hipLaunchKernelGGL(rmsnorm_any_kernel<false>, grid, block, 0, st, x, ldx, w, eps, y, ldy,
                           rstd, (int)H);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}
