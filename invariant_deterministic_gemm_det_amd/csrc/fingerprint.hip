// Tensor fingerprints and the first-mismatch comparator (declared in
// include/det_fingerprint.h).
//
// Reading notes "Bitwise-Deterministic Pretraining at Scale", section
// "5. Fingerprinting Tensors on the GPU": bit-pattern digests computed in GPU
// memory, per-row digests for order-sensitive data, a byte-level comparison
// to settle a difference.
//
// All three are streaming reads of HBM: 16-byte loads per lane, several in
// flight per thread, and one integer reduction at the end of each workgroup.
// The digest terms combine by addition mod 2^64 and the mismatch by minimum,
// both associative and commutative, so the workgroups may finish in any
// order: the integer atomics that merge them give the same bits every run.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "det_fingerprint.h"
#include "device_check.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte chunks in flight per thread (comparator, rows)
constexpr int kUnrollDigest = 8;
constexpr int64_t kMaxBlocks = 4096;

// A 16-byte chunk of a buffer read once.  NT: a non-temporal load (measured:
// the whole-buffer digest and the comparator gain 7 and 9 %; the row digests,
// one wave per row, do not, and keep plain loads).
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
template <bool NT = true>
__device__ __forceinline__ uint4 load_once(const uint4 *q) {
    if constexpr (NT) {
        const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(q));
        return make_uint4(v[0], v[1], v[2], v[3]);
    } else {
        return *q;
    }
}

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

// Word i of n bytes at p (any alignment), bytes past n read as 0.
__device__ __forceinline__ uint64_t word_bytes(const uint8_t *p, int64_t n, int64_t i) {
    uint64_t w = 0;
    for (int b = 0; b < 8; ++b) {
        const int64_t k = 8 * i + b;
        if (k < n)
            w |= (uint64_t)p[k] << (8 * b);
    }
    return w;
}

// The terms of the chunk's two words; g = GAMMA * (first word's index + 1).
__device__ __forceinline__ uint64_t chunk_terms(uint4 v, uint64_t g) {
    const uint64_t w0 = (uint64_t)v.x | ((uint64_t)v.y << 32);
    const uint64_t w1 = (uint64_t)v.z | ((uint64_t)v.w << 32);
    return mix64(w0 + g) + mix64(w1 + g + kGamma);
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t s) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        s += __shfl_xor(s, m, 64);
    return s;
}

__device__ __forceinline__ unsigned long long wave_min(unsigned long long s) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const unsigned long long o = __shfl_xor(s, m, 64);
        s = o < s ? o : s;
    }
    return s;
}

// This thread's part of S: the terms of chunks first, first + stride, ...
// (two words each) when the bytes are 16-byte aligned (VEC), then the words
// past the last whole chunk (or all words) from single bytes.  The position
// term advances by a constant from one chunk of the thread to the next.
template <bool VEC, int U, bool NT>
__device__ __forceinline__ uint64_t partial_sum(const uint8_t *p, int64_t n, int64_t first,
                                                int64_t stride) {
    const int64_t W = (n + 7) / 8;
    uint64_t s = 0;
    int64_t wdone = 0;  // words covered by whole chunks
    if constexpr (VEC) {
        const int64_t C = n / 16;  // chunks entirely inside the bytes
        const uint4 *q = reinterpret_cast<const uint4 *>(p);
        const uint64_t step = kGamma * (uint64_t)(2 * stride);
        uint64_t g = kGamma * (uint64_t)(2 * first + 1);
        int64_t c = first;
        for (; c + (U - 1) * stride < C; c += U * stride) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = load_once<NT>(q + c + u * stride);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                s += chunk_terms(v[u], g);
                g += step;
            }
        }
        for (; c < C; c += stride) {
            s += chunk_terms(load_once<NT>(q + c), g);
            g += step;
        }
        wdone = 2 * C;
    }
    for (int64_t i = wdone + first; i < W; i += stride)
        s += mix64(word_bytes(p, n, i) + kGamma * (uint64_t)(i + 1));
    return s;
}

__global__ void fill_kernel(unsigned long long *x, unsigned long long v) { *x = v; }

template <bool VEC>
__global__ __launch_bounds__(kThreads) void digest_sum_kernel(const uint8_t *p, int64_t n,
                                                              unsigned long long *acc) {
    __shared__ uint64_t part[kThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint64_t s = partial_sum<VEC, kUnrollDigest, true>(p, n, (int64_t)blockIdx.x * kThreads + threadIdx.x,
                                                        stride);
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int w = 0; w < kThreads / 64; ++w)
            t += part[w];
        atomicAdd(acc, (unsigned long long)t);
    }
}

__global__ void digest_final_kernel(unsigned long long *acc, int64_t n) {
    *acc = mix64(*acc + (uint64_t)n);
}

// One wave per row.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void digest_rows_kernel(const uint8_t *p, int64_t rows,
                                                               int64_t row_bytes, int64_t ld,
                                                               uint64_t *out) {
    const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (r >= rows)
        return;
    const uint64_t s =
        wave_sum(partial_sum<VEC, kUnroll, false>(p + r * ld, row_bytes, threadIdx.x & 63, 64));
    if ((threadIdx.x & 63) == 0)
        out[r] = mix64(s + (uint64_t)row_bytes);
}

// First differing byte of the 16-byte chunk pair, or ~0.
__device__ __forceinline__ unsigned long long chunk_mismatch(uint4 x, uint4 y, int64_t c) {
    const uint32_t d[4] = {x.x ^ y.x, x.y ^ y.y, x.z ^ y.z, x.w ^ y.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (d[k])
            return (unsigned long long)(16 * c + 4 * k + (__builtin_ctz(d[k]) >> 3));
    return ~0ull;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void mismatch_kernel(const uint8_t *a, const uint8_t *b,
                                                            int64_t n, unsigned long long *out) {
    __shared__ unsigned long long part[kThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    unsigned long long best = ~0ull;
    int64_t bdone = 0;  // bytes covered by whole chunks
    if constexpr (VEC) {
        const int64_t C = n / 16;
        const uint4 *qa = reinterpret_cast<const uint4 *>(a);
        const uint4 *qb = reinterpret_cast<const uint4 *>(b);
        // a thread's chunks ascend, so its first difference is its smallest
        for (int64_t c = first; c < C && best == ~0ull; c += kUnroll * stride) {
            uint4 va[kUnroll], vb[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t cu = c + u * stride;
                va[u] = cu < C ? load_once(qa + cu) : uint4{0u, 0u, 0u, 0u};
                vb[u] = cu < C ? load_once(qb + cu) : uint4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const unsigned long long m = chunk_mismatch(va[u], vb[u], c + u * stride);
                best = m < best ? m : best;
            }
        }
        bdone = 16 * C;
    }
    for (int64_t k = bdone + first; k < n && best == ~0ull; k += stride)
        if (a[k] != b[k])
            best = (unsigned long long)k;
    best = wave_min(best);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long t = ~0ull;
        for (int w = 0; w < kThreads / 64; ++w)
            t = part[w] < t ? part[w] : t;
        if (t != ~0ull)
            atomicMin(out, t);
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool disjoint(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return na <= 0 || nb <= 0 || a0 + (uintptr_t)na <= b0 || b0 + (uintptr_t)nb <= a0;
}

int64_t grid_for(int64_t units, int unroll) {
    const int64_t g = (units + (int64_t)kThreads * unroll - 1) / ((int64_t)kThreads * unroll);
    return g < 1 ? 1 : (g > kMaxBlocks ? kMaxBlocks : g);
}

int launched() { return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP; }

}  // namespace

extern "C" {

int det_fingerprint(const void *data, int64_t nbytes, uint64_t *digest, void *stream) {
    if (nbytes < 0 || !digest || (nbytes > 0 && !data) || !disjoint(data, nbytes, digest, 8))
        return DET_GEMM_EINVAL;
    const int dev = detgemm::check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    unsigned long long *acc = reinterpret_cast<unsigned long long *>(digest);
    const uint8_t *p = static_cast<const uint8_t *>(data);
    hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(1), 0, st, acc, 0ull);
    if (nbytes > 0) {
        const dim3 grid((unsigned)grid_for((nbytes + 15) / 16, kUnrollDigest));
        if (aligned16(p))
            hipLaunchKernelGGL(digest_sum_kernel<true>, grid, dim3(kThreads), 0, st, p, nbytes, acc);
        else
            hipLaunchKernelGGL(digest_sum_kernel<false>, grid, dim3(kThreads), 0, st, p, nbytes,
                               acc);
    }
    hipLaunchKernelGGL(digest_final_kernel, dim3(1), dim3(1), 0, st, acc, nbytes);
    return launched();
}

int det_fingerprint_rows(const void *data, int64_t rows, int64_t row_bytes, int64_t ld_bytes,
                         uint64_t *digests, void *stream) {
    if (rows < 0 || row_bytes < 0 || (rows > 1 && ld_bytes < row_bytes))
        return DET_GEMM_EINVAL;
    if (rows == 0)
        return DET_GEMM_OK;
    if (!digests || (row_bytes > 0 && !data))
        return DET_GEMM_EINVAL;
    const int64_t span = rows > 1 ? (rows - 1) * ld_bytes + row_bytes : row_bytes;
    if (!disjoint(data, span, digests, rows * 8))
        return DET_GEMM_EINVAL;
    const int64_t blocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks > 0x7FFFFFFF)
        return DET_GEMM_EINVAL;
    const int dev = detgemm::check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint8_t *p = static_cast<const uint8_t *>(data);
    const bool vec = aligned16(p) && (rows == 1 || ld_bytes % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(digest_rows_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                           p, rows, row_bytes, ld_bytes, digests);
    else
        hipLaunchKernelGGL(digest_rows_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           st, p, rows, row_bytes, ld_bytes, digests);
    return launched();
}

int det_first_mismatch(const void *a, const void *b, int64_t nbytes, int64_t *index,
                       void *stream) {
    if (nbytes < 0 || !index || (nbytes > 0 && (!a || !b)) || !disjoint(a, nbytes, index, 8) ||
        !disjoint(b, nbytes, index, 8))
        return DET_GEMM_EINVAL;
    const int dev = detgemm::check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    unsigned long long *out = reinterpret_cast<unsigned long long *>(index);
    // ~0 read as int64 is -1: the answer when nothing differs
    hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(1), 0, st, out, ~0ull);
    if (nbytes > 0) {
        const uint8_t *pa = static_cast<const uint8_t *>(a), *pb = static_cast<const uint8_t *>(b);
        const dim3 grid((unsigned)grid_for((nbytes + 15) / 16, kUnroll));
        if (aligned16(pa) && aligned16(pb))
            hipLaunchKernelGGL(mismatch_kernel<true>, grid, dim3(kThreads), 0, st, pa, pb, nbytes,
                               out);
        else
            hipLaunchKernelGGL(mismatch_kernel<false>, grid, dim3(kThreads), 0, st, pa, pb, nbytes,
                               out);
    }
    return launched();
}

}  // extern "C"
