// Decode attention with a fixed split-KV size (declared in
// include/det_attention.h).
//
// Summary page of "Defeating Nondeterminism in LLM Inference", section on
// batch-invariant kernel design, attention: split-KV stays batch-invariant
// when the split size is fixed.
//
// Two kernels.  attn_split_kernel: one workgroup (256 threads) per (split,
// key/value head, sequence) computes the split's scores for the G query heads
// of the key/value head, its max, its sum of weights and its weighted value
// sum, and writes them to the caller's work buffer.  attn_combine_kernel: one
// workgroup per (query head, sequence) merges the sequence's splits in
// ascending order.  Keys go from global memory straight to the registers of
// the threads that use them; values pass through LDS in 64-row tiles (rows
// padded to 272 bytes so that reads of different rows fall in different
// banks), each tile fetched into registers while the previous one is used.  Every reduction has a fixed shape, so a sequence's bits
// depend only on its own data and length.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "bf16_device.h"
#include "det_attention.h"
#include "device_check.h"

using namespace detgemm;

namespace {

constexpr int kSplit = DET_ATTN_SPLIT;
constexpr int kD = DET_ATTN_HEAD_DIM;
constexpr int kGMax = DET_ATTN_MAX_GROUP;
constexpr int kThreads = 256;
constexpr int kTile = 64;            // positions per LDS tile
constexpr int kRowBytes = kD * 2 + 16;  // padded LDS row of one key or value
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bfv(uint32_t bits16) { return __uint_as_float(bits16 << 16); }


// Positions [p0, p0 + 64) of one head's key or value rows, as this thread's
// four 16-byte chunks (16 per row; rows at or past n are zero): fetched into
// registers one tile ahead of their use, then written to the LDS tile.
constexpr int kPer = kTile * 16 / kThreads;

__device__ __forceinline__ void fetch_tile(uint4 (&v)[kPer], const uint16_t *rows, int p0, int n) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int c = threadIdx.x + i * kThreads;
        const int r = c >> 4, col = c & 15;
        v[i] = p0 + r < n ? *reinterpret_cast<const uint4 *>(rows + (int64_t)(p0 + r) * kD + col * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ void put_tile(char *tile, const uint4 (&v)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int c = threadIdx.x + i * kThreads;
        *reinterpret_cast<uint4 *>(tile + (c >> 4) * kRowBytes + (c & 15) * 16) = v[i];
    }
}

__device__ __forceinline__ bf16x2 as_pair(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// Query rows of a prefill launch, grouped by sequence: sequence q owns rows
// row_start[q] .. row_start[q] + rows[q] - 1 and the launch's tiles
// tile_start[q] .. tile_start[q + 1] - 1, each of `qt` consecutive rows (the
// last one of a sequence possibly fewer).
constexpr int kMaxPrefillSeqs = 128;
struct PrefillTiles {
    int32_t seqs, qt;
    int32_t tile_start[kMaxPrefillSeqs + 1];
    int32_t row_start[kMaxPrefillSeqs];
    int32_t rows[kMaxPrefillSeqs];
};

// GM: the virtual heads of a workgroup, a power of two (the register arrays
// are sized by it).  Decode (PF false): workgroup z is sequence z, and its
// virtual heads are the G query heads of key/value head y.  Prefill (PF true):
// workgroup z is a tile of query rows of one sequence, and its virtual heads
// are the G heads of each of those rows (rows * G <= GM); every virtual head
// has its own length, and the arithmetic of each one is that of a decode
// query with that length.
template <int GM, bool PF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void attn_split_kernel(
    const uint16_t *Q, const uint16_t *K, const uint16_t *V, const int32_t *lens, int Hq, int Hkv,
    int Smax, int G, int NS, float scale_log2, float *work, PrefillTiles pt) {
    __shared__ __attribute__((aligned(16))) float sc[GM][kSplit];
    __shared__ __attribute__((aligned(16))) char tile[kTile * kRowBytes];
    __shared__ float red[GM][kThreads / 64];

    const int s = blockIdx.x, kvh = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int j0 = s * kSplit;
    int seq = blockIdx.z, row0 = blockIdx.z, VG = G;  // sequence, first query row, virtual heads
    if constexpr (PF) {
        int lo = 0, hi = pt.seqs;  // the last sequence whose first tile is <= z
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pt.tile_start[mid] <= (int)blockIdx.z)
                lo = mid;
            else
                hi = mid;
        }
        seq = lo;
        const int k = blockIdx.z - pt.tile_start[lo];
        row0 = pt.row_start[lo] + k * pt.qt;
        const int nrows = pt.rows[lo] - k * pt.qt < pt.qt ? pt.rows[lo] - k * pt.qt : pt.qt;
        VG = nrows * G;
    }
    // per virtual head v: its query row and head, and its positions in this split
    int nv[GM];
    int n = 0;
#pragma unroll
    for (int v = 0; v < GM; ++v) {
        nv[v] = 0;
        if (v < VG) {
            int len = lens[row0 + v / G];
            len = len < 0 ? 0 : (len > Smax ? Smax : len);
            nv[v] = len - j0 <= 0 ? 0 : (len - j0 < kSplit ? len - j0 : kSplit);
            n = nv[v] > n ? nv[v] : n;
        }
    }
    if (n == 0)
        return;  // the whole workgroup: no barrier is reached
    const int64_t head = ((int64_t)seq * Hkv + kvh) * Smax;
    const uint16_t *Kh = K + (head + j0) * kD, *Vh = V + (head + j0) * kD;

    // ---- scores.  Lane l of wave w holds the 16-byte chunk cc = l % 16 of
    // four key rows of a tile, rows w * 16 + 4c + l / 16 for c = 0..3, so each
    // of its four loads reads 1 KB of whole rows; its q chunk cc of every
    // head stays in four registers.  The score of a row is the sum over the
    // 16 chunks of each chunk's 4-pair v_dot2 chain (pairs in ascending
    // order), the chunks meeting in a balanced tree: cc with cc ^ 8 first,
    // then ^ 4, ^ 2, ^ 1.  The first two levels spread the four rows over the
    // lanes (bit 3 of the lane picks rows 2,3 over rows 0,1, bit 2 the odd
    // row), so each lane ends with one row's score.
    const int cc = lane & 15, rq = lane >> 4;
    const int h3 = (lane >> 3) & 1, h2 = (lane >> 2) & 1;
    const int myrow = wave * 16 + (2 * h3 + h2) * 4 + rq;  // the row whose score this lane ends with
    uint32_t qc[GM][4];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (g < VG)
            v = *reinterpret_cast<const uint4 *>(
                Q + ((int64_t)(row0 + g / G) * Hq + kvh * G + g % G) * kD + cc * 8);
        qc[g][0] = v.x;
        qc[g][1] = v.y;
        qc[g][2] = v.z;
        qc[g][3] = v.w;
    }
    const int ntiles = (n + kTile - 1) / kTile;
    auto key_chunks = [&](uint4 (&kv)[4], int sub) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int row = sub * kTile + wave * 16 + c * 4 + rq;
            kv[c] = row < n ? *reinterpret_cast<const uint4 *>(Kh + (int64_t)row * kD + cc * 8)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    uint4 kcur[4], knext[4];
    key_chunks(knext, 0);
    for (int sub = 0; sub < ntiles; ++sub) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            kcur[c] = knext[c];
        if (sub + 1 < ntiles)
            key_chunks(knext, sub + 1);
        const int j = sub * kTile + myrow;
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < VG) {
                float part[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t kw[4] = {kcur[c].x, kcur[c].y, kcur[c].z, kcur[c].w};
                    float x = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x = __builtin_amdgcn_fdot2_f32_bf16(as_pair(qc[g][e]), as_pair(kw[e]), x, false);
                    part[c] = x;
                }
                // level cc ^ 8: keep rows 2 h3, 2 h3 + 1, hand the other two over
                const float s0 = h3 ? part[0] : part[2], s1 = h3 ? part[1] : part[3];
                const float k0 = h3 ? part[2] : part[0], k1 = h3 ? part[3] : part[1];
                const float a0 = k0 + __shfl_xor(s0, 8, 64), a1 = k1 + __shfl_xor(s1, 8, 64);
                // level cc ^ 4: keep row 2 h3 + h2
                float v = (h2 ? a1 : a0) + __shfl_xor(h2 ? a0 : a1, 4, 64);
                v = v + __shfl_xor(v, 2, 64);
                v = v + __shfl_xor(v, 1, 64);
                if ((lane & 3) == 0)
                    sc[g][j] = j < nv[g] ? v * scale_log2 : -__builtin_inff();
            }
        }
    }
    uint4 nxt[kPer];
    fetch_tile(nxt, Vh, 0, n);  // the first value tile, in flight through the softmax
    // slots past the last tile read are empty
    for (int i = t; i < VG * kSplit; i += kThreads)
        if (i % kSplit >= ntiles * kTile)
            sc[i / kSplit][i % kSplit] = -__builtin_inff();
    __syncthreads();
    // ---- per head: max, weights, pairwise sum of the 256 weight slots
    float m[GM], l[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g >= VG)
            break;
        float x = sc[g][t];
#pragma unroll
        for (int k = 1; k < 64; k <<= 1)
            x = fmaxf(x, __shfl_xor(x, k, 64));
        if (lane == 0)
            red[g][wave] = x;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g >= VG)
            break;
        m[g] = fmaxf(fmaxf(red[g][0], red[g][1]), fmaxf(red[g][2], red[g][3]));
        const float p = t < nv[g] ? exp2f(sc[g][t] - m[g]) : 0.0f;
        sc[g][t] = p;
        float x = p;
#pragma unroll
        for (int k = 1; k < 64; k <<= 1)
            x = x + __shfl_xor(x, k, 64);
        l[g] = x;
    }
    __syncthreads();  // every max read from red before it is reused
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g >= VG)
            break;
        if (lane == 0)
            red[g][wave] = l[g];
    }
    // ---- weighted values: output pair o = t, t + 256 (head o / 64, columns
    // 2 (o % 64) and 2 (o % 64) + 1); positions in ascending order, four
    // weights read at a time
    float acc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
    const int npairs = VG * (kD / 2);
    int nown[2];  // the length of the virtual head of output pair i (static selects)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int g = (t + i * kThreads) >> 6;
        nown[i] = 0;
#pragma unroll
        for (int v = 0; v < GM; ++v)
            nown[i] = v == g ? nv[v] : nown[i];
    }
    for (int sub = 0; sub < ntiles; ++sub) {
        __syncthreads();
        put_tile(tile, nxt);
        if (sub + 1 < ntiles)
            fetch_tile(nxt, Vh, (sub + 1) * kTile, n);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int o = t + i * kThreads;
            if (o < npairs) {
                const int g = o >> 6, dp = o & 63;
                const float *pw = &sc[g][sub * kTile];
#pragma unroll 4
                for (int rr = 0; rr < kTile; rr += 4) {
                    const float4 w4 = *reinterpret_cast<const float4 *>(pw + rr);
                    const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t vv =
                            *reinterpret_cast<const uint32_t *>(tile + (rr + u) * kRowBytes + dp * 4);
                        // Prefill: the value rows of a longer row of the tile, past
                        // this head's length, are skipped (a decode query of that
                        // length sees zero rows there, which leave acc unchanged).
                        if (!PF || sub * kTile + rr + u < nown[i]) {
                            acc[i][0] = fmaf(wv[u], bfv(vv & 0xFFFFu), acc[i][0]);
                            acc[i][1] = fmaf(wv[u], bfv(vv >> 16), acc[i][1]);
                        }
                    }
                }
            }
        }
    }
    __syncthreads();  // the l values in red
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int o = t + i * kThreads;
        if (o < npairs) {
            const int g = o >> 6, dp = o & 63;
            float *w = work + (((int64_t)(row0 + g / G) * Hq + kvh * G + g % G) * NS + s) * (kD + 2);
            w[2 * dp] = acc[i][0];
            w[2 * dp + 1] = acc[i][1];
            if (dp == 0) {
                w[kD] = m[g];
                w[kD + 1] = (red[g][0] + red[g][1]) + (red[g][2] + red[g][3]);
            }
        }
    }
}

// One workgroup of 128 threads (one per column) per (query head, sequence).
// The partials are read kChunk splits at a time, all loads of a chunk issued
// before its arithmetic, so a sequence waits for memory once per chunk and
// not once per split; the max and the two sums still run over the splits in
// ascending order.
constexpr int kChunk = 16;

__global__ __launch_bounds__(kD) void attn_combine_kernel(const int32_t *lens, int Hq, int Smax,
                                                          int NS, const float *work, uint16_t *O) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    int len = lens[b];
    len = len < 0 ? 0 : (len > Smax ? Smax : len);
    const int ns = (len + kSplit - 1) / kSplit;
    uint16_t *o = O + ((int64_t)b * Hq + h) * kD;
    if (ns == 0) {
        o[d] = 0;
        return;
    }
    const float *w = work + ((int64_t)b * Hq + h) * NS * (kD + 2);
    float M = w[kD];
    for (int s0 = 1; s0 < ns; s0 += kChunk) {
        float m[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            m[i] = s0 + i < ns ? w[(int64_t)(s0 + i) * (kD + 2) + kD] : 0.0f;
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            if (s0 + i < ns)
                M = fmaxf(M, m[i]);
    }
    float L = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += kChunk) {
        float m[kChunk], l[kChunk], v[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const float *ws = w + (int64_t)(s0 + i) * (kD + 2);
            const bool in = s0 + i < ns;
            m[i] = in ? ws[kD] : 0.0f;
            l[i] = in ? ws[kD + 1] : 0.0f;
            v[i] = in ? ws[d] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            if (s0 + i < ns) {
                const float f = exp2f(m[i] - M);
                L = fmaf(l[i], f, L);
                acc = fmaf(v[i], f, acc);
            }
    }
    o[d] = (uint16_t)pair_bits(round_pair(acc / L, 0.0f));
}

bool disjoint(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return na <= 0 || nb <= 0 || a0 + (uintptr_t)na <= b0 || b0 + (uintptr_t)nb <= a0;
}

// ---- the allocation-free variant: the per-split partials in a file-scope
// device array instead of a caller's buffer.  Each device the library runs on
// holds its own copy until the process ends; its address on a device is taken
// once, with that device current, and used from then on (the array's name is a
// host-side stand-in, not a device address).
constexpr int64_t kScratchFloats = DET_ATTN_SCRATCH_FLOATS;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices];

// The current device's copy of `scratch`, or nullptr on a runtime error.
float *scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        g_scratch[dev] = static_cast<float *>(p);
    }
    return g_scratch[dev];
}

// Shape checks shared by both entry points; NS receives the split count.
int check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Smax, int64_t D, int64_t &NS) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Smax < 0 || D != kD || Hq % Hkv != 0 ||
        Hq / Hkv > kGMax || B > 65535 || Hkv > 65535 || Hq > 65535 || Smax > (1 << 24))
        return DET_GEMM_EINVAL;
    NS = (Smax + kSplit - 1) / kSplit;
    return DET_GEMM_OK;
}

int run_attention(const det_bf16 *Q, const det_bf16 *K, const det_bf16 *V, const int32_t *lens,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Smax, int64_t NS, float scale,
                  float *work, det_bf16 *O, void *stream) {
    if (!Q || !lens || !O || (NS > 0 && (!K || !V || !work)))
        return DET_GEMM_EINVAL;
    const int64_t qb = B * Hq * kD * 2, kvb = B * Hkv * Smax * kD * 2;
    const int64_t wb = B * Hq * NS * (kD + 2) * 4;
    if (!disjoint(O, qb, Q, qb) || !disjoint(O, qb, K, kvb) || !disjoint(O, qb, V, kvb) ||
        !disjoint(O, qb, lens, B * 4) || !disjoint(O, qb, work, wb) ||
        !disjoint(work, wb, Q, qb) || !disjoint(work, wb, K, kvb) || !disjoint(work, wb, V, kvb) ||
        !disjoint(work, wb, lens, B * 4))
        return DET_GEMM_EINVAL;
    if (((reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15) != 0)
        return DET_GEMM_EINVAL;  // 16-byte rows
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int G = (int)(Hq / Hkv);
    if (NS > 0) {
        const dim3 grid((unsigned)NS, (unsigned)Hkv, (unsigned)B);
        const float sl = scale * kLog2e;
        PrefillTiles none;
        std::memset(&none, 0, sizeof none);
        if (G == 1)
            hipLaunchKernelGGL((attn_split_kernel<1, false>), grid, dim3(kThreads), 0, st, Q, K, V,
                               lens, (int)Hq, (int)Hkv, (int)Smax, G, (int)NS, sl, work, none);
        else if (G == 2)
            hipLaunchKernelGGL((attn_split_kernel<2, false>), grid, dim3(kThreads), 0, st, Q, K, V,
                               lens, (int)Hq, (int)Hkv, (int)Smax, G, (int)NS, sl, work, none);
        else if (G <= 4)
            hipLaunchKernelGGL((attn_split_kernel<4, false>), grid, dim3(kThreads), 0, st, Q, K, V,
                               lens, (int)Hq, (int)Hkv, (int)Smax, G, (int)NS, sl, work, none);
        else
            hipLaunchKernelGGL((attn_split_kernel<8, false>), grid, dim3(kThreads), 0, st, Q, K, V,
                               lens, (int)Hq, (int)Hkv, (int)Smax, G, (int)NS, sl, work, none);
    }
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)Hq, (unsigned)B), dim3(kD), 0, st, lens,
                       (int)Hq, (int)Smax, (int)NS, work, O);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

}  // namespace

extern "C" int det_attention_decode(const det_bf16 *Q, const det_bf16 *K, const det_bf16 *V,
                                    const int32_t *lens, int64_t B, int64_t Hq, int64_t Hkv,
                                    int64_t Smax, int64_t D, float scale, float *work,
                                    det_bf16 *O, void *stream) {
    int64_t NS = 0;
    const int rc = check_shape(B, Hq, Hkv, Smax, D, NS);
    if (rc != DET_GEMM_OK || B == 0)
        return rc;
    return run_attention(Q, K, V, lens, B, Hq, Hkv, Smax, NS, scale, work, O, stream);
}

extern "C" int det_attention_prefill(const det_bf16 *Q, const det_bf16 *K, const det_bf16 *V,
                                     const int64_t *row_offsets, const int32_t *lens, int64_t NQ,
                                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Smax, int64_t D,
                                     float scale, float *work, det_bf16 *O, void *stream) {
    int64_t NS = 0;
    int rc = check_shape(B, Hq, Hkv, Smax, D, NS);
    if (rc != DET_GEMM_OK)
        return rc;
    if (NQ < 0 || NQ > 65535 || B > kMaxPrefillSeqs || !row_offsets)
        return DET_GEMM_EINVAL;
    if (row_offsets[0] != 0 || row_offsets[B] != NQ)
        return DET_GEMM_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (row_offsets[b + 1] < row_offsets[b])
            return DET_GEMM_EINVAL;
    if (NQ == 0)
        return DET_GEMM_OK;
    if (!Q || !lens || !O || (NS > 0 && (!K || !V || !work)))
        return DET_GEMM_EINVAL;
    const int64_t qb = NQ * Hq * kD * 2, kvb = B * Hkv * Smax * kD * 2;
    const int64_t wb = NQ * Hq * NS * (kD + 2) * 4;
    if (!disjoint(O, qb, Q, qb) || !disjoint(O, qb, K, kvb) || !disjoint(O, qb, V, kvb) ||
        !disjoint(O, qb, lens, NQ * 4) || !disjoint(O, qb, work, wb) ||
        !disjoint(work, wb, Q, qb) || !disjoint(work, wb, K, kvb) || !disjoint(work, wb, V, kvb) ||
        !disjoint(work, wb, lens, NQ * 4))
        return DET_GEMM_EINVAL;
    if (((reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15) != 0)
        return DET_GEMM_EINVAL;  // 16-byte rows
    const int dev = check_device();
    if (dev != DET_GEMM_OK)
        return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int G = (int)(Hq / Hkv);
    if (NS > 0) {
        // tiles of qt consecutive rows of one sequence: qt * G <= 8 virtual heads
        PrefillTiles pt;
        std::memset(&pt, 0, sizeof pt);
        pt.seqs = (int32_t)B;
        pt.qt = kGMax / G;
        int64_t tiles = 0;
        for (int64_t b = 0; b < B; ++b) {
            const int64_t rows = row_offsets[b + 1] - row_offsets[b];
            pt.tile_start[b] = (int32_t)tiles;
            pt.row_start[b] = (int32_t)row_offsets[b];
            pt.rows[b] = (int32_t)rows;
            tiles += (rows + pt.qt - 1) / pt.qt;
        }
        pt.tile_start[B] = (int32_t)tiles;
        if (tiles > 65535)
            return DET_GEMM_EINVAL;
        if (tiles > 0)
            hipLaunchKernelGGL((attn_split_kernel<kGMax, true>),
                               dim3((unsigned)NS, (unsigned)Hkv, (unsigned)tiles), dim3(kThreads), 0,
                               st, Q, K, V, lens, (int)Hq, (int)Hkv, (int)Smax, G, (int)NS,
                               scale * kLog2e, work, pt);
    }
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)Hq, (unsigned)NQ), dim3(kD), 0, st, lens,
                       (int)Hq, (int)Smax, (int)NS, work, O);
    return hipGetLastError() == hipSuccess ? DET_GEMM_OK : DET_GEMM_EHIP;
}

extern "C" int det_attention_decode_noalloc(const det_bf16 *Q, const det_bf16 *K,
                                            const det_bf16 *V, const int32_t *lens, int64_t B,
                                            int64_t Hq, int64_t Hkv, int64_t Smax, int64_t D,
                                            float scale, det_bf16 *O, void *stream) {
    int64_t NS = 0;
    const int rc = check_shape(B, Hq, Hkv, Smax, D, NS);
    if (rc != DET_GEMM_OK || B == 0)
        return rc;
    // B, Hq <= 65535 and NS <= 2^16: the product fits in int64
    if (B * Hq * NS * (kD + 2) > kScratchFloats)
        return DET_ATTN_ESCRATCH;
    if (check_device() != DET_GEMM_OK)
        return DET_GEMM_EHIP;
    float *work = scratch_on_current_device();
    if (!work)
        return DET_GEMM_EHIP;
    return run_attention(Q, K, V, lens, B, Hq, Hkv, Smax, NS, scale, work, O, stream);
}
