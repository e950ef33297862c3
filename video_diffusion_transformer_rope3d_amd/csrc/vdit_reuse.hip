// Block-wise feature reuse indicator ("BWCache: Accelerating Video Diffusion Transformers
// through Block-Wise Caching", section 2, dynamic similarity indicator): for every block b of
// a DiT, the relative L1 distance sum |F_t - F_{t-1}| / sum |F_{t-1}| between its features
// at two consecutive timesteps, and the mean over the blocks.
//
// A streaming reduction, bound by HBM: every element of both feature sets is read once with
// 16-byte non-temporal loads, four steps of loads in flight per thread.  Pass 1: a workgroup
// sums |cur - prev| and |prev| over one chunk of one block in fp32 (per-thread runs, then a
// tree over the workgroup).  Pass 2: one workgroup adds each block's chunk sums in fp64 in a
// fixed order (deterministic, no atomics), divides, and averages over the blocks.
#include <utility>

#include "vdit_internal.hpp"

namespace vdit {

namespace {

constexpr int kReuseThreads = 256;
constexpr int kVec = 8;                               // elements per 16-byte bf16 load
constexpr int64_t kChunk = kReuseThreads * kVec * 16;  // elements per workgroup of pass 1

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// Eight consecutive elements as floats.  The features are read once: non-temporal loads keep
// them from displacing other data in the caches.
__device__ inline void load8f(const void* base, int64_t off, bool f32, float (&x)[8]) {
    if (f32) {
        const f32x4v* p = reinterpret_cast<const f32x4v*>(static_cast<const float*>(base) + off);
        const f32x4v a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
    } else {
        const u32x4v u =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(static_cast<const uint16_t*>(base) + off));
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(w[k] << 16);
            x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
}

__device__ inline float load1f(const void* base, int64_t off, bool f32) {
    return f32 ? static_cast<const float*>(base)[off]
               : __uint_as_float((uint32_t) static_cast<const uint16_t*>(base)[off] << 16);
}

template <class T>
__device__ inline T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Pass 1: workgroup (p, b) sums elements [p kChunk, (p + 1) kChunk) of block b.
template <bool F32>
__global__ __launch_bounds__(kReuseThreads) void rel_l1_partial_kernel(const void* cur, const void* prev,
                                                                       int64_t block_elems, int64_t block_stride,
                                                                       int32_t chunks, float2* part) {
    __shared__ float2 s_red[kReuseThreads / 64];
    const int p = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int64_t base = (int64_t)b * block_stride, lo = (int64_t)p * kChunk;
    const int64_t hi = lo + kChunk < block_elems ? lo + kChunk : block_elems;
    float num = 0.f, den = 0.f;
    // full vectors: every 16-byte load lies inside the block; the loads of U steps are issued
    // before their arithmetic
    const int64_t vhi = lo + (hi - lo) / kVec * kVec;
    constexpr int U = 4;
    constexpr int64_t kStep = kReuseThreads * kVec;
    auto accumulate = [&](const float (&x)[8], const float (&y)[8]) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            num += fabsf(x[k] - y[k]);
            den += fabsf(y[k]);
        }
    };
    int64_t e = lo + (int64_t)t * kVec;
    for (; e + (U - 1) * kStep < vhi; e += U * kStep) {
        float x[U][8], y[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            load8f(cur, base + e + u * kStep, F32, x[u]);
            load8f(prev, base + e + u * kStep, F32, y[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) accumulate(x[u], y[u]);
    }
    for (; e < vhi; e += kStep) {
        float x[8], y[8];
        load8f(cur, base + e, F32, x);
        load8f(prev, base + e, F32, y);
        accumulate(x, y);
    }
    // ragged end of the block (fewer than 8 elements)
    for (int64_t e = vhi + t; e < hi; e += kReuseThreads) {
        const float x = load1f(cur, base + e, F32), y = load1f(prev, base + e, F32);
        num += fabsf(x - y);
        den += fabsf(y);
    }
    num = wave_sum(num);
    den = wave_sum(den);
    if ((t & 63) == 0) s_red[t >> 6] = make_float2(num, den);
    __syncthreads();
    if (t == 0) {
        float2 r = s_red[0];
        for (int w = 1; w < kReuseThreads / 64; ++w) r.x += s_red[w].x, r.y += s_red[w].y;
        part[(size_t)b * chunks + p] = r;
    }
}

// Pass 2: one workgroup of 16 waves; wave w takes blocks w, w + 16, ...: the block's chunk
// sums in fp64 (lane-strided, then a shuffle tree), its ratio; the mean adds the waves' sums
// in wave order (deterministic).
constexpr int kFinalThreads = 1024;
__global__ __launch_bounds__(kFinalThreads) void rel_l1_final_kernel(const float2* part, int32_t chunks,
                                                                     int32_t n_blocks, float* out) {
    constexpr int W = kFinalThreads / 64;
    __shared__ double s_sum[W];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double wsum = 0.0;
    for (int b = wave; b < n_blocks; b += W) {
        double num = 0.0, den = 0.0;
        for (int p = lane; p < chunks; p += 64) {
            const float2 v = part[(size_t)b * chunks + p];
            num += v.x;
            den += v.y;
        }
        num = wave_sum(num);
        den = wave_sum(den);
        const double r = den > 0.0 ? num / den : (num == 0.0 ? 0.0 : (double)INFINITY);
        if (lane == 0) out[b] = (float)r;
        wsum += r;
    }
    if (lane == 0) s_sum[wave] = wsum;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < W; ++w) tot += s_sum[w];
        out[n_blocks] = (float)(tot / n_blocks);
    }
}

}  // namespace

int64_t rel_l1_chunks(int64_t block_elems) { return block_elems > 0 ? (block_elems + kChunk - 1) / kChunk : 1; }

size_t rel_l1_workspace_bytes(int32_t n_blocks, int64_t block_elems) {
    return (size_t)rel_l1_chunks(block_elems) * n_blocks * sizeof(float2);
}

hipError_t launch_rel_l1(const void* cur, const void* prev, bool f32, int32_t n_blocks, int64_t block_elems,
                         int64_t block_stride, float* out, void* workspace, hipStream_t s) {
    const int32_t chunks = (int32_t)rel_l1_chunks(block_elems);
    float2* part = static_cast<float2*>(workspace);
    const dim3 grid(chunks, n_blocks);
    if (f32)
        rel_l1_partial_kernel<true><<<grid, kReuseThreads, 0, s>>>(cur, prev, block_elems, block_stride, chunks, part);
    else
        rel_l1_partial_kernel<false><<<grid, kReuseThreads, 0, s>>>(cur, prev, block_elems, block_stride, chunks, part);
    rel_l1_final_kernel<<<1, kFinalThreads, 0, s>>>(part, chunks, n_blocks, out);
    return hipGetLastError();
}

}  // namespace vdit
