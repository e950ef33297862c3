// Fused QKV projection with RoPE3D at the global time index and the K/V cache append
// ("Accelerating Video Generation Inference with Sequential-Parallel 3D Positional Encoding
// Using a Global Time Index", section 2.C: the QKV projection and the rotary embedding in one
// kernel, with precomputed tables; section 2.A: keys and values go to the KV cache).
//
// qkv = x W^T + b for the call's tokens, computed as C^T = W x^T with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  With W as the A operand every lane owns
// one token and holds the channels (r % 4) + 8 (r / 4) + 4 (lane / 32) of a 32-channel
// block in its 16 accumulators, so the pairs (2i, 2i + 1) that RoPE rotates are in the same
// lane.  A workgroup computes 128 features x 128 tokens (4 waves of 64 x 64); with
// head_dim 128 the tile is one head of Q, K or V.  W and x tiles of 64 channels go from
// global memory straight to LDS (buffer loads into LDS, XOR-swizzled rows), double-buffered.
// Epilogue: + bias, rotation of Q and K at (t0 + f, h, w) in fp32, one rounding to bf16;
// Q to its output, K to the ring's K rows, V to the ring's transposed V rows.
#include "vdit_bf16.hpp"
#include "vdit_internal.hpp"

namespace vdit {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kPT = 128;                 // tokens and features per tile
constexpr int kPK = 64;                  // hidden channels per k-step
constexpr int kPThreads = 256;           // 4 waves
constexpr int kRowBytes = kPK * 2;       // 128 bytes per tile row
constexpr int kTileBytes = kPT * kRowBytes;  // 16 KB
constexpr int kStage = 2 * kTileBytes;   // W tile, then x tile

struct ProjArgs {
    const uint16_t* x;
    int64_t x_st;  // elements between tokens
    int32_t n_tokens, hidden;
    const uint16_t* w;
    int64_t w_st;  // elements between W rows
    const float* bias;
    int32_t heads, head_dim;
    RopeDev rope;
    int32_t has_rope;
    int32_t hw, wf, t0;
    uint16_t* q;
    int64_t q_st, q_sh;
    uint16_t* kc;
    uint16_t* vt;
    int64_t kv_rows;
    int32_t frame_stride, capacity;
    int32_t feat_tiles, tok_tiles;
};

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Workgroups are dispatched round-robin over the 8 XCDs; each XCD gets a contiguous range of
// tiles (feature tile major), so the W tiles it reads stay in its L2.
__device__ inline int xcd_item(int bid, int total) {
    constexpr int kXcd = 8;
    const int q = total / kXcd, r = total % kXcd, xcd = bid % kXcd, idx = bid / kXcd;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__global__ __launch_bounds__(kPThreads, 2) void qkv_rope_append_kernel(ProjArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
    const int item = xcd_item(blockIdx.x, a.feat_tiles * a.tok_tiles);
    const int n0 = (item / a.tok_tiles) * kPT, m0 = (item % a.tok_tiles) * kPT;

    // DMA: a tile is 16 blocks of 1 KB (8 rows of 128 B); wave w fills blocks 4 i + w.  Lane l
    // writes row l / 8, position l % 8 of a block, i.e. data chunk (l % 8) ^ swz(row), where
    // swz(row) = (row >> 1) & 7 = ((block & 1) << 2) | (rib >> 1) and block & 1 = w & 1.
    const int rib = lane >> 3;
    const int dchunk = (lane & 7) ^ (((wave & 1) << 2) | (rib >> 1));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)(((int64_t)(a.feat_tiles * kPT - 1) * a.w_st + a.hidden) * 2));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(((int64_t)(a.n_tokens - 1) * a.x_st + a.hidden) * 2));
    uint32_t w_off[4], x_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (4 * i + wave) * 8 + rib;
        const int tok = min(m0 + row, a.n_tokens - 1);  // rows past the last token repeat it
        w_off[i] = (uint32_t)((int64_t)(n0 + row) * a.w_st * 2) + dchunk * 16;
        x_off[i] = (uint32_t)((int64_t)tok * a.x_st * 2) + dchunk * 16;
    }
    auto load_stage = [&](int kk, char* st) {
        const uint32_t koff = (uint32_t)kk * kPK * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = 4 * i + wave;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(st + blk * 1024), 16, w_off[i], koff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(st + kTileBytes + blk * 1024), 16, x_off[i],
                                                     koff, 0, 0);
        }
    };

    // fragments: row r of a tile, chunk c (8 channels) at r * 128 + ((c ^ swz(r)) * 16)
    const int sw = (li >> 1) & 7;
    const int wf_row = 64 * (wave & 1) + li;   // W rows of this wave (+ 32 fb)
    const int xt_row = 64 * (wave >> 1) + li;  // x rows of this wave (+ 32 tb)
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int nk = a.hidden / kPK;
    load_stage(0, smem);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int kk = 0; kk < nk; ++kk) {
        char* cur = smem + (kk & 1) * kStage;
        if (kk + 1 < nk) load_stage(kk + 1, smem + ((kk + 1) & 1) * kStage);
#pragma unroll
        for (int j = 0; j < kPK / 16; ++j) {
            const int coff = (((2 * j + g) ^ sw) * 16);
            bf16x8 af[2], bf[2];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                af[f] = *reinterpret_cast<const bf16x8*>(cur + (wf_row + 32 * f) * kRowBytes + coff);
                bf[f] = *reinterpret_cast<const bf16x8*>(cur + kTileBytes + (xt_row + 32 * f) * kRowBytes + coff);
            }
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[f][t] = mfma32(af[f], bf[t], acc[f][t]);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue
    const int hd = a.heads * a.head_dim;
    const int part = n0 / hd;  // 0: Q, 1: K, 2: V (a tile never straddles two)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int m = m0 + 64 * (wave >> 1) + 32 * t + li;
        if (m >= a.n_tokens) continue;
        const int fr = m / a.hw, s = m - fr * a.hw;
        const int tg = a.t0 + fr, ph = s / a.wf, pw = s - ph * a.wf;
        const int64_t phys = (int64_t)(tg % a.capacity) * a.frame_stride + s;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int nb = n0 + 64 * (wave & 1) + 32 * f + 4 * g;  // + (r % 4) + 8 (r / 4)
            const int c0 = nb - part * hd;
            const int h = c0 / a.head_dim, db = c0 - h * a.head_dim;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {  // channels db + 8 q4 + (0..3)
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[e] = acc[f][t][4 * q4 + e];
                    if (a.bias) y[e] += a.bias[nb + 8 * q4 + e];
                }
                const int d = db + 8 * q4;
                if (part < 2 && a.has_rope) {
#pragma unroll
                    for (int e = 0; e < 4; e += 2) rope_apply(rope_cs(a.rope, (d + e) >> 1, tg, ph, pw), y[e], y[e + 1]);
                }
                if (part == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t u = pack_bf16x2(y[e], 0.f);
                        a.vt[((int64_t)h * a.head_dim + d + e) * a.kv_rows + phys] = (uint16_t)(u & 0xffffu);
                    }
                } else {
                    const uint2 u = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                    uint16_t* dst = part == 0 ? a.q + (int64_t)m * a.q_st + (int64_t)h * a.q_sh + d
                                              : a.kc + ((int64_t)h * a.kv_rows + phys) * a.head_dim + d;
                    *reinterpret_cast<uint2*>(dst) = u;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_qkv_rope_append(const ProjLaunch& L, hipStream_t s) {
    ProjArgs a{};
    a.x = static_cast<const uint16_t*>(L.x);
    a.x_st = L.x_st;
    a.n_tokens = L.n_tokens;
    a.hidden = L.hidden;
    a.w = static_cast<const uint16_t*>(L.w);
    a.w_st = L.w_st;
    a.bias = L.bias;
    a.heads = L.heads;
    a.head_dim = L.head_dim;
    a.rope = L.rope;
    a.has_rope = L.has_rope ? 1 : 0;
    a.hw = L.hw;
    a.wf = L.wf;
    a.t0 = L.t0;
    a.q = static_cast<uint16_t*>(L.q);
    a.q_st = L.q_st;
    a.q_sh = L.q_sh;
    a.kc = static_cast<uint16_t*>(L.kc);
    a.vt = static_cast<uint16_t*>(L.vt);
    a.kv_rows = L.kv_rows;
    a.frame_stride = L.frame_stride;
    a.capacity = L.capacity;
    a.feat_tiles = 3 * L.heads * L.head_dim / kPT;
    a.tok_tiles = (L.n_tokens + kPT - 1) / kPT;
    qkv_rope_append_kernel<<<a.feat_tiles * a.tok_tiles, kPThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace vdit
