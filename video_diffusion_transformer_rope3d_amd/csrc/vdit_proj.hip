// Fused QKV projection with RoPE3D at the global time index and the K/V cache append
// ("Accelerating Video Generation Inference with Sequential-Parallel 3D Positional Encoding
// Using a Global Time Index", section 2.C: the QKV projection and the rotary embedding in one
// kernel, with precomputed tables; section 2.A: keys and values go to the KV cache).
//
// qkv = x W^T + b for the call's tokens, computed as C^T = W x^T with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  With W as the A operand every lane owns
// one token and holds the channels (r % 4) + 8 (r / 4) + 4 (lane / 32) of a 32-channel
// block in its 16 accumulators, so the pairs (2i, 2i + 1) that RoPE rotates are in the same
// lane.  A workgroup computes 128 features x 192 tokens (4 waves of 64 x 96); with
// head_dim 128 the features are one head of Q, K or V.  W and x tiles of 64 channels go from
// global memory straight to LDS (buffer loads into LDS, XOR-swizzled rows) in two stages, so
// the loads of the next k-step are in flight while one is computed.  The bytes a k-step moves
// into LDS are what bounds the loop, so the token tile is as long as two 40 KB stages allow at
// two workgroups per CU (80 KB of LDS each); one's epilogue and barrier waits overlap the
// other's MFMAs.
// Epilogue: + bias, rotation of Q and K at (t0 + f, h, w) in fp32, one rounding to bf16;
// Q to its output, K to the ring's K rows, V to the ring's transposed V rows.
#include "vdit_bf16.hpp"
#include "vdit_internal.hpp"

namespace vdit {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kPN = 128;                 // features per tile
constexpr int kPM = 192;                 // tokens per tile
constexpr int kPK = 64;                  // hidden channels per k-step
constexpr int kPWaves = 4;
constexpr int kPThreads = kPWaves * 64;
constexpr int kRowBytes = kPK * 2;       // 128 bytes per tile row
constexpr int kWBytes = kPN * kRowBytes;  // 16 KB
constexpr int kXBytes = kPM * kRowBytes;  // 24 KB
constexpr int kTBW = kPM / 64;           // 32-token blocks per wave (two waves per token half)
constexpr int kStage = kWBytes + kXBytes;
constexpr int kNStage = 2;               // the next k-step is in flight
constexpr int kWLoads = kWBytes / 1024 / kPWaves, kXLoads = kXBytes / 1024 / kPWaves;  // per thread

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
    int32_t* slot_frame;
    int32_t frames;
    int32_t feat_tiles, tok_tiles;
};

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Workgroups are dispatched round-robin over the 8 XCDs; each XCD gets a contiguous range of
// a tile list ordered in blocks of 8 token tiles x 8 feature tiles, so the 64 workgroups an
// XCD runs at once (two per CU) share 8 x tiles and 8 W tiles, which stay in its L2 (x and W
// of a chunk are 14 MB each, more than one XCD's L2).
__device__ inline int xcd_item(int bid, int total) {
    constexpr int kXcd = 8;
    const int q = total / kXcd, r = total % kXcd, xcd = bid % kXcd, idx = bid / kXcd;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__device__ inline void block_tile(int item, int tok_tiles, int feat_tiles, int& tt, int& ft) {
    constexpr int BT = 8, BF = 8;
    const int nbt = (tok_tiles + BT - 1) / BT, nbf = (feat_tiles + BF - 1) / BF;
    for (int bf = 0; bf < nbf; ++bf)
        for (int bt = 0; bt < nbt; ++bt) {
            const int st = min(BT, tok_tiles - bt * BT), sf = min(BF, feat_tiles - bf * BF);
            if (item < st * sf) {
                tt = bt * BT + item % st;
                ft = bf * BF + item / st;
                return;
            }
            item -= st * sf;
        }
    tt = ft = 0;  // not reached: item < tok_tiles * feat_tiles
}

__global__ __launch_bounds__(kPThreads, 2) void qkv_rope_append_kernel(ProjArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kNStage * kStage];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 31, g = lane >> 5;
    if (blockIdx.x == 0)  // the device slot table, as the append kernel keeps it
        for (int f = tid; f < a.frames; f += kPThreads) a.slot_frame[(a.t0 + f) % a.capacity] = a.t0 + f;
    int tt, ft;
    block_tile(xcd_item(blockIdx.x, a.feat_tiles * a.tok_tiles), a.tok_tiles, a.feat_tiles, tt, ft);
    const int n0 = __builtin_amdgcn_readfirstlane(ft * kPN), m0 = __builtin_amdgcn_readfirstlane(tt * kPM);

    // DMA: a tile is blocks of 1 KB (8 rows of 128 B); wave w fills blocks 8 i + w.  Lane l
    // writes row l / 8, position l % 8 of a block, i.e. data chunk (l % 8) ^ swz(row), where
    // swz(row) = (row >> 1) & 7 = ((block & 1) << 2) | (rib >> 1) and block & 1 = w & 1.
    const int rib = lane >> 3;
    const int dchunk = (lane & 7) ^ (((wave & 1) << 2) | (rib >> 1));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)(((int64_t)(a.feat_tiles * kPN - 1) * a.w_st + a.hidden) * 2));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(((int64_t)(a.n_tokens - 1) * a.x_st + a.hidden) * 2));
    uint32_t w_off[kWLoads], x_off[kXLoads];
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) w_off[i] = (uint32_t)((int64_t)(n0 + (kPWaves * i + wave) * 8 + rib) * a.w_st * 2) + dchunk * 16;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int tok = min(m0 + (kPWaves * i + wave) * 8 + rib, a.n_tokens - 1);  // rows past the end repeat the last
        x_off[i] = (uint32_t)((int64_t)tok * a.x_st * 2) + dchunk * 16;
    }
    auto load_stage = [&](int kk, char* st) {
        const uint32_t koff = (uint32_t)kk * kPK * 2;
#pragma unroll
        for (int i = 0; i < kWLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(st + (kPWaves * i + wave) * 1024), 16, w_off[i],
                                                     koff, 0, 0);
#pragma unroll
        for (int i = 0; i < kXLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(st + kWBytes + (kPWaves * i + wave) * 1024), 16,
                                                     x_off[i], koff, 0, 0);
    };

    // fragments: row r of a tile, chunk c (8 channels) at r * 128 + ((c ^ swz(r)) * 16)
    const int sw = (li >> 1) & 7;
    const int wf_row = 64 * (wave & 1) + li;   // W rows of this wave (+ 32 fb)
    const int xt_row = (kPM / 2) * (wave >> 1) + li;  // x rows of this wave (+ 32 tb); wave >> 1 in 0..1
    f32x16 acc[2][kTBW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kTBW; ++j) acc[i][j] = f32x16{};

    // The wave's place in the tile and in the Q, K, V layout, and the epilogue's bias.
    const int hd = a.heads * a.head_dim;
    const int part = n0 / hd;  // 0: Q, 1: K, 2: V (a tile never straddles two)
    const int fcol0 = 64 * (wave & 1);        // the wave's first feature inside the tile
    const int mrow0 = m0 + (kPM / 2) * (wave >> 1);  // the wave's first token
    const int c_w = n0 + fcol0 - part * hd;   // first channel of the wave inside its part
    const int h = c_w / a.head_dim, d_w = c_w - h * a.head_dim;
    const bool rot = part < 2 && a.has_rope;
    float bias_r[2][4][4];  // [channel block][group of 4][channel]: the lane's 32 channels
    // Loaded at the start of the last k-step, which issues no DMA: the registers are free
    // through the loop and the loads land during that k-step's MFMAs.  The (cos, sin) tables
    // are read per token block in the epilogue.
    auto load_epilogue_inputs = [&]() {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bias_r[f][q4][e] = a.bias ? a.bias[n0 + fcol0 + 32 * f + 8 * q4 + 4 * g + e] : 0.f;
    };

    const int nk = a.hidden / kPK;
    load_stage(0, smem);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int st = 0;
    for (int kk = 0; kk < nk; ++kk) {
        char* cur = smem + st * kStage;
        if (kk == nk - 1) load_epilogue_inputs();
        // the other stage was consumed before the last barrier
        if (kk + 1 < nk) load_stage(kk + 1, smem + (st ^ 1) * kStage);
        // fragments of 16-channel step j + 1 are read while the MFMAs of step j run
        bf16x8 af[2][2], bf[2][kTBW];
        auto read_frags = [&](int j, int b) {
            const int coff = (((2 * j + g) ^ sw) * 16);
#pragma unroll
            for (int f = 0; f < 2; ++f)
                af[b][f] = *reinterpret_cast<const bf16x8*>(cur + (wf_row + 32 * f) * kRowBytes + coff);
#pragma unroll
            for (int tb = 0; tb < kTBW; ++tb)
                bf[b][tb] = *reinterpret_cast<const bf16x8*>(cur + kWBytes + (xt_row + 32 * tb) * kRowBytes + coff);
        };
        read_frags(0, 0);
#pragma unroll
        for (int j = 0; j < kPK / 16; ++j) {
            if (j + 1 < kPK / 16) read_frags(j + 1, (j + 1) & 1);
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int t = 0; t < kTBW; ++t) acc[f][t] = mfma32(af[j & 1][f], bf[j & 1][t], acc[f][t]);
            // issue order: one fragment read of step j + 1, one MFMA of step j, then the last MFMA
            if (j + 1 < kPK / 16) {
#pragma unroll
                for (int i = 0; i < 2 + kTBW; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * kTBW - 2 - kTBW, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the next stage must have landed: each wave waits for its own DMA, then a plain
        // barrier (no fence is needed: the fragment reads of this step were consumed by its
        // MFMAs before the barrier).
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        st ^= 1;
    }

    // ---- epilogue.  The stages are free (the loop ended on a barrier).  Each wave turns its
    // 64 x 96 block into bf16 (+ bias, RoPE) in an LDS region of its own, token rows for Q and
    // K, channel rows for V, then writes whole rows to global memory (128 bytes per token for Q
    // and K, 16 bytes per 8 tokens of a V^T row).
    constexpr int kPitch = 136;                   // Q, K: token rows of 64 bf16 and 8 bytes of padding
    constexpr int kVPitch = (kPM / 2) * 2 + 8;    // V: channel rows of the wave's tokens and 8 bytes of padding
    constexpr int kRegion = (kPM / 2) * kPitch > 64 * kVPitch ? (kPM / 2) * kPitch : 64 * kVPitch;
    char* region = smem + wave * kRegion;
#pragma unroll
    for (int t = 0; t < kTBW; ++t) {
        const int ml = 32 * t + li;
        float2 cs[2][4][2];  // this token block's (cos, sin): [channel block][group of 4][pair]
        if (rot) {
            const int m = min(mrow0 + ml, a.n_tokens - 1);
            const int fr = m / a.hw, sp = m - fr * a.hw;
            const int tg = a.t0 + fr, ph = sp / a.wf, pw = sp - ph * a.wf;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        cs[f][q4][e] = rope_cs(a.rope, (d_w + 32 * f + 8 * q4 + 4 * g + 2 * e) >> 1, tg, ph, pw);
        }
#pragma unroll
        for (int f = 0; f < 2; ++f) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int cl = 32 * f + 8 * q4 + 4 * g;  // channel inside the wave's 64
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[f][t][4 * q4 + e] + bias_r[f][q4][e];
                if (rot) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) rope_apply(cs[f][q4][e], y[2 * e], y[2 * e + 1]);
                }
                if (part == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<uint16_t*>(region + (cl + e) * kVPitch + ml * 2) =
                            (uint16_t)(pack_bf16x2(y[e], 0.f) & 0xffffu);
                } else {
                    *reinterpret_cast<uint2*>(region + ml * kPitch + cl * 2) =
                        make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                }
            }
        }
    }
    __syncthreads();
    if (part < 2) {
        // token rows: 8 lanes write one token's 64 channels (128 bytes)
#pragma unroll
        for (int pass = 0; pass < kPM / 16; ++pass) {
            const int row = pass * 8 + (lane >> 3), ch = (lane & 7) * 8;
            const int m = mrow0 + row;
            if (m >= a.n_tokens) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(region + row * kPitch + ch * 2);
            uint16_t* dst;
            if (part == 0) {
                dst = a.q + (int64_t)m * a.q_st + (int64_t)h * a.q_sh + d_w + ch;
            } else {
                const int fr = m / a.hw, sp = m - fr * a.hw;
                const int64_t phys = (int64_t)((a.t0 + fr) % a.capacity) * a.frame_stride + sp;
                dst = a.kc + ((int64_t)h * a.kv_rows + phys) * a.head_dim + d_w + ch;
            }
            *reinterpret_cast<uint4*>(dst) = v;
        }
    } else {
        // channel rows: each 16 bytes hold 8 consecutive tokens of one channel
        constexpr int kChunks = kPM / 16;  // 16-byte chunks per channel row
#pragma unroll
        for (int pass = 0; pass < kChunks; ++pass) {
            const int c = pass * 64 + lane;
            const int row = c / kChunks, ch = (c % kChunks) * 8;
            const int m = mrow0 + ch;
            if (m >= a.n_tokens) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(region + row * kVPitch + ch * 2);
            const int fr = m / a.hw, sp = m - fr * a.hw;
            uint16_t* dst = a.vt + ((int64_t)h * a.head_dim + d_w + row) * a.kv_rows;
            const int64_t phys = (int64_t)((a.t0 + fr) % a.capacity) * a.frame_stride + sp;
            if ((a.hw & 7) == 0 && m + 8 <= a.n_tokens) {  // 8 tokens of one frame, 16-byte aligned
                *reinterpret_cast<uint4*>(dst + phys) = v;
            } else {
                const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&v);
                for (int e = 0; e < 8 && m + e < a.n_tokens; ++e) {
                    const int me = m + e, fe = me / a.hw, se = me - fe * a.hw;
                    dst[(int64_t)((a.t0 + fe) % a.capacity) * a.frame_stride + se] = e16[e];
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
    a.slot_frame = L.slot_frame;
    a.frames = L.frames;
    a.feat_tiles = 3 * L.heads * L.head_dim / kPN;
    a.tok_tiles = (L.n_tokens + kPM - 1) / kPM;
    qkv_rope_append_kernel<<<a.feat_tiles * a.tok_tiles, kPThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace vdit
