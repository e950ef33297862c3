// Bandwidth-bound kernels of libvdit: token positions, RoPE3D in place, the ring KV-cache
// append (keys rotated at their global positions, values transposed) and the device
// block-plan builder.
#include <type_traits>

#include "vdit_bf16.hpp"
#include "vdit_internal.hpp"

namespace vdit {

namespace {

constexpr int kThreads = 256;

// ---- positions: global time index = start frame + local frame ("Accelerating Video
// Generation Inference ... Using a Global Time Index", section 2.B).
__global__ void positions_kernel(int32_t n, int32_t hw, int32_t width, int32_t t0, int32_t* out) {
    int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    int32_t s = i % hw;
    out[3 * i + 0] = t0 + i / hw;
    out[3 * i + 1] = s / width;
    out[3 * i + 2] = s % width;
}

__global__ void fill_i32_kernel(int32_t* p, int32_t value, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

// Loads 8 channels starting at `ch` of one token/head into fp32.
template <bool F32>
__device__ inline void load8(const void* base, int64_t off, float x[8]) {
    if constexpr (F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
        float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
        unpack_bf16x8(u, x);
    }
}

template <bool F32>
__device__ inline void store8(void* base, int64_t off, const float x[8]) {
    if constexpr (F32) {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
        p[0] = make_float4(x[0], x[1], x[2], x[3]);
        p[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else {
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + off) = pack_bf16x8(x);
    }
}

// ---- RoPE3D in place: one thread per (token, head, 8-channel chunk) of tokens
// [tok0, tok0 + n) of x0, and of x1 in the grid's second row when the call rotates two
// tensors (Q and K in one launch).  The host keeps n * heads * chunks below 2^31, so the index
// arithmetic is 32-bit.
template <bool F32>
__global__ void rope_inplace_kernel(RopeDev r, int32_t tok0, int32_t n, int32_t hw, int32_t width, int32_t t0,
                                    int32_t heads, int32_t head_dim, void* x0, int64_t st0, int64_t sh0, void* x1,
                                    int64_t st1, int64_t sh1) {
    const int32_t chunks = head_dim / 8, per_tok = heads * chunks;
    const int32_t i = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= n * per_tok) return;
    const int32_t lt = i / per_tok, rem = i - lt * per_tok;
    const int32_t h = rem / chunks, c = rem - h * chunks;
    const int32_t tok = tok0 + lt, s = tok % hw;
    const int32_t pos_t = t0 + tok / hw, pos_h = s / width, pos_w = s % width;
    const bool second = blockIdx.y != 0;
    void* x = second ? x1 : x0;
    const int64_t off = (int64_t)tok * (second ? st1 : st0) + (int64_t)h * (second ? sh1 : sh0) + c * 8;
    float v[8];
    load8<F32>(x, off, v);
    rope_rotate8(r, c * 4, pos_t, pos_h, pos_w, v);
    store8<F32>(x, off, v);
}

// ---- device plan builder: one workgroup.
// 1. Every tile's geometry (LDS) and its qtile words; the slot table into LDS, with the
//    frames of an append of the same launch placed in their slots.
// 2. One thread per (tile, slot) pair: the slot's within-frame key range for the tile,
//    packed into LDS (the divisions of the visibility rule run in parallel here).
// 3. Rounds of THREADS tiles, a thread per tile: it merges its slots' ranges into runs and
//    counts them, a block scan turns the counts into row pointers, then it writes its spans.
// Plans too large for the LDS tables take the same rounds with the ranges computed inline.
// All integer, with the host builder's merge (plan_runs), so the words equal the host's.
constexpr int kPlanMaxSlots = 1024;
constexpr uint32_t kPlanNoRange = 0xFFFFFFFFu;

template <int THREADS, int MAX_TILES, int PAIR_WORDS>
struct PlanLds {
    static constexpr int kThreads = THREADS, kMaxTiles = MAX_TILES, kPairWords = PAIR_WORDS;
    int32_t slot[kPlanMaxSlots];
    uint32_t range[PAIR_WORDS];  // (a | b << 16) of pair tile * capacity + slot
    int32_t tq[MAX_TILES], piece[MAX_TILES];
    int32_t wave_sum[THREADS / 64];
    long long pairs[THREADS / 64];
};

// The standalone kernel: 1024 threads, tables for 2048 tiles and 16384 pairs (84 KB).
using PlanLdsBig = PlanLds<1024, 2048, 16384>;
// The plan workgroup of the append kernel: 256 threads, tables for 512 tiles and 6144
// pairs (32 KB, shared with the append's transpose buffer).
using PlanLdsAppend = PlanLds<256, 512, 6144>;

// Frames [upd_t0, upd_t0 + upd_frames) are placed in slot t mod capacity before the plan
// is built (upd_frames = 0: the slot table as it is); needs capacity <= kPlanMaxSlots.  With
// an update, this workgroup is also the only writer of the device table: each thread writes
// back the slots it changed after reading them.
template <class L>
__device__ void plan_build_block(const PlanGeom& g, int32_t* slot_frame, int32_t upd_t0, int32_t upd_frames,
                                 int32_t nq, int32_t* plan, L& lds) {
    constexpr int T = L::kThreads, W = T / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t cap = g.capacity;
    const bool slots_in_lds = cap <= kPlanMaxSlots;
    const bool tables = slots_in_lds && nq <= L::kMaxTiles && (int64_t)nq * cap <= L::kPairWords && g.hw <= 0xFFFF;
    int32_t* qtiles = plan + VDIT_PLAN_HEADER_WORDS;
    int32_t* row_ptr = qtiles + 2 * nq;
    int32_t* spans = row_ptr + nq + 1;

    for (int32_t i = tid; i < nq; i += T) {
        const QTile qt = plan_qtile(g, i);
        qtiles[2 * i] = qt.q_start;
        qtiles[2 * i + 1] = qt.q_len;
        if (tables) {
            lds.tq[i] = qt.t_q;
            lds.piece[i] = qt.piece;
        }
    }
    if (slots_in_lds) {
        for (int32_t j = tid; j < cap; j += T) {
            // slot j after the append: the newest appended frame t with t mod cap = j, if any
            int32_t t = slot_frame[j];
            if (upd_frames > 0) {
                const int32_t last = upd_t0 + upd_frames - 1;
                const int32_t cand = last - ((last - j) % cap + cap) % cap;
                if (cand >= upd_t0) {
                    t = cand;
                    slot_frame[j] = t;
                }
            }
            lds.slot[j] = t;
        }
    }
    __syncthreads();
    const int32_t* sf = slots_in_lds ? lds.slot : slot_frame;
    if (tables) {
        for (int32_t p = tid; p < nq * cap; p += T) {
            const int32_t i = p / cap, j = p - i * cap;
            const QTile qt{0, 0, lds.tq[i], 0, lds.piece[i]};
            int32_t a, b;
            lds.range[p] = plan_slot_range(g, qt, sf[j], &a, &b) ? (uint32_t)a | ((uint32_t)b << 16) : kPlanNoRange;
        }
        __syncthreads();
    }

    // the spans of tile i, from the LDS table or computed inline
    auto tile_runs = [&](int32_t i, const QTile& qt, auto&& emit) {
        if (tables) {
            const uint32_t* rr = lds.range + i * cap;
            plan_runs(
                cap, g.frame_stride,
                [&](int32_t slot, int32_t* a, int32_t* b) {
                    const uint32_t r = rr[slot];
                    *a = (int32_t)(r & 0xFFFFu);
                    *b = (int32_t)(r >> 16);
                    return r != kPlanNoRange;
                },
                emit);
        } else {
            plan_tile_spans(g, sf, qt, emit);
        }
    };

    int32_t carry = 0;
    long long pairs = 0;
    for (int32_t base = 0; base < nq; base += T) {
        const int32_t i = base + tid;
        int32_t cnt = 0;
        QTile qt{0, 0, 0, 0, 0};
        if (i < nq) {
            qt = plan_qtile(g, i);
            long long keys = 0;
            tile_runs(i, qt, [&](int32_t, int32_t len) {
                ++cnt;
                keys += len;
            });
            pairs += keys * qt.q_len;
        }
        // block-wide inclusive scan of the counts: within the wave, then over the waves
        int32_t incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        if (lane == 63) lds.wave_sum[wave] = incl;
        __syncthreads();
        int32_t before = 0, total = 0;
        for (int w = 0; w < W; ++w) {
            const int32_t v = lds.wave_sum[w];
            before += w < wave ? v : 0;
            total += v;
        }
        __syncthreads();  // wave_sum is rewritten by the next round
        incl += before;
        if (i < nq) {
            row_ptr[i + 1] = carry + incl;
            int32_t kk = carry + incl - cnt;
            tile_runs(i, qt, [&](int32_t st, int32_t len) {
                spans[2 * kk] = st;
                spans[2 * kk + 1] = len;
                ++kk;
            });
        }
        carry += total;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pairs += __shfl_xor(pairs, off);
    if (lane == 0) lds.pairs[wave] = pairs;
    __syncthreads();
    if (tid == 0) {
        long long tot_pairs = 0;
        for (int w = 0; w < W; ++w) tot_pairs += lds.pairs[w];
        const unsigned long long tot = (unsigned long long)tot_pairs;
        row_ptr[0] = 0;
        plan[0] = (int32_t)VDIT_PLAN_MAGIC;
        plan[1] = VDIT_PLAN_VERSION;
        plan[2] = g.kind;
        plan[3] = g.tile;
        plan[4] = nq;
        plan[5] = carry;
        plan[6] = (int32_t)(uint32_t)(tot & 0xFFFFFFFFull);
        plan[7] = (int32_t)(uint32_t)(tot >> 32);
        plan_set_call(plan, g);
    }
}

__global__ __launch_bounds__(PlanLdsBig::kThreads) void plan_build_kernel(PlanGeom g, const int32_t* slot_frame,
                                                                          int32_t nq, int32_t* plan) {
    __shared__ PlanLdsBig lds;
    // no update: the table is only read
    plan_build_block(g, const_cast<int32_t*>(slot_frame), 0, 0, nq, plan, lds);
}

// The plan built by the append kernel's extra workgroup: the call's own chunk as the query.
struct AppendPlan {
    PlanGeom g;
    int32_t nq;
    int32_t* plan;
};

// ---- KV append.  Block = 64 tokens x one head.  Every thread issues all its global loads
// (K and V, then the RoPE (cos, sin) of its pairs) before its first store (the compiler
// cannot move a load above a possibly aliasing store).  Keys: rotated (optional) and written
// to k[h][phys][:].  Values: staged in LDS by token rows and written transposed to
// v[h][d][phys], 16 bytes (8 consecutive keys of one channel row) per lane where the 8 keys
// are consecutive in the ring (one frame, frames a multiple of 8 tokens), else key by key.
// With PLAN, workgroup x = 0 of head 0 builds the plan of the same chunk (AppendPlan) from the
// slot table with this append's frames placed, and writes those slots of the device table,
// while the other workgroups append (token block x - 1); the plan then costs no launch of its
// own and runs under the append.
constexpr int kAppendTok = 64;

template <int D>
struct AppendLds {
    static constexpr int PITCH = D + 2;  // bf16 elements per LDS row, odd dword count per row
    uint16_t sv[kAppendTok * PITCH];
};
template <int D>
union AppendPlanLds {
    AppendLds<D> app;
    PlanLdsAppend plan;
};

template <int D, bool F32, bool PLAN>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(RopeDev r, bool has_rope, int32_t n, int32_t hw,
                                                             int32_t width, int32_t t0, int32_t capacity,
                                                             int32_t frame_stride, int64_t kv_rows,
                                                             const void* k, int64_t k_st, int64_t k_sh,
                                                             const void* v, int64_t v_st, int64_t v_sh,
                                                             uint16_t* kc, uint16_t* vt, int32_t* slot_frame,
                                                             int32_t frames, AppendPlan ap) {
    constexpr int CH = D / 8;
    constexpr int PER = kAppendTok * CH / kThreads;  // chunks per thread
    constexpr int PITCH = AppendLds<D>::PITCH;
    constexpr int VT_ITEMS = D * (kAppendTok / 8) / kThreads;  // (channel, 8-key group) items per thread
    __shared__ std::conditional_t<PLAN, AppendPlanLds<D>, AppendLds<D>> lds;
    // Workgroups are dispatched round-robin over the 8 XCDs; each XCD takes a contiguous range
    // of (head, token block) pairs instead, so neighbouring token blocks of a head, which share
    // the 128-byte lines at the ends of their V^T row pieces (a frame's keys start at
    // slot * frame_stride, not on a line), write them into one L2.
    int32_t h, bx;
    {
        constexpr int kXcd = 8;
        const int total = (int)(gridDim.x * gridDim.y), lin = (int)(blockIdx.y * gridDim.x + blockIdx.x);
        const int q = total / kXcd, r = total % kXcd, xcd = lin % kXcd, idx = lin / kXcd;
        const int item = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
        h = item / (int)gridDim.x;
        bx = item % (int)gridDim.x;
    }
    if constexpr (PLAN) {
        if (bx == 0) {
            if (h == 0) plan_build_block(ap.g, slot_frame, t0, frames, ap.nq, ap.plan, lds.plan);
            return;
        }
        --bx;
    }
    uint16_t* sv;
    if constexpr (PLAN)
        sv = lds.app.sv;
    else
        sv = lds.sv;
    const int32_t n0 = bx * kAppendTok;
    const int tid = threadIdx.x;

    if (!PLAN && bx == 0 && h == 0)  // with PLAN the plan workgroup updates the table
        for (int32_t f = tid; f < frames; f += kThreads) slot_frame[(t0 + f) % capacity] = t0 + f;

    float xk[PER][8], xv[PER][8];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = tid + i * kThreads;
        const int32_t tok = n0 + c / CH, ch = c % CH;
        if (tok < n) {
            load8<F32>(k, (int64_t)tok * k_st + (int64_t)h * k_sh + ch * 8, xk[i]);
            load8<F32>(v, (int64_t)tok * v_st + (int64_t)h * v_sh + ch * 8, xv[i]);
        }
    }
    float2 cs[PER][4];
    if (has_rope) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * kThreads;
            const int32_t tok = min(n0 + c / CH, n - 1), ch = c % CH;
            const int32_t f = tok / hw, s = tok % hw;
#pragma unroll
            for (int e = 0; e < 4; ++e) cs[i][e] = rope_cs(r, ch * 4 + e, t0 + f, s / width, s % width);
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = tid + i * kThreads;
        const int32_t lt = c / CH, ch = c % CH, tok = n0 + lt;
        if (tok >= n) continue;
        const int32_t f = tok / hw, s = tok % hw;
        const int64_t phys = (int64_t)((t0 + f) % capacity) * frame_stride + s;
        if (has_rope) {
#pragma unroll
            for (int e = 0; e < 4; ++e) rope_apply(cs[i][e], xk[i][2 * e], xk[i][2 * e + 1]);
        }
        *reinterpret_cast<u32x4*>(kc + ((int64_t)h * kv_rows + phys) * D + ch * 8) = pack_bf16x8(xk[i]);
        const u32x4 pv = pack_bf16x8(xv[i]);
        uint16_t* row = sv + lt * PITCH + ch * 8;
        const uint16_t* src = reinterpret_cast<const uint16_t*>(&pv);
#pragma unroll
        for (int e = 0; e < 8; ++e) row[e] = src[e];
    }
    __syncthreads();
    // item = (channel d, keys 8 g .. 8 g + 7 of the block); eight 2-byte LDS reads down a column
    // (rows 65 dwords apart: the lanes of a read hit distinct banks)
#pragma unroll
    for (int it = 0; it < VT_ITEMS; ++it) {
        const int j = tid + it * kThreads;
        const int d = j >> 3, g8 = j & 7;
        const int32_t tok0 = n0 + 8 * g8;
        if (tok0 >= n) continue;
        uint16_t e16[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) e16[u] = sv[(8 * g8 + u) * PITCH + d];
        uint16_t* row = vt + ((int64_t)h * D + d) * kv_rows;
        const int32_t f0 = tok0 / hw, s0 = tok0 % hw;
        if ((hw & 7) == 0 && tok0 + 8 <= n) {  // 8 keys of one frame, 16-byte aligned in the ring
            const int64_t phys0 = (int64_t)((t0 + f0) % capacity) * frame_stride + s0;
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = (uint32_t)e16[2 * q] | ((uint32_t)e16[2 * q + 1] << 16);
            *reinterpret_cast<u32x4*>(row + phys0) = w;
        } else {
            for (int u = 0; u < 8 && tok0 + u < n; ++u) {
                const int32_t tu = tok0 + u, fu = tu / hw, su = tu % hw;
                row[(int64_t)((t0 + fu) % capacity) * frame_stride + su] = e16[u];
            }
        }
    }
}

// Zeroes the padding tokens [hw, frame_stride) of the written slots in k and v.
template <int D>
__global__ void kv_zero_pad_kernel(int32_t hw, int32_t frame_stride, int32_t t0, int32_t capacity, int64_t kv_rows,
                                   uint16_t* kc, uint16_t* vt) {
    const int32_t f = blockIdx.x, h = blockIdx.y;
    const int32_t pad = frame_stride - hw;
    const int64_t base = (int64_t)((t0 + f) % capacity) * frame_stride + hw;
    for (int i = threadIdx.x; i < pad * D; i += blockDim.x) {
        int32_t p = i / D, d = i % D;
        kc[((int64_t)h * kv_rows + base + p) * D + d] = 0;
        vt[((int64_t)h * D + d) * kv_rows + base + p] = 0;
    }
}

}  // namespace

hipError_t launch_positions(vdit_grid grid, int32_t t0, int32_t* out, hipStream_t s) {
    int32_t hw = grid.height * grid.width, n = grid.frames * hw;
    if (n == 0) return hipSuccess;
    positions_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, s>>>(n, hw, grid.width, t0, out);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    fill_i32_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(p, value, n);
    return hipGetLastError();
}

hipError_t launch_rope_inplace(const RopeDev& r, vdit_grid grid, int32_t t0, int32_t heads, int32_t head_dim,
                               vdit_tensor x0, const vdit_tensor* x1, hipStream_t s) {
    const int32_t hw = grid.height * grid.width, n = grid.frames * hw;
    const int64_t per_tok = (int64_t)heads * (head_dim / 8);
    // token ranges of fewer than 2^31 threads per tensor
    const int32_t step = (int32_t)std::min<int64_t>(n, (((int64_t)1 << 31) - kThreads) / per_tok);
    const vdit_tensor y = x1 ? *x1 : x0;
    for (int32_t tok0 = 0; tok0 < n; tok0 += step) {
        const int32_t cnt = std::min(step, n - tok0);
        const dim3 blocks((unsigned)((cnt * per_tok + kThreads - 1) / kThreads), x1 ? 2 : 1);
        if (x0.dtype == VDIT_DTYPE_FP32)
            rope_inplace_kernel<true><<<blocks, kThreads, 0, s>>>(r, tok0, cnt, hw, grid.width, t0, heads, head_dim,
                                                                  x0.data, x0.stride_token, x0.stride_head, y.data,
                                                                  y.stride_token, y.stride_head);
        else
            rope_inplace_kernel<false><<<blocks, kThreads, 0, s>>>(r, tok0, cnt, hw, grid.width, t0, heads, head_dim,
                                                                   x0.data, x0.stride_token, x0.stride_head, y.data,
                                                                   y.stride_token, y.stride_head);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, bool F32>
static void append_d(const vdit_kv_cache& c, const RopeDev* r, vdit_grid grid, int32_t t0, vdit_tensor k,
                     vdit_tensor v, const AppendPlan* ap, hipStream_t s) {
    int32_t hw = c.tokens_per_frame, n = grid.frames * hw;
    int32_t fs = frame_stride_of(hw);
    int64_t kv_rows = (int64_t)c.capacity * fs;
    const unsigned token_blocks = (n + kAppendTok - 1) / kAppendTok;
    RopeDev rr = r ? *r : RopeDev{};
    if (ap)
        kv_append_kernel<D, F32, true><<<dim3(token_blocks + 1, c.heads), kThreads, 0, s>>>(
            rr, r != nullptr, n, hw, grid.width, t0, c.capacity, fs, kv_rows, k.data, k.stride_token,
            k.stride_head, v.data, v.stride_token, v.stride_head, static_cast<uint16_t*>(c.k),
            static_cast<uint16_t*>(c.v), c.slot_frame_dev, grid.frames, *ap);
    else
        kv_append_kernel<D, F32, false><<<dim3(token_blocks, c.heads), kThreads, 0, s>>>(
            rr, r != nullptr, n, hw, grid.width, t0, c.capacity, fs, kv_rows, k.data, k.stride_token,
            k.stride_head, v.data, v.stride_token, v.stride_head, static_cast<uint16_t*>(c.k),
            static_cast<uint16_t*>(c.v), c.slot_frame_dev, grid.frames, AppendPlan{});
    if (fs > hw)
        kv_zero_pad_kernel<D><<<dim3(grid.frames, c.heads), kThreads, 0, s>>>(
            hw, fs, t0, c.capacity, kv_rows, static_cast<uint16_t*>(c.k), static_cast<uint16_t*>(c.v));
}

static hipError_t kv_append_any(const vdit_kv_cache& c, const RopeDev* r, vdit_grid grid, int32_t t0,
                                vdit_tensor k, vdit_tensor v, const AppendPlan* ap, hipStream_t s) {
    // K and V share one kernel: both must have the same dtype
    if (k.dtype != v.dtype) return hipErrorInvalidValue;
    bool f32 = k.dtype == VDIT_DTYPE_FP32;
    if (c.head_dim == 128) {
        if (f32) append_d<128, true>(c, r, grid, t0, k, v, ap, s);
        else append_d<128, false>(c, r, grid, t0, k, v, ap, s);
    } else {
        if (f32) append_d<64, true>(c, r, grid, t0, k, v, ap, s);
        else append_d<64, false>(c, r, grid, t0, k, v, ap, s);
    }
    return hipGetLastError();
}

hipError_t launch_kv_append(const vdit_kv_cache& c, const RopeDev* r, vdit_grid grid, int32_t t0, vdit_tensor k,
                            vdit_tensor v, hipStream_t s) {
    return kv_append_any(c, r, grid, t0, k, v, nullptr, s);
}

hipError_t launch_kv_append_plan(const vdit_kv_cache& c, const RopeDev* r, vdit_grid grid, int32_t t0,
                                 vdit_tensor k, vdit_tensor v, const PlanGeom& g, int32_t n_qtiles, int32_t* plan,
                                 hipStream_t s) {
    if (c.capacity > kPlanMaxSlots) {  // the plan workgroup keeps the slot table in LDS: two launches
        hipError_t e = kv_append_any(c, r, grid, t0, k, v, nullptr, s);
        if (e != hipSuccess) return e;
        plan_build_kernel<<<1, PlanLdsBig::kThreads, 0, s>>>(g, c.slot_frame_dev, n_qtiles, plan);
        return hipGetLastError();
    }
    const AppendPlan ap{g, n_qtiles, plan};
    return kv_append_any(c, r, grid, t0, k, v, &ap, s);
}

hipError_t launch_kv_zero_pad(const vdit_kv_cache& c, vdit_grid grid, int32_t t0, hipStream_t s) {
    const int32_t hw = c.tokens_per_frame, fs = frame_stride_of(hw);
    const int64_t kv_rows = (int64_t)c.capacity * fs;
    if (fs > hw) {
        if (c.head_dim == 128)
            kv_zero_pad_kernel<128><<<dim3(grid.frames, c.heads), kThreads, 0, s>>>(
                hw, fs, t0, c.capacity, kv_rows, static_cast<uint16_t*>(c.k), static_cast<uint16_t*>(c.v));
        else
            kv_zero_pad_kernel<64><<<dim3(grid.frames, c.heads), kThreads, 0, s>>>(
                hw, fs, t0, c.capacity, kv_rows, static_cast<uint16_t*>(c.k), static_cast<uint16_t*>(c.v));
    }
    return hipGetLastError();
}

hipError_t launch_plan_build(const PlanGeom& g, const int32_t* slot_frame_dev, int32_t n_qtiles, int32_t* plan,
                             hipStream_t s) {
    plan_build_kernel<<<1, PlanLdsBig::kThreads, 0, s>>>(g, slot_frame_dev, n_qtiles, plan);
    return hipGetLastError();
}

}  // namespace vdit
