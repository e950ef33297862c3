// Internal declarations shared by the host API and the HIP kernels of libvdit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vdit.h"

namespace vdit {

// ------------------------------------------------------------------------------------
// Block-plan geometry.  The same code enumerates query tiles and key spans on the host
// (vdit_plan_mask with VDIT_WHERE_HOST) and in the device builder kernel, so both emit
// identical words.
//
// Visibility rules: Wave Forcing / WaveRT page (block-causal attention: a block sees
// itself and the blocks before it, blocks of 3 latent frames starting at multiples of 3)
// and "DynamicRad: Content-Adaptive Sparse Attention for Long Video Diffusion", section 2
// (window shrinking exponentially with temporal distance, long-range factor for periodic
// frames, static-ratio mode).
// ------------------------------------------------------------------------------------
struct PlanGeom {
    int32_t kind, chunk_frames, tile, w0, decay_log2, period;
    int32_t frames, hw, t0;          // query call: frames of hw tokens from global frame t0
    int32_t capacity, frame_stride;  // cache
};

// Header words 8..11 of a plan: the query call it was built for (global start frame, frames,
// tokens per frame) and a reserved zero.  Attention on another call rejects the plan.
__host__ __device__ inline void plan_set_call(int32_t* plan, const PlanGeom& g) {
    plan[8] = g.t0;
    plan[9] = g.frames;
    plan[10] = g.hw;
    plan[11] = 0;
}

__host__ __device__ inline int32_t frame_stride_of(int32_t tokens_per_frame) {
    return (tokens_per_frame + 7) / 8 * 8;
}

// Window of the log-radial rule in tiles: ceil(w0 / 2^(decay_log2 * d)).
__host__ __device__ inline int32_t radial_window(int32_t d, int32_t w0, int32_t decay_log2) {
    int64_t sh = (int64_t)d * decay_log2;
    if (sh >= 40) return w0 > 0 ? 1 : 0;
    int64_t den = (int64_t)1 << sh;
    return (int32_t)(((int64_t)w0 + den - 1) >> sh);
}

// The log-radial rules (full clip and streaming): query tiles per frame, windowed key ranges.
__host__ __device__ inline bool is_radial(int32_t kind) {
    return kind == VDIT_MASK_LOG_RADIAL || kind == VDIT_MASK_LOG_RADIAL_CAUSAL;
}

// Number of mask units of the call and [first, end) call frames of unit u.
__host__ __device__ inline int32_t plan_units(const PlanGeom& g) {
    if (g.frames <= 0) return 0;
    if (g.kind == VDIT_MASK_DENSE) return 1;
    if (is_radial(g.kind)) return g.frames;
    int32_t c0 = g.t0 / g.chunk_frames, c1 = (g.t0 + g.frames - 1) / g.chunk_frames;
    return c1 - c0 + 1;
}

__host__ __device__ inline void plan_unit_frames(const PlanGeom& g, int32_t u, int32_t* f_begin, int32_t* f_end) {
    if (g.kind == VDIT_MASK_DENSE) {
        *f_begin = 0;
        *f_end = g.frames;
    } else if (is_radial(g.kind)) {
        *f_begin = u;
        *f_end = u + 1;
    } else {
        int32_t c = g.t0 / g.chunk_frames + u;
        int32_t b = c * g.chunk_frames - g.t0, e = (c + 1) * g.chunk_frames - g.t0;
        *f_begin = b < 0 ? 0 : b;
        *f_end = e > g.frames ? g.frames : e;
    }
}

__host__ __device__ inline int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

__host__ __device__ inline int32_t plan_qtile_count(const PlanGeom& g) {
    int32_t n = 0, nu = plan_units(g);
    for (int32_t u = 0; u < nu; ++u) {
        int32_t fb, fe;
        plan_unit_frames(g, u, &fb, &fe);
        n += ceil_div((fe - fb) * g.hw, g.tile);
    }
    return n;
}

// Query tile i: rows [q_start, q_start + q_len), the global frame of its first row and,
// for the log-radial rule, its spatial tile index inside the frame.
struct QTile {
    int32_t q_start, q_len, t_q, unit_first_frame, piece;
};

__host__ __device__ inline QTile plan_qtile(const PlanGeom& g, int32_t i) {
    QTile qt{0, 0, 0, 0, 0};
    if (is_radial(g.kind) && g.frames > 0) {  // every unit is one whole frame: same tile count
        const int32_t nt = ceil_div(g.hw, g.tile);
        const int32_t u = i / nt;
        if (i < 0 || u >= g.frames) return qt;
        const int32_t off = (i - u * nt) * g.tile;
        qt.q_start = u * g.hw + off;
        qt.q_len = (g.hw - off) < g.tile ? (g.hw - off) : g.tile;
        qt.unit_first_frame = u;
        qt.t_q = g.t0 + u + off / g.hw;
        qt.piece = i - u * nt;
        return qt;
    }
    int32_t nu = plan_units(g);
    for (int32_t u = 0; u < nu; ++u) {
        int32_t fb, fe;
        plan_unit_frames(g, u, &fb, &fe);
        int32_t len = (fe - fb) * g.hw;
        int32_t nt = ceil_div(len, g.tile);
        if (i < nt) {
            int32_t off = i * g.tile;
            qt.q_start = fb * g.hw + off;
            qt.q_len = (len - off) < g.tile ? (len - off) : g.tile;
            qt.unit_first_frame = fb;
            qt.t_q = g.t0 + fb + off / g.hw;
            qt.piece = i;
            return qt;
        }
        i -= nt;
    }
    return qt;
}

// Within-frame key range [a, b) visible from query tile qt in a slot holding frame t;
// returns false when the slot contributes nothing.
__host__ __device__ inline bool plan_slot_range(const PlanGeom& g, const QTile& qt, int32_t t, int32_t* a,
                                                int32_t* b) {
    if (t < 0) return false;
    if (g.kind == VDIT_MASK_DENSE) {
        *a = 0;
        *b = g.hw;
        return true;
    }
    if (g.kind == VDIT_MASK_CHUNK_CAUSAL || g.kind == VDIT_MASK_LOG_RADIAL_CAUSAL) {
        if (t / g.chunk_frames > qt.t_q / g.chunk_frames) return false;
        if (g.kind == VDIT_MASK_CHUNK_CAUSAL) {
            *a = 0;
            *b = g.hw;
            return true;
        }
    }
    int32_t d = t > qt.t_q ? t - qt.t_q : qt.t_q - t;
    if (d == 0 || (g.period > 0 && d % g.period == 0)) {
        *a = 0;
        *b = g.hw;
        return true;
    }
    int32_t wd = radial_window(d, g.w0, g.decay_log2);
    int32_t ntiles = ceil_div(g.hw, g.tile);
    int32_t lo = qt.piece - wd, hi = qt.piece + wd;
    if (lo < 0) lo = 0;
    if (hi > ntiles - 1) hi = ntiles - 1;
    *a = lo * g.tile;
    int32_t e = (hi + 1) * g.tile;
    *b = e < g.hw ? e : g.hw;
    return *b > *a;
}

// Merges the per-slot key ranges (range(slot, &a, &b): within-frame [a, b), false when the
// slot contributes nothing) into maximal ascending runs of physical key indices.
template <class Range, class Emit>
__host__ __device__ inline void plan_runs(int32_t capacity, int32_t frame_stride, Range&& range, Emit&& emit) {
    int32_t run_start = 0, run_end = -1;
    for (int32_t slot = 0; slot < capacity; ++slot) {
        int32_t a, b;
        if (!range(slot, &a, &b)) continue;
        int32_t s0 = slot * frame_stride + a, s1 = slot * frame_stride + b;
        if (s0 == run_end) {
            run_end = s1;
        } else {
            if (run_end >= 0) emit(run_start, run_end - run_start);
            run_start = s0;
            run_end = s1;
        }
    }
    if (run_end >= 0) emit(run_start, run_end - run_start);
}

// Emits the maximal ascending runs of visible physical key indices of query tile qt.
template <class Emit>
__host__ __device__ inline void plan_tile_spans(const PlanGeom& g, const int32_t* slot_frame, const QTile& qt,
                                                Emit&& emit) {
    plan_runs(
        g.capacity, g.frame_stride,
        [&](int32_t slot, int32_t* a, int32_t* b) { return plan_slot_range(g, qt, slot_frame[slot], a, b); },
        emit);
}

__host__ __device__ inline size_t plan_bound_words(int32_t n_qtiles, int32_t capacity) {
    return (size_t)VDIT_PLAN_HEADER_WORDS + 2 * (size_t)n_qtiles + (size_t)n_qtiles + 1 +
           2 * (size_t)n_qtiles * (size_t)capacity;
}

// ------------------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files).  Arguments are validated by the caller.
// ------------------------------------------------------------------------------------
struct RopeDev {
    const float2* tab_t;
    const float2* tab_h;
    const float2* tab_w;
    int32_t pairs_t, pairs_h, pairs_w;
};

hipError_t launch_positions(vdit_grid grid, int32_t t0, int32_t* out, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s);
// Rotates x0, and x1 (of the same dtype) in the same launch when it is not NULL.
hipError_t launch_rope_inplace(const RopeDev& r, vdit_grid grid, int32_t t0, int32_t heads, int32_t head_dim,
                               vdit_tensor x0, const vdit_tensor* x1, hipStream_t s);
hipError_t launch_kv_append(const vdit_kv_cache& c, const RopeDev* r, vdit_grid grid, int32_t t0, vdit_tensor k,
                            vdit_tensor v, hipStream_t s);
hipError_t launch_plan_build(const PlanGeom& g, const int32_t* slot_frame_dev, int32_t n_qtiles, int32_t* plan,
                             hipStream_t s);
// The append and the device plan of the same chunk in one launch (two where the capacity
// exceeds the plan workgroup's LDS slot table).
hipError_t launch_kv_append_plan(const vdit_kv_cache& c, const RopeDev* r, vdit_grid grid, int32_t t0,
                                 vdit_tensor k, vdit_tensor v, const PlanGeom& g, int32_t n_qtiles, int32_t* plan,
                                 hipStream_t s);

struct AttnLaunch {
    vdit_tensor q, o;
    float* lse;
    const void* kc;
    const void* vt;
    int64_t kv_rows;
    const int32_t* plan;
    RopeDev rope;
    bool has_rope;
    int32_t hw, wf, t0, n_tokens, heads, head_dim, n_qtiles;
    int32_t mask_kind;
    int32_t plan_kind, plan_tile;  // header words 2 and 3 the call's plan must carry
    bool unpaired;  // plan from vdit_plan_dynamic: neighbouring tiles do not share span lists
    float scale_log2;
    void* workspace;  // caller-owned, attn_workspace_bytes
};
struct DynLaunch {
    PlanGeom geom;  // static rule of the call (candidates and query tiles)
    vdit_tensor q;
    RopeDev rope;
    bool has_rope;
    int32_t width, heads, head_dim, n_qtiles;
    const int32_t* slot_frame;
    const void* kc;
    int64_t kv_rows;
    float scale, keep_frac;  // keep_frac = 1 - tau
    float* proxies;          // optional [n_qtiles][capacity * tiles per frame]
    int32_t* plan;
    void* workspace;         // caller-owned, dyn_workspace_bytes
};
hipError_t launch_plan_dynamic(const DynLaunch& a, hipStream_t s);
// Fused QKV projection + RoPE + K/V append (validated by the caller).
struct ProjLaunch {
    const void* x;
    int64_t x_st;
    int32_t n_tokens, hidden;
    const void* w;
    int64_t w_st;
    const float* bias;
    int32_t heads, head_dim;
    RopeDev rope;
    bool has_rope;
    int32_t hw, wf, t0;
    void* q;
    int64_t q_st, q_sh;
    void* kc;
    void* vt;
    int64_t kv_rows;
    int32_t frame_stride, capacity;
    int32_t* slot_frame;  // device slot table (written by the kernel)
    int32_t frames;
};
hipError_t launch_qkv_rope_append(const ProjLaunch& L, hipStream_t s);
// After K/V rows of frames t0 .. t0 + frames - 1 were written by another kernel: zeros in the pad
// tokens of those slots (when frames are padded), as the append does.
hipError_t launch_kv_zero_pad(const vdit_kv_cache& c, vdit_grid grid, int32_t t0, hipStream_t s);
hipError_t launch_rel_l1(const void* cur, const void* prev, bool f32, int32_t n_blocks, int64_t block_elems,
                         int64_t block_stride, float* out, void* workspace, hipStream_t s);

// Query tiles one attention call can hold (its unit table lives in LDS).
constexpr int32_t kAttnMaxQTiles = 4096;
// key tiles (cache slots x tiles per frame) one dynamic plan may weigh
constexpr int32_t kDynMaxKeyTiles = 4096;
hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t s);
// Neighbouring log-radial query tiles (and the tiles of dynamic plans) do not share span
// lists: those plans run one tile per workgroup; chunk-causal and dense plans pair tiles
// into units.
inline bool attn_uses_tile_kernel(int32_t mask_kind, bool unpaired) { return is_radial(mask_kind) || unpaired; }
// Grid of the unit kernel on the current device, and the workspace a call needs.
hipError_t attn_unit_grid(int* grid);
size_t attn_workspace_bytes(int grid, int32_t heads, int32_t n_qtiles, bool unit_kernel, bool split);
size_t attn_workspace_counter_offset(int grid);
// The static scratch of vdit_block_attn_fwd_static: a device array of this many bytes per GPU,
// and its address on the current device.
constexpr size_t kAttnStaticScratchBytes = size_t(72) << 20;
hipError_t attn_static_scratch(void** ptr);
// Workspace of vdit_plan_dynamic and of vdit_block_rel_l1 (bytes).
size_t dyn_workspace_bytes(const PlanGeom& g, int32_t n_qtiles, int32_t heads, int32_t head_dim);
size_t rel_l1_workspace_bytes(int32_t n_blocks, int64_t block_elems);

}  // namespace vdit
