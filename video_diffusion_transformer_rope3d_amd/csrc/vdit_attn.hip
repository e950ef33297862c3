// Block-sparse flash-attention forward for CDNA4 (gfx950), bf16 MFMA with fp32 online
// softmax.  A query tile (<= 128 rows of one head) is processed by 4 waves of 32 query
// rows each.  The key loop walks the plan's spans in tiles of 64 keys; K and V^T tiles are
// double-buffered in LDS, the next tile's global loads are in flight while the current
// tile is computed.  Keys outside the spans are never loaded.
//
// Work distribution of the unit kernel: the grid is persistent, as many workgroups as fit on
// the device at once.  Units (pairs of query tiles with equal span lists) go out in rounds
// of whole units; the units that do not fill a last round either run as one more round of
// whole units (when that costs a workgroup little more than the balanced share) or have
// their key iterations laid end to end, every workgroup taking an equal contiguous share
// (stream-K), so no CU idles while others finish a last partial wave.  A unit whose
// iterations are split over several workgroups is finished by the one that arrives last:
// the others leave their unnormalised partial O^T with its running max and sum in a
// workspace and count themselves in on a per-unit counter; the last one merges all partials
// in a fixed order (deterministic) and writes O and the LSE.  No workgroup ever waits on
// another, so the schedule needs no co-residency guarantee.
//
// Math per key tile (FlashAttention-style online softmax, exact up to rounding): the
// scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so every
// lane owns one query row and the row max / sum are in-lane except one exchange between
// the two 32-lane halves; O^T += V^T P^T keeps the output in the same lane-per-row layout,
// so the rescale by exp(m_old - m_new) is a per-lane scalar.  The key order inside an
// MFMA is chosen (bits 2 and 3 of the S row index swapped) so that the bf16 P operand is
// taken from the S accumulator registers as they are and V^T is read from LDS with one
// 16-byte read per lane.
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "vdit_bf16.hpp"
#include "vdit_internal.hpp"

namespace vdit {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileWaves = 4;  // waves per query tile (32 rows each)
constexpr int kUnitWaves = 8;  // unit kernel: one workgroup per CU, two query tiles
constexpr int kBM = 128;  // query rows per tile (= plan tile)
constexpr int kBN = 64;   // keys per iteration
constexpr int kMaxTiles = kAttnMaxQTiles;  // query tiles per call (the unit table lives in LDS)
constexpr int kTableBytes = (2 * (kMaxTiles + 1) * 4 + 255) / 256 * 256;

// Work item of the tile kernel on a dynamic plan: key steps [begin, end) of query tile `tile`,
// the first of them `skip` steps into plan span `span`; slot >= 0 for chunk `chunk` of a tile
// split into `chunks` (its partial-result slot, per head), -1 for a whole tile; chunks < 0 for
// a tile whose spans the schedule rejected.
struct TileItem {
    int32_t tile, begin, end, slot, chunk, chunks, span, skip;
};
static_assert(sizeof(TileItem) == 32, "two 16-byte loads per item");
// Balancing target of the dynamic-plan schedule: tile workgroups resident at once (two per CU
// on 256 CUs).  Split chunks of all heads stay below kSplitCap; no chunk is cut below about
// kSplitMin key steps.
constexpr int kTileSlots = 512;
constexpr int kSplitCap = 2 * kTileSlots;
constexpr int kSplitMin = 8;
__host__ __device__ constexpr int32_t tile_items_max(int32_t n_qtiles, int32_t heads) {
    return n_qtiles + kSplitCap / heads;
}

struct AttnArgs {
    const void* q;
    int64_t q_st, q_sh;
    void* o;
    int64_t o_st, o_sh;
    float* lse;
    const uint16_t* kc;
    const uint16_t* vt;
    int64_t kv_rows;
    const int32_t* plan;
    RopeDev rope;
    int32_t has_rope;
    int32_t hw, wf, t0, n_tokens, heads, n_qtiles;
    int32_t plan_kind, plan_tile;  // header words 2 and 3 of the call's plan
    float scale_log2;
    int32_t* cnt;  // per-tile arrival counters, zero between calls
    float* part;   // partial results, two slots per workgroup
    // tile kernel on a dynamic plan: the work list (NULL: one item per tile and head, plan order)
    const TileItem* items;
    const int32_t* n_items;
};

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keeps the instruction scheduler from moving anything across this point, so that the
// fragment reads of one phase are not hoisted into the previous one (register pressure).
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazy-rescale margin of the pipelined loop (log2 units): p = exp2(s - m) < 2^kLazyP.
constexpr float kLazyP = 8.0f;

// swap bits 2 and 3
__device__ inline int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;

// LDS stage = K tile [kBN keys][D] + V^T tile [D][kBN keys], both dense, in 16-byte chunks.
// Chunk c of row r is stored at chunk position c ^ swz(r), so that the 16-byte fragment
// reads of 16 consecutive lanes (16 different rows, same c) hit 16 different bank groups.
// Tiles are filled by global_load_lds_dwordx4: lane l of a wave writes the 16 bytes at
// LDS base + 16 l, so each lane loads the global chunk that belongs at its LDS position.
template <int D, int WAVES>
struct Tile {
    static constexpr int KCH = D / 8;    // 16-byte chunks per K row
    static constexpr int VCH = kBN / 8;  // 16-byte chunks per V^T row
    static constexpr int K_BYTES = kBN * D * 2;
    static constexpr int V_BYTES = D * kBN * 2;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int K_LOADS = kBN * KCH / (WAVES * 64);  // direct loads per thread
    static constexpr int V_LOADS = D * VCH / (WAVES * 64);
};

template <int CH>
__device__ inline int swz(int r) {
    return CH == 16 ? (r & 15) : ((r >> 1) & 7);
}

// Per-lane constants of the tile DMA.  Load i of wave w fills 1 KB block b = WAVES i + w of a
// tile whose rows hold CH chunks: the lane writes row b * (64 / CH) + lane / CH, chunk
// position lane % CH, i.e. data chunk (lane % CH) ^ swz(row); swz(row) depends on the lane
// and on w only, so each lane has one byte offset per tile: rib * row_pitch + chunk * 16.
template <int CH>
struct DmaLane {
    int rib;    // row inside the 1 KB block
    int chunk;  // data chunk this lane copies
};

template <int CH>
__device__ inline DmaLane<CH> dma_lane(int wave, int lane) {
    constexpr int RPB = 64 / CH;
    DmaLane<CH> d;
    d.rib = lane / CH;
    // swz(b * RPB + rib) with b = WAVES i + wave, WAVES a multiple of 4
    const int s = CH == 16 ? ((wave & 3) << 2) | d.rib : ((wave & 1) << 2) | (d.rib >> 1);
    d.chunk = (lane % CH) ^ s;
    (void)RPB;
    return d;
}

// Buffer descriptor over one head's K rows or V^T rows (raw, byte-addressed).  Loads through
// it are range-checked by the hardware against `bytes`.
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Enqueues the DMA of K rows [k0, k0 + kBN) and the V^T columns of the same keys into
// `stage`.  In a tail tile, keys at or beyond kend are replaced by in-bounds keys of the
// span (their scores are masked) and V^T chunks by the last chunk holding a valid key.
// Uniform parts of the addresses go to the scalar offset, the lane's part to voffset.
template <int D, int WAVES>
__device__ inline void load_tile_lds(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t vpitch, int k0,
                                     int kend, int wave, const DmaLane<D / 8>& kl, const DmaLane<kBN / 8>& vl,
                                     char* stage) {
    using T = Tile<D, WAVES>;
    constexpr int KRPB = 64 / T::KCH, VRPB = 64 / T::VCH;
    // every address stays inside the span: scalar offset = tile start k0 (< kend), the lane's
    // row delta is clamped to kend - 1 - k0 >= 0
    const int last = kend - 1 - k0;
#pragma unroll
    for (int i = 0; i < T::K_LOADS; ++i) {
        const int blk = i * WAVES + wave;
        const int rowd = min(blk * KRPB + kl.rib, last);
        const uint32_t voff = (uint32_t)rowd * (D * 2) + kl.chunk * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(stage + blk * 1024), 16, voff,
                                                 (uint32_t)k0 * (D * 2), 0, 0);
    }
    const int vkey = min(k0 + vl.chunk * 8, (kend - 1) & ~7);  // >= k0: k0 is a multiple of 8
    const uint32_t vcol = (uint32_t)(vkey - k0) * 2;
#pragma unroll
    for (int i = 0; i < T::V_LOADS; ++i) {
        const int blk = i * WAVES + wave;
        const uint32_t voff = (uint32_t)vl.rib * vpitch + vcol;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(stage + T::K_BYTES + blk * 1024), 16, voff,
                                                 (uint32_t)(blk * VRPB) * vpitch + (uint32_t)k0 * 2, 0, 0);
    }
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ inline void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Logical workgroup index.  Workgroups are dispatched round-robin over the 8 XCDs; the
// grid is a multiple of 8 and logical index = xcd * (G / 8) + position inside the XCD, so
// each XCD works on one contiguous part of the iteration space (mostly one or two heads),
// whose K/V then stream through that XCD's L2.
__device__ inline int xcd_logical(int bid, int grid) {
    constexpr int kXcd = 8;
    return (bid % kXcd) * (grid / kXcd) + bid / kXcd;
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline long long uniform64(long long x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(x & 0xffffffffu));
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// A plan word read by the whole workgroup.  The plan does not change while a kernel runs,
// so it is read through the constant address space: uniform addresses become scalar loads
// served by the scalar cache (eight spans per line) instead of vector loads with the full
// L2 latency on the path to the next DMA.  The broadcast keeps the value in a scalar
// register whatever load the compiler picks (no waterfall loops on buffer offsets).
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
// The plan was built for this query call: its start frame, frames and tokens per frame.
__device__ inline bool plan_for_call(const int32_t* plan, const AttnArgs& a) {
    return plan[8] == a.t0 && plan[10] == a.hw && (int64_t)plan[9] * plan[10] == a.n_tokens;
}

__device__ inline int plan_word(const int32_t* p) {
    return __builtin_amdgcn_readfirstlane(*(const const_i32_t*)p);
}

// Q rows of one wave (this lane's row), RoPE applied at the global position while loading.
// All row loads are issued first, then the table loads of half the chunks at a time (a
// bound on live registers), so the segment start waits for a few round trips instead of
// one per chunk.
// qscale multiplies the rotated row before its one bf16 rounding (the unit kernel folds the
// softmax scale and log2(e) into Q, so its scores come out in log2 units).
template <int D, bool QF32>
__device__ __forceinline__ void load_q_rows(const AttnArgs& a, int h, int row, int g, bf16x8 (&qreg)[D / 16],
                                            float qscale = 1.0f) {
    constexpr int KS = D / 16, HALF = KS / 2;
    using Raw = std::conditional_t<QF32, float4, u32x4>;
    constexpr int PER = QF32 ? 2 : 1;  // 16-byte loads per chunk of 8 channels
    const int f = row / a.hw, s = row % a.hw;
    const int pt = a.t0 + f, ph = s / a.wf, pw = s % a.wf;
    const int64_t qoff = (int64_t)row * a.q_st + (int64_t)h * a.q_sh;
    Raw raw[KS][PER];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + g * 8;
        if constexpr (QF32) {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qoff + d0);
            raw[ks][0] = p[0];
            raw[ks][1] = p[1];
        } else {
            raw[ks][0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qoff + d0);
        }
    }
    auto unpack = [&](int ks, float (&x)[8]) {
        if constexpr (QF32) {
            const float4 u = raw[ks][0], v = raw[ks][1];
            x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
            x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
        } else {
            unpack_bf16x8(raw[ks][0], x);
        }
    };
    // The table choice of a pair depends only on the lane; left visible, it is hoisted out of
    // the segment loop and its pointers stay live through the key loop (spills).
    int g4 = g * 4;
    asm volatile("" : "+v"(g4));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        float2 cs[HALF][4];
        if (a.has_rope) {
#pragma unroll
            for (int i = 0; i < HALF; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) cs[i][e] = rope_cs(a.rope, (hf * HALF + i) * 8 + g4 + e, pt, ph, pw);
        }
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const int ks = hf * HALF + i;
            float x[8];
            unpack(ks, x);
            if (a.has_rope) {
#pragma unroll
                for (int e = 0; e < 4; ++e) rope_apply(cs[i][e], x[2 * e], x[2 * e + 1]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= qscale;
            qreg[ks] = __builtin_bit_cast(bf16x8, pack_bf16x8(x));
        }
    }
}

// The same rows in two phases, for a kernel that starts one query tile per workgroup: issue()
// sends the row loads and every table load at once, finish() rotates, scales and packs.  The
// tile DMA is issued in between, so the rotation runs while the K/V tiles are in flight and
// the loads of the rows never wait behind it.
template <int D, bool QF32>
struct QRows {
    static constexpr int KS = D / 16, PER = QF32 ? 2 : 1;
    using Raw = std::conditional_t<QF32, float4, u32x4>;
    Raw raw[KS][PER];
    float2 cs[KS][4];

    __device__ __forceinline__ void issue(const AttnArgs& a, int h, int row, int g) {
        const int f = row / a.hw, s = row % a.hw;
        const int pt = a.t0 + f, ph = s / a.wf, pw = s % a.wf;
        const int64_t qoff = (int64_t)row * a.q_st + (int64_t)h * a.q_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = ks * 16 + g * 8;
            if constexpr (QF32) {
                const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qoff + d0);
                raw[ks][0] = p[0];
                raw[ks][1] = p[1];
            } else {
                raw[ks][0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qoff + d0);
            }
        }
        if (a.has_rope) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) cs[ks][e] = rope_cs(a.rope, ks * 8 + g * 4 + e, pt, ph, pw);
        }
    }

    __device__ __forceinline__ void finish(const AttnArgs& a, bf16x8 (&qreg)[KS], float qscale) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
            if constexpr (QF32) {
                const float4 u = raw[ks][0], v = raw[ks][1];
                x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
                x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
            } else {
                unpack_bf16x8(raw[ks][0], x);
            }
            if (a.has_rope) {
#pragma unroll
                for (int e = 0; e < 4; ++e) rope_apply(cs[ks][e], x[2 * e], x[2 * e + 1]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= qscale;
            qreg[ks] = __builtin_bit_cast(bf16x8, pack_bf16x8(x));
        }
    }
};

// Lane-level fragment addressing of one wave inside a stage.
struct FragLane {
    int qi, g;   // query row of the lane inside the wave's 32, half-wave
    int krow;    // key of each 32-key block held by S row qi (bits 2 and 3 swapped)
    int kswz, vswz;
};

// One key tile: S^T = K Q^T, online softmax, O^T += V^T P^T for the wave's 32 query rows.
// kst / vst: the stage's K and V^T tiles; keys >= kend - k0 of the tile are masked.
// m_run is the exponent base, raised only when a tile max exceeds it by more than
// lazy_raw (raw score units), so most tiles skip the rescale of O.
template <int D, int WAVES>
__device__ __forceinline__ void tile_step(const char* kst, const FragLane& fl, const bf16x8 (&qreg)[D / 16],
                                          f32x16 (&oacc)[D / 32], float& m_run, float& l_run, float c,
                                          float lazy_raw, int k0, int kend) {
    using T = Tile<D, WAVES>;
    constexpr int KS = D / 16, DB = D / 32;
    const char* vst = kst + T::K_BYTES;
    const int qi = fl.qi, g = fl.g;
    auto read_k = [&](int ks, int kb) {
        return *reinterpret_cast<const bf16x8*>(kst + (kb * 32 + fl.krow) * (T::KCH * 16) +
                                                (((2 * ks + g) ^ fl.kswz) * 16));
    };
    auto read_v = [&](int j, int db) {
        return *reinterpret_cast<const bf16x8*>(vst + (db * 32 + qi) * (T::VCH * 16) + (((2 * j + g) ^ fl.vswz) * 16));
    };
    // S^T = K Q^T over 2 blocks of 32 keys, fragments read half a tile ahead
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    constexpr int KH = KS / 2;
    bf16x8 kf[KH][2];
#pragma unroll
    for (int ks = 0; ks < KH; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kf[ks][kb] = read_k(ks, kb);
    sched_fence();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int ks = 0; ks < KH; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = mfma32(kf[ks][kb], qreg[half * KH + ks], sacc[kb]);
                if (half == 0) kf[ks][kb] = read_k(KH + ks, kb);
            }
        sched_fence();
    }
    // first half of the V^T fragments, read while the softmax runs
    bf16x8 vf[2][DB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[j][db] = read_v(j, db);
    sched_fence();
    // online softmax
    if (k0 + kBN > kend) {  // ragged last tile of a span: hide keys >= kend
        asm volatile("");     // keeps this a branch instead of selects on every tile
        const int lim = kend - k0 - g * 8;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kb * 32 + (r >> 3) * 16 + (r & 7) >= lim) sacc[kb][r] = -INFINITY;
    }
    float mt = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
    // the row's other half (lane ^ 32) through a lane swap on the VALU: an LDS permute would
    // also wait for the V^T fragment reads issued above
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
    mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    if (__any(mt > m_run + lazy_raw)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = fast_exp2((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float mc = -m_run * c;
    bf16x8 pk[4];
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(sacc[j >> 1][(j & 1) * 8 + e], c, mc));
        const u32x4 u = pack_bf16x8(p);
        pk[j] = __builtin_bit_cast(bf16x8, u);
        // the row sum adds the bf16-rounded P (the weights P.V uses), two per dot product;
        // the words are named (a bit_cast of a vector subscript in an unrolled loop is
        // compiled as reads of the first word only)
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i]), one2, l_run, false);
    }
    sched_fence();
    // O^T += V^T P^T
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            oacc[db] = mfma32(vf[j][db], pk[j], oacc[db]);
            vf[j][db] = read_v(j + 2, db);
        }
    sched_fence();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = mfma32(vf[j][db], pk[j + 2], oacc[db]);
}

// Epilogue of one wave: O = O^T / l for the lane's row and the row's LSE.  l_lane is this
// lane's half of the row sum; m_fin the exponent base.
template <int D, bool OF32>
__device__ __forceinline__ void store_rows(const AttnArgs& a, int h, int row, bool row_valid, int g,
                                           const f32x16 (&oacc)[D / 32], float m_fin, float l_lane, float c) {
    const float l = l_lane + __shfl_xor(l_lane, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (!row_valid) return;
    const int64_t ooff = (int64_t)row * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = db * 32 + j * 8 + g * 4;
            float v0 = oacc[db][4 * j] * inv, v1 = oacc[db][4 * j + 1] * inv;
            float v2 = oacc[db][4 * j + 2] * inv, v3 = oacc[db][4 * j + 3] * inv;
            if constexpr (OF32) {
                *reinterpret_cast<float4*>(static_cast<float*>(a.o) + ooff + d) = make_float4(v0, v1, v2, v3);
            } else {
                uint2 u = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + ooff + d) = u;
            }
        }
    }
    if (a.lse && g == 0)
        a.lse[(int64_t)h * a.n_tokens + row] = l > 0.f ? (m_fin * c + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// Lazy-rescale threshold of the online softmax (log2 units): p = exp2((s - m) c) < 2^kLazy.
constexpr float kLazy = 8.0f;

// A plan that does not belong to the call (wrong magic or tile count, tiles or spans outside the
// call or the cache) is not computed: the kernel writes NaN instead, so that the failure shows
// in the outputs.  poison_rows covers rows [row0, row0 + n) of head h; poison_share covers this
// workgroup's share (part of parts) of all the call's (token, head) rows.
template <int D, bool OF32>
__device__ void poison_row(const AttnArgs& a, int tok, int h, int t) {
    const int64_t off = (int64_t)tok * a.o_st + (int64_t)h * a.o_sh;
    for (int d = t * 4; d < D; d += 64 * 4) {
        if constexpr (OF32) *reinterpret_cast<float4*>(static_cast<float*>(a.o) + off + d) = make_float4(NAN, NAN, NAN, NAN);
        else *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off + d) = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
    }
    if (a.lse && t == 0) a.lse[(int64_t)h * a.n_tokens + tok] = NAN;
}

template <int D, bool OF32>
__device__ void poison_rows(const AttnArgs& a, int h, int row0, int n) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, waves = blockDim.x >> 6;
    for (int r = wave; r < n; r += waves) poison_row<D, OF32>(a, row0 + r, h, lane);
}

template <int D, bool OF32>
__device__ void poison_share(const AttnArgs& a, int part, int parts) {
    const int64_t rows = (int64_t)a.n_tokens * a.heads;
    const int64_t b = rows * part / parts, e = rows * (part + 1) / parts;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, waves = blockDim.x >> 6;
    for (int64_t r = b + wave; r < e; r += waves) poison_row<D, OF32>(a, (int)(r / a.heads), (int)(r % a.heads), lane);
}

// Tile kernel item numbering: workgroups are dispatched round-robin over the 8 XCDs; renumber
// so that each XCD gets a contiguous range of (head, query tile) items, whose K/V then stream
// through its L2.
__device__ inline int xcd_remap(int bid, int total) {
    constexpr int kXcd = 8;
    int q = total / kXcd, r = total % kXcd;
    int xcd = bid % kXcd, idx = bid / kXcd;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// ---------------------------------------------------------------- partial results
// A workgroup that computes part of a (query tile, head)'s keys leaves a partial result: per
// wave the O^T accumulators of its 64 lanes (DB * 16 floats each, stored float4-interleaved
// over lanes) and the lanes' (max, sum), all relative to the lane's own exponent base.
// Partials are written and read with device-scope (sc1) accesses, which go to the point of
// coherence of all XCDs, so the per-XCD L2s need no write-back or invalidation; each wave waits
// for its stores to complete before the workgroup counts in.
constexpr int kSc1 = 16;  // cache-policy operand of the buffer builtins: device scope (sc1)

template <int D, int WAVES = kUnitWaves>
struct Partial {
    static constexpr int DB = D / 32;
    static constexpr int O_FLOATS = DB * 16 * 64;
    static constexpr int WAVE = O_FLOATS + 2 * 64;
    static constexpr int SLOT = WAVES * WAVE;
};

// This wave's partial at byte offset pw (the wave's base) of rpart.
template <int D>
__device__ __forceinline__ void partial_store(__amdgpu_buffer_rsrc_t rpart, uint32_t pw, int lane,
                                              const f32x16 (&oacc)[D / 32], float m, float l) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 v = {__float_as_uint(oacc[db][4 * j]), __float_as_uint(oacc[db][4 * j + 1]),
                             __float_as_uint(oacc[db][4 * j + 2]), __float_as_uint(oacc[db][4 * j + 3])};
            // the block's constant offset goes to the scalar offset, so the lane needs one
            // address register for all sixteen stores
            __builtin_amdgcn_raw_buffer_store_b128(v, rpart, pw + lane * 16, (db * 4 + j) * 1024, kSc1);
        }
    const u32x2 ml = {__float_as_uint(m), __float_as_uint(l)};
    __builtin_amdgcn_raw_buffer_store_b64(ml, rpart, pw + Partial<D>::O_FLOATS * 4 + lane * 8, 0, kSc1);
}

// Folds the wave's partial at byte offset pu into (oacc, M, L): all three start empty
// (zeros, -inf, 0) before the first fold.
template <int D>
__device__ __forceinline__ void partial_fold(__amdgpu_buffer_rsrc_t rpart, uint32_t pu, int lane,
                                             f32x16 (&oacc)[D / 32], float& M, float& L) {
    const u32x2 mlu = __builtin_amdgcn_raw_buffer_load_b64(rpart, pu + Partial<D>::O_FLOATS * 4 + lane * 8, 0, kSc1);
    const float mu = __uint_as_float(mlu[0]), lu = __uint_as_float(mlu[1]);
    const float mn = fmaxf(M, mu);
    const float a1 = M == -INFINITY ? 0.f : fast_exp2(M - mn);
    const float a2 = mu == -INFINITY ? 0.f : fast_exp2(mu - mn);
    // one 32-row block at a time (a bound on the loads in flight)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 vu = __builtin_amdgcn_raw_buffer_load_b128(rpart, pu + lane * 16, (db * 4 + j) * 1024, kSc1);
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[db][4 * j + e] = oacc[db][4 * j + e] * a1 + __uint_as_float(vu[e]) * a2;
        }
        sched_fence();
    }
    L = L * a1 + lu * a2;
    M = mn;
}

// ---------------------------------------------------------------- dynamic-plan schedule
// Query tiles of a dynamic-threshold plan carry very different numbers of keys, and with one
// workgroup per (tile, head) the longest tiles alone would set the kernel's duration.  One
// workgroup ahead of the attention kernel lists the work:
//  * n_t = key steps (kBN keys each) of tile t, W = heads * (sum of n_t), and the chunk length
//    L = max(kSplitMin, ceil(W / kTileSlots)), kTileSlots being the tile workgroups the target
//    device holds at once (two per CU on 256 CUs);
//  * a tile with n_t > L becomes c_t = ceil(n_t / L) chunks whose lengths differ by at most one
//    step.  Each chunk leaves its partial result (unnormalised O, row max, row sum) in the
//    workspace; the last chunk of a (tile, head) to arrive folds them in chunk order, so the
//    result does not depend on which chunk finishes last;
//  * the items (whole tiles and chunks) are listed longest first (buckets of one step; lengths
//    from kLenBuckets - 1 on share a bucket), so the workgroups that start last run short items.
// A split tile has c_t < n_t / L + 1 < 2 n_t / L chunks, so the split chunks of all heads number
// fewer than 2 W / L <= 2 kTileSlots = kSplitCap: the partial slots, the arrival counters and
// the item list have bounds that need no knowledge of the plan.  The counters are zeroed here,
// on the stream of the attention kernel that uses them.  A plan that does not belong to the
// call gives one item per tile (the tile kernel then rejects the plan itself).
constexpr int kSchedThreads = 1024;
constexpr int kLenBuckets = 1024;
static_assert(kLenBuckets == kSchedThreads, "one histogram bucket per thread in the scan");

// Block-wide exclusive prefix sum of one value per thread (every thread calls it); *total gets
// the sum of all values.  tmp holds kSchedThreads / 64 + 1 words.
__device__ int sched_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < kSchedThreads / 64; ++w) {
            const int t = tmp[w];
            tmp[w] = run;
            run += t;
        }
        tmp[kSchedThreads / 64] = run;
    }
    __syncthreads();
    const int r = tmp[wave] + x - v;
    *total = tmp[kSchedThreads / 64];
    __syncthreads();  // tmp may be reused by the next call
    return r;
}

// Block-wide sum of one 64-bit value per thread, returned to every thread.
__device__ int64_t sched_sum64(int64_t v, int64_t* tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) tmp[wave] = v;
    __syncthreads();
    int64_t r = 0;
    for (int w = 0; w < kSchedThreads / 64; ++w) r += tmp[w];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kSchedThreads) void tile_schedule_kernel(const int32_t* plan, int32_t nq, int32_t heads,
                                                                      int64_t kv_rows, TileItem* items,
                                                                      int32_t* n_items, int32_t* cnt) {
    constexpr int PER = (kMaxTiles + kSchedThreads - 1) / kSchedThreads;  // tiles per thread in scans
    constexpr int NW = kSchedThreads / 64;
    __shared__ int32_t s_rp[kMaxTiles + 1];     // the plan's row pointers
    __shared__ unsigned long long s_n64[kMaxTiles];
    __shared__ int32_t s_n[kMaxTiles];     // key steps of tile t; -1: its spans are rejected
    __shared__ int32_t s_f[kMaxTiles];     // a rejected span of tile t, then its first split slot
    __shared__ int32_t s_rows_ok;
    __shared__ int32_t s_cur[kLenBuckets];
    __shared__ int32_t s_span[kSplitCap];  // per split slot: the chunk's first span and its skip
    __shared__ int32_t s_skip[kSplitCap];
    __shared__ int32_t s_tmp[NW + 1];
    __shared__ int64_t s_tmp64[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool ok = plan[0] == (int32_t)VDIT_PLAN_MAGIC && plan[4] == nq && nq <= kMaxTiles;
    const int n_spans = ok ? plan[5] : 0;
    const int32_t* row_ptr = plan + VDIT_PLAN_HEADER_WORDS + 2 * nq;
    const int32_t* spans = row_ptr + nq + 1;
    // Key steps per tile, and the checks the tile kernel would make: row pointers that rise
    // inside the span list (else every tile is rejected), every span non-empty, 8-aligned and
    // inside the cache.  The spans are cut into one contiguous run per thread, read eight at a
    // time; a run's tile is found by binary search in the row pointers and followed from there.
    for (int t = tid; t <= nq; t += kSchedThreads) s_rp[t] = ok ? row_ptr[t] : 0;
    for (int t = tid; t < nq; t += kSchedThreads) {
        s_n64[t] = 0;
        s_f[t] = 0;
    }
    if (tid == 0) s_rows_ok = ok ? 1 : 0;
    __syncthreads();
    for (int t = tid; t < nq; t += kSchedThreads)
        if (s_rp[t] < 0 || s_rp[t] > s_rp[t + 1] || s_rp[t + 1] > n_spans) s_rows_ok = 0;
    __syncthreads();
    const bool rows_ok = s_rows_ok != 0;
    if (rows_ok) {
        const int lo = s_rp[0], hi = s_rp[nq];
        const int per = (hi - lo + kSchedThreads - 1) / kSchedThreads;
        const int first = lo + tid * per, end = min(first + per, hi);
        int t = 0;  // last tile with s_rp[t] <= first
        for (int step = 1 << 12; step > 0; step >>= 1)
            if (t + step <= nq && s_rp[t + step] <= first) t += step;
        unsigned long long acc = 0;
        bool bad = false;
        auto flush = [&]() {
            if (acc) atomicAdd(&s_n64[t], acc);
            if (bad) s_f[t] = 1;
            acc = 0;
            bad = false;
        };
        for (int base = first; base < end; base += 8) {
            int k0[8], kl[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (base + j < end) {
                    k0[j] = spans[2 * (base + j)];
                    kl[j] = spans[2 * (base + j) + 1];
                }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sp = base + j;
                if (sp >= end) break;
                while (s_rp[t + 1] <= sp) {  // the next tile (empty ones passed over)
                    flush();
                    ++t;
                }
                bad |= k0[j] < 0 || (k0[j] & 7) || kl[j] < 1 || (int64_t)k0[j] + kl[j] > kv_rows;
                acc += ((unsigned long long)max(kl[j], 0) + kBN - 1) / kBN;
            }
        }
        if (first < end) flush();
    }
    __syncthreads();
    for (int t = tid; t < nq; t += kSchedThreads)
        s_n[t] = !rows_ok || s_f[t] ? -1 : (int32_t)min(s_n64[t], 1ull << 24);
    __syncthreads();
    // W (64-bit: a tile has at most 2^24 steps) and the chunk length
    int64_t mine = 0;
    for (int t = tid; t < nq; t += kSchedThreads) mine += max(s_n[t], 0);
    const int64_t W = sched_sum64(mine, s_tmp64) * heads;
    int64_t L = max((int64_t)kSplitMin, (W + kTileSlots - 1) / kTileSlots);
    auto chunks = [&](int n) { return (int64_t)n > L ? (int)(((int64_t)n + L - 1) / L) : 1; };
    // first split slot of each tile: prefix over tiles of c_t (split tiles only), in tile order
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int t = tid * PER + i;
        const int c = t < nq ? chunks(s_n[t]) : 1;
        loc[i] = c > 1 ? c : 0;
        sum += loc[i];
    }
    int n_split = 0;
    int pre = sched_scan(sum, s_tmp, &n_split);
    if ((int64_t)n_split * heads > kSplitCap) {  // cannot happen (see above); then split nothing
        L = INT64_MAX / 2;
        n_split = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) loc[i] = 0;
        pre = 0;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int t = tid * PER + i;
        if (t < nq) s_f[t] = pre;
        pre += loc[i];
    }
    s_cur[tid] = 0;
    __syncthreads();
    // First span of every chunk after the first of a split tile, a wave per split tile: the
    // lanes take 64 spans at a time with their step prefix; chunk k starts at step
    // k * (n / c) + min(k, n % c).
    for (int t = wave; t < nq; t += NW) {
        const int n = s_n[t], c = chunks(n);
        if (c == 1) continue;
        const int b = row_ptr[t], e = row_ptr[t + 1];
        int base = 0;  // steps of the spans before this batch
        for (int sp0 = b; sp0 < e; sp0 += 64) {
            const int sp = sp0 + lane;
            const int st = sp < e ? (spans[2 * sp + 1] + kBN - 1) / kBN : 0;
            int incl = st;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            const int lo = base + incl - st, hi = base + incl;
            for (int k = 1; k < c; ++k) {
                const int bk = k * (n / c) + min(k, n % c);
                if (lo <= bk && bk < hi) {
                    s_span[s_f[t] + k] = sp;
                    s_skip[s_f[t] + k] = bk - lo;
                }
            }
            base += __shfl(incl, 63);
        }
    }
    // items per length bucket (longest first), their start positions, then the items
    auto bucket = [](int len) { return kLenBuckets - 1 - min(len, kLenBuckets - 1); };
    for (int t = tid; t < nq; t += kSchedThreads) {
        const int n = max(s_n[t], 0), c = chunks(n);
        for (int k = 0; k < c; ++k) atomicAdd(&s_cur[bucket(n / c + (k < n % c))], 1);
    }
    __syncthreads();
    int count = 0;
    const int start = sched_scan(s_cur[tid], s_tmp, &count);
    s_cur[tid] = start;
    __syncthreads();
    for (int t = tid; t < nq; t += kSchedThreads) {
        const int n = s_n[t];
        if (n < 0) {
            items[atomicAdd(&s_cur[bucket(0)], 1)] = TileItem{t, 0, 0, -1, 0, -1, 0, 0};
            continue;
        }
        const int c = chunks(n), b = ok ? row_ptr[t] : 0;
        int beg = 0;
        for (int k = 0; k < c; ++k) {
            const int len = n / c + (k < n % c);
            const int pos = atomicAdd(&s_cur[bucket(len)], 1);
            const int span = k == 0 ? b : s_span[s_f[t] + k], skip = k == 0 ? 0 : s_skip[s_f[t] + k];
            items[pos] = TileItem{t, beg, beg + len, c > 1 ? s_f[t] + k : -1, k, c, span, skip};
            beg += len;
        }
    }
    if (tid == 0) *n_items = count;
    for (int i = tid; i < kSplitCap; i += kSchedThreads) cnt[i] = 0;
}

// ---------------------------------------------------------------- pipelined key loop
// The key loops are software-pipelined inside each wave: while the softmax of key tile n runs
// on the VALU, the score MFMAs of tile n + 1 run on the matrix core, then the P.V MFMAs of
// tile n follow, interleaved with the row sum of tile n and the row max of tile n + 1.  A step
// therefore reads K of tile n + 1 and V^T of tile n.  The unit kernel keeps NST = 3 stages of
// both (the DMA of tile n + 2 in flight); the tile kernel, two workgroups per CU, keeps two K
// stages and two V^T stages and moves V^T one tile behind K (K of tile n + 2 and V^T of tile
// n + 1 in flight).  The K tiles of all stages come first, then the V^T tiles, so every
// fragment read takes its stage and block as an immediate offset.
template <int D, int NST = 3>
struct Pipe {
    static constexpr int KS = D / 16;  // k-steps of the score contraction
    static constexpr int DB = D / 32;  // 32-row blocks of O^T
    static constexpr int KCH = D / 8, VCH = kBN / 8;
    static constexpr int KROW = KCH * 16, VROW = VCH * 16;  // LDS bytes per K row / V^T row
    static constexpr int K_BYTES = kBN * KROW, V_BYTES = D * VROW;
    static constexpr int V_BASE = NST * K_BYTES;
    static constexpr int BYTES = NST * (K_BYTES + V_BYTES);
    static constexpr int NS = 2 * KS;   // score MFMAs per step
    static constexpr int NP = 4 * DB;   // P.V MFMAs per step
    static constexpr int NM = NS + NP;
    static constexpr int LOOK = 2;      // fragment reads issued this many MFMAs ahead
};

// Per-lane LDS byte offsets of the fragment reads in stage 0: the K fragment of k-step ks
// (key block 0; block 1 is 32 rows further) and the V^T fragment of 16-key group j (row block
// 0; block db is 32 V^T rows further).  Rows hold 16-byte chunks at position chunk ^ swz(row)
// (see Tile), which the DMA writes.
template <int D>
struct PipeLane {
    uint32_t k[D / 16];
    uint32_t v[4];
};

template <int D, int NST>
__device__ inline PipeLane<D> pipe_lane(int qi, int g) {
    using P = Pipe<D, NST>;
    PipeLane<D> pl;
    const int krow = swap23(qi);
    const int kswz = swz<P::KCH>(krow), vswz = swz<P::VCH>(qi);
#pragma unroll
    for (int ks = 0; ks < P::KS; ++ks) pl.k[ks] = (uint32_t)(krow * P::KROW + (((2 * ks + g) ^ kswz) * 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) pl.v[j] = (uint32_t)(P::V_BASE + qi * P::VROW + (((2 * j + g) ^ vswz) * 16));
    // the offsets are lane constants of the whole segment loop; kept opaque so that the
    // compiler does not rematerialise them inside the loop
#pragma unroll
    for (int ks = 0; ks < P::KS; ++ks) asm volatile("" : "+v"(pl.k[ks]));
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(pl.v[j]));
    return pl;
}

// DMA of key tile [k0, k0 + kBN) of a span ending at kend: its K rows into K stage kst, its V^T
// columns into V^T stage vst (either part skipped when its stage is negative).  In a tail tile,
// keys at or beyond kend are replaced by in-bounds keys of the span (their scores are masked)
// and V^T chunks by the last chunk holding a valid key.
template <int D, int WAVES, int NST>
__device__ inline void pipe_load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t vpitch, int k0,
                                 int kend, int wave, const DmaLane<D / 8>& kl, const DmaLane<kBN / 8>& vl, char* smem,
                                 int kst, int vst) {
    using T = Tile<D, WAVES>;
    using P = Pipe<D, NST>;
    constexpr int KRPB = 64 / T::KCH, VRPB = 64 / T::VCH;
    const int last = kend - 1 - k0;
    // The LDS destinations are recomputed from the stage base at every call (one scalar add
    // each): seen as loop constants, they are hoisted and kept live through the key loop, one
    // scalar register per stage and load, which the unit kernel then spills and reloads.
    int z = 0;
    asm volatile("" : "+s"(z));
    smem += z;
    if (kst >= 0) {
        char* kdst = smem + kst * P::K_BYTES;
#pragma unroll
        for (int i = 0; i < T::K_LOADS; ++i) {
            const int blk = i * WAVES + wave;
            const int rowd = min(blk * KRPB + kl.rib, last);
            const uint32_t voff = (uint32_t)rowd * (D * 2) + kl.chunk * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + blk * 1024), 16, voff,
                                                     (uint32_t)k0 * (D * 2), 0, 0);
        }
    }
    if (vst >= 0) {
        char* vdst = smem + P::V_BASE + vst * P::V_BYTES;
        const int vkey = min(k0 + vl.chunk * 8, (kend - 1) & ~7);
        const uint32_t vcol = (uint32_t)(vkey - k0) * 2;
#pragma unroll
        for (int i = 0; i < T::V_LOADS; ++i) {
            const int blk = i * WAVES + wave;
            const uint32_t voff = (uint32_t)vl.rib * vpitch + vcol;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + blk * 1024), 16, voff,
                                                     (uint32_t)(blk * VRPB) * vpitch + (uint32_t)k0 * 2, 0, 0);
        }
    }
}

// Masks the keys >= lim of a score tile (lim = valid keys of the tile minus 8 g): S row
// kb * 32 + (r >> 3) * 16 + (r & 7) + 8 g of the lane's accumulator element r.
__device__ inline void pipe_mask(f32x16 (&s)[2], int lim) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (kb * 32 + (r >> 3) * 16 + (r & 7) >= lim) s[kb][r] = -INFINITY;
}

// Row max of a score tile: this lane's 32 keys, then the other half of the row (lane ^ 32)
// through a VALU lane swap.
__device__ inline float pipe_row_max(const f32x16 (&s)[2]) {
    float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int t = 1; t < 16; ++t) mt = fmaxf(fmaxf(mt, s[t >> 3][2 * (t & 7)]), s[t >> 3][2 * (t & 7) + 1]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// End of a step (rare, uniform branch): the next tile is the ragged end of a span (mask its
// scores and take its max again) or its max exceeds the exponent base by more than the lazy
// margin (raise the base by mt; O, the row sum, the new scores and negm follow).  Scores are
// relative to the base and in log2 units, so p = exp2(s) stays below 2^kLazy.
template <int D>
__device__ __forceinline__ void pipe_fixup(f32x16 (&sn)[2], bool tail, int lim, float mt, float& m_run,
                                           float& l_run, f32x16 (&oacc)[D / 32], f32x16& negm) {
    if (tail) {
        pipe_mask(sn, lim);
        mt = pipe_row_max(sn);
    }
    if (__any(mt > kLazyP)) {
        const float d = fmaxf(mt, 0.f);  // the base rises by d >= 0
        const float alpha = fast_exp2(-d);
        m_run += d;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sn[kb] -= d;
        negm = f32x16{} - m_run;
    }
}

// First tile of a segment: its row max becomes the exponent base (the ragged end of a span
// masked first), the scores are taken relative to it and negm holds -base.
__device__ inline void pipe_first(f32x16 (&s)[2], bool tail, int lim, float& m_run, f32x16& negm) {
    if (tail) pipe_mask(s, lim);
    const float mt = pipe_row_max(s);
    m_run = mt;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] -= mt;
    negm = f32x16{} - mt;
}

// Score MFMAs of one tile, not interleaved (the segment's first tile): S^T = K Q^T from K stage st.
template <int D, int NST>
__device__ __forceinline__ void pipe_scores(const char* smem, const PipeLane<D>& pl, int st,
                                            const bf16x8 (&qreg)[D / 16], f32x16 (&sn)[2]) {
    using P = Pipe<D, NST>;
    sn[0] = f32x16{};
    sn[1] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < P::KS; ++ks)
            sn[kb] = mfma32(*reinterpret_cast<const bf16x8*>(smem + pl.k[ks] + st * P::K_BYTES + kb * 32 * P::KROW),
                            qreg[ks], sn[kb]);
}

// One step of the pipelined loop.  Scores are in log2 units (Q carries the softmax scale
// and log2(e)), and their accumulators start from negm (every element -m, m the exponent
// base), so the MFMAs give s - m and the exponentials take them as they are.
// In: s = S^T - m of tile n (masked), V^T of tile n in stage ST, K of tile n + 1 in stage ST1.
// Out: sn = S^T - m of tile n + 1 (unmasked), mt_next = its row max; O^T and the row sum
// include tile n.
//
// Four quarters, each a run of MFMAs with VALU work spread evenly between them:
//   1. scores of key block 0 of tile n + 1   | exponentials and bf16 packing of key group 0,
//                                               half of group 1
//   2. P.V of key groups 0, 1 of tile n      | the rest of group 1 (done before the first
//                                               group-1 MFMA), group 2
//   3. scores of key block 1 of tile n + 1   | group 3, max of the new key block 0
//   4. P.V of key groups 2, 3 of tile n      | max of the new key block 1 and of the row's
//                                               other half, row sum of the packed P
// About 20 VALU items per quarter: with the VALU work piled into the first half of the step
// (its dependency order) both waves of a SIMD saturate the VALU there while the matrix core
// waits.  Groups 0, 1 of tile n are the scores of its key block 0, which quarter 1 consumes
// while it builds block 0 of tile n + 1; so at most three 16-register score blocks are live.
// Each MFMA with its share of VALU work and its fragment read LOOK MFMAs ahead is one
// scheduling group, in this order.
template <int D, int NST, int ST, int ST1>
__device__ __forceinline__ void pipe_step(const char* smem, const PipeLane<D>& pl, const bf16x8 (&qreg)[D / 16],
                                          f32x16 (&oacc)[D / 32], const f32x16 (&s)[2], f32x16 (&sn)[2],
                                          const f32x16& negm, float& l_run, float& mt_next) {
    using P = Pipe<D, NST>;
    constexpr int KS = P::KS, DB = P::DB, NM = P::NM, L = P::LOOK;
    constexpr int Q1 = KS, Q2 = Q1 + 2 * DB, Q3 = Q2 + KS;  // quarter boundaries
    auto is_score = [](int i) { return i < Q1 || (i >= Q2 && i < Q3); };
    auto score_ks = [](int i) { return i < Q1 ? i : i - Q2; };
    auto score_kb = [](int i) { return i < Q1 ? 0 : 1; };
    auto pv_index = [](int i) { return i < Q2 ? i - Q1 : i - Q3 + 2 * DB; };  // 0 .. NP-1
    // fragment of MFMA i
    auto frag = [&](int i) -> bf16x8 {
        if (is_score(i))
            return *reinterpret_cast<const bf16x8*>(smem + pl.k[score_ks(i)] + ST1 * P::K_BYTES +
                                                    score_kb(i) * 32 * P::KROW);
        const int pi = pv_index(i), j = pi / DB, db = pi % DB;
        return *reinterpret_cast<const bf16x8*>(smem + pl.v[j] + ST * P::V_BYTES + db * 32 * P::VROW);
    };
    float x[32];
    uint32_t pw[16];
    float mt = 0.f;
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    // VALU item k of quarter q.  Softmax items are numbered 12 j + u over key groups j (u < 8:
    // exponential, else a bf16 pack); quarters 1, 2 and the first 12 items of quarter 3 take
    // them in order, then come the row max and the row sum.
    auto valu = [&](int q, int k) {
        const int gidx = q == 0 ? k : q == 1 ? 18 + k : q == 2 && k < 12 ? 36 + k : -1;
        if (gidx >= 0) {
            const int jj = gidx / 12, u = gidx % 12;
            const int base = jj * 8;
            if (u < 8) x[base + u] = fast_exp2(s[jj >> 1][(jj & 1) * 8 + u]);
            else pw[jj * 4 + u - 8] = pack_bf16x2(x[base + 2 * (u - 8)], x[base + 2 * (u - 8) + 1]);
        } else if (q == 2) {  // max of the new key block 0
            const int t = k - 12;
            if (t == 0) mt = fmaxf(sn[0][0], sn[0][1]);
            else mt = fmaxf(fmaxf(mt, sn[0][2 * t]), sn[0][2 * t + 1]);
        } else if (k < 8) {  // max of the new key block 1
            mt = fmaxf(fmaxf(mt, sn[1][2 * k]), sn[1][2 * k + 1]);
        } else if (k == 8) {  // and of the other half of the row (lane ^ 32)
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
            mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        } else {  // row sum of the bf16-rounded P (the weights P.V uses), two per dot product
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[k - 9]), one2, l_run, false);
        }
    };
    bf16x8 fr[L + 1];
#pragma unroll
    for (int i = 0; i < L; ++i) fr[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        if (i + L < NM) fr[(i + L) % (L + 1)] = frag(i + L);
        const bf16x8 a = fr[i % (L + 1)];
        if (is_score(i)) {
            const int kb = score_kb(i), ks = score_ks(i);
            sn[kb] = mfma32(a, qreg[ks], ks == 0 ? negm : sn[kb]);
        } else {
            const int pi = pv_index(i), j = pi / DB, db = pi % DB;
            const u32x4 pj = {pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]};
            oacc[db] = mfma32(a, __builtin_bit_cast(bf16x8, pj), oacc[db]);
        }
        const int q = i < Q1 ? 0 : i < Q2 ? 1 : i < Q3 ? 2 : 3;
        const int q0 = q == 0 ? 0 : q == 1 ? Q1 : q == 2 ? Q2 : Q3;
        const int n = (q == 0 ? Q1 : q == 1 ? Q2 : q == 2 ? Q3 : NM) - q0, r = i - q0;
        const int items = q < 2 ? 18 : q == 2 ? 20 : 25;
        const int k_lo = items * r / n, k_hi = items * (r + 1) / n;
#pragma unroll
        for (int k = k_lo; k < k_hi; ++k) valu(q, k);
        sched_fence();
    }
    mt_next = mt;
}

// ---------------------------------------------------------------- tile kernel
// One workgroup = one (query tile, head), 4 waves, two workgroups per CU; the grid covers all
// tiles of all heads.  Used where neighbouring query tiles have different span lists
// (log-radial, dynamic plans), so that two tiles cannot share one K/V stream.  The key loop is
// the pipelined one with two K stages and two V^T stages: step n reads K of tile n + 1 and V^T
// of tile n while K of tile n + 2 and V^T of tile n + 1 are in flight.
template <int D, bool QF32, bool OF32>
__global__ __launch_bounds__(kTileWaves * 64, 2) void attn_tile_kernel(AttnArgs a) {
    using PP = Pipe<D, 2>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    // one LDS object (see the unit kernel): the stages, then the arrival word of split items
    __shared__ __attribute__((aligned(1024))) char smem[PP::BYTES + 64];
    int& s_arrived = *reinterpret_cast<int*>(smem + PP::BYTES);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qi = lane & 31, g = lane >> 5;

    const int32_t* plan = a.plan;
    const int nq = plan[4];
    // a plan that does not belong to this call (another magic, rule, tile size, tile count or
    // query call) is not read out of bounds: NaN outputs instead
    if (plan[0] != (int32_t)VDIT_PLAN_MAGIC || plan[2] != a.plan_kind || plan[3] != a.plan_tile || nq != a.n_qtiles ||
        !plan_for_call(plan, a)) {
        poison_share<D, OF32>(a, blockIdx.x, gridDim.x);
        return;
    }
    // the work item: whole tile (begin 0, end -1: all its key steps) or chunk of a split tile
    int h, qt, it_begin = 0, it_end = -1, it_slot = -1, it_chunk = 0, it_chunks = 1, it_span = 0, it_skip = 0;
    if (a.items) {  // the list is longest first, all heads of an item together
        const int it = blockIdx.x / a.heads;
        h = blockIdx.x % a.heads;
        if (it >= uniform(*a.n_items)) return;
        const int4 w0 = reinterpret_cast<const int4*>(a.items + it)[0];
        const int4 w1 = reinterpret_cast<const int4*>(a.items + it)[1];
        qt = uniform(w0.x);
        it_begin = uniform(w0.y);
        it_end = uniform(w0.z);
        it_slot = uniform(w0.w);
        it_chunk = uniform(w1.x);
        it_chunks = uniform(w1.y);
        it_span = uniform(w1.z);
        it_skip = uniform(w1.w);
    } else {
        const int item = xcd_remap(blockIdx.x, a.n_qtiles * a.heads);
        h = item / a.n_qtiles;
        qt = item % a.n_qtiles;
    }
    if (qt < 0 || qt >= nq) {
        poison_share<D, OF32>(a, blockIdx.x, gridDim.x);
        return;
    }
    const int32_t* qtiles = plan + VDIT_PLAN_HEADER_WORDS;
    const int32_t* row_ptr = qtiles + 2 * nq;
    const int32_t* spans = row_ptr + nq + 1;
    const int q_start = plan_word(qtiles + 2 * qt), q_len = plan_word(qtiles + 2 * qt + 1);
    if (q_start < 0 || q_len < 1 || q_len > kBM || q_start + q_len > a.n_tokens) {
        poison_share<D, OF32>(a, blockIdx.x, gridDim.x);
        return;
    }
    bool bad;
    if (a.items) {
        // the schedule kernel has checked the tile's spans (the same rules as below; chunks < 0:
        // rejected) and located the item's first key step; the slot range is checked here
        bad = it_chunks < 0 || it_begin < 0 || it_begin > it_end ||
              (it_end > it_begin && (it_span < 0 || it_span >= plan[5] || it_skip < 0)) ||
              (it_slot >= 0 && (it_chunk < 0 || it_chunk >= it_chunks || it_slot < it_chunk ||
                                (int64_t)(it_slot - it_chunk + it_chunks) * a.heads > kSplitCap));
    } else {
        const int sp_begin = plan_word(row_ptr + qt), sp_end = plan_word(row_ptr + qt + 1);
        bad = sp_begin < 0 || sp_begin > sp_end || sp_end > plan[5];
        int n_tiles = 0;  // key tiles of the query tile
        for (int sp = sp_begin; !bad && sp < sp_end; ++sp) {  // spans must lie inside the cache, 8-aligned
            const int k0 = spans[2 * sp], kl = spans[2 * sp + 1];
            bad = k0 < 0 || (k0 & 7) || kl < 1 || (int64_t)k0 + kl > a.kv_rows;
            n_tiles += (kl + kBN - 1) / kBN;
        }
        it_end = n_tiles;
        it_span = sp_begin;
    }
    if (bad) {
        poison_rows<D, OF32>(a, h, q_start, q_len);
        return;
    }

    const int r_in = wave * 32 + qi;
    const bool row_valid = r_in < q_len;
    const int row = q_start + (row_valid ? r_in : q_len - 1);
    // a wave whose 32 rows all lie past the tile's end (the short last tile of a frame) keeps
    // its share of the DMA and the barriers but skips the math
    const bool wave_rows = uniform(wave) * 32 < q_len;
    const float c = a.scale_log2;
    bf16x8 qreg[KS];
    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;  // in log2 units: Q carries the softmax scale and log2(e)

    if (it_end > it_begin) {
        const int wave_u = uniform(wave);
        const DmaLane<D / 8> kdl = dma_lane<D / 8>(wave_u, lane);
        const DmaLane<kBN / 8> vdl = dma_lane<kBN / 8>(wave_u, lane);
        const uint32_t head_bytes = (uint32_t)(a.kv_rows * D * 2);
        const __amdgpu_buffer_rsrc_t rk = head_rsrc(a.kc + (int64_t)h * a.kv_rows * D, head_bytes);
        const __amdgpu_buffer_rsrc_t rv = head_rsrc(a.vt + (int64_t)h * D * a.kv_rows, head_bytes);
        const uint32_t vpitch = (uint32_t)(a.kv_rows * 2);
        const PipeLane<D> pl = pipe_lane<D, 2>(qi, g);
        // key tiles n (k0, kend), n + 1 (k1, kend1), n + 2 (k2, kend2), and the span of the
        // furthest tile located so far; the item starts it_skip steps into span it_span
        int span = it_span;
        const int span_k0 = plan_word(spans + 2 * span);
        int k0 = span_k0 + it_skip * kBN, kend = span_k0 + plan_word(spans + 2 * span + 1);
        int k1 = 0, kend1 = 0;
        auto advance = [&](int k, int ke, int& nk, int& nke) {
            nk = k + kBN;
            nke = ke;
            if (nk >= ke) {
                ++span;
                nk = plan_word(spans + 2 * span);
                nke = nk + plan_word(spans + 2 * span + 1);
            }
        };
        int left = it_end - it_begin - 1;  // tiles after tile n
        QRows<D, QF32> qr;
        if (wave_rows) qr.issue(a, h, row, g);
        pipe_load<D, kTileWaves, 2>(rk, rv, vpitch, k0, kend, wave_u, kdl, vdl, smem, 0, 0);
        if (left >= 1) {
            advance(k0, kend, k1, kend1);
            pipe_load<D, kTileWaves, 2>(rk, rv, vpitch, k1, kend1, wave_u, kdl, vdl, smem, 1, -1);
        }
        if (wave_rows) qr.finish(a, qreg, c);
        wait_tile_loads();
        __syncthreads();
        f32x16 sacc[2][2];
        f32x16 negm;
        if (wave_rows) {
            pipe_scores<D, 2>(smem, pl, 0, qreg, sacc[0]);
            pipe_first(sacc[0], k0 + kBN > kend, kend - k0 - g * 8, m_run, negm);
        }
        // step n: V^T of tile n in V stage n mod 2, K of tile n + 1 in K stage (n + 1) mod 2
        auto key_step = [&](auto stc) {  // returns false after the last key tile
            constexpr int ST = decltype(stc)::value, ST1 = ST ^ 1;
            wait_tile_loads();
            __syncthreads();  // K of tile n + 1 and V^T of tile n landed; K stage ST, V^T stage ST1 free
            int k2 = 0, kend2 = 0;
            if (left >= 2) {
                advance(k1, kend1, k2, kend2);
                pipe_load<D, kTileWaves, 2>(rk, rv, vpitch, k2, kend2, wave_u, kdl, vdl, smem, ST, -1);
            }
            if (left >= 1) pipe_load<D, kTileWaves, 2>(rk, rv, vpitch, k1, kend1, wave_u, kdl, vdl, smem, -1, ST1);
            if (wave_rows) {
                float mt;
                pipe_step<D, 2, ST, ST1>(smem, pl, qreg, oacc, sacc[ST], sacc[ST1], negm, l_run, mt);
                if (left >= 1)
                    pipe_fixup<D>(sacc[ST1], k1 + kBN > kend1, kend1 - k1 - g * 8, mt, m_run, l_run, oacc, negm);
            }
            if (left == 0) return false;
            --left;
            k0 = k1;
            kend = kend1;
            k1 = k2;
            kend1 = kend2;
            return true;
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        while (key_step(I0{}) && key_step(I1{})) {
        }
    }
    if (it_slot < 0) {
        store_rows<D, OF32>(a, h, row, row_valid, g, oacc, m_run, l_run, 1.0f);
        return;
    }
    // chunk of a split tile: leave the partial in its slot, count in; the last chunk of the
    // (tile, head) to arrive folds all of them in chunk order
    using TP = Partial<D, kTileWaves>;
    using TP128 = Partial<128, kTileWaves>;  // slots are sized for head_dim 128
    const __amdgpu_buffer_rsrc_t rpart = head_rsrc(a.part, (uint32_t)((size_t)kSplitCap * TP128::SLOT * 4));
    const int first = it_slot - it_chunk;  // slot of chunk 0
    if (wave_rows)
        partial_store<D>(rpart, (uint32_t)(((it_slot * a.heads + h) * TP128::SLOT + wave * TP::WAVE) * 4), lane,
                         oacc, m_run, l_run);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) s_arrived = atomicAdd(a.cnt + (first * a.heads + h), 1);
    __syncthreads();
    if (uniform(s_arrived) != it_chunks - 1 || !wave_rows) return;
    float M = -INFINITY, L = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    for (int k = 0; k < it_chunks; ++k)
        partial_fold<D>(rpart, (uint32_t)((((first + k) * a.heads + h) * TP128::SLOT + wave * TP::WAVE) * 4), lane,
                        oacc, M, L);
    store_rows<D, OF32>(a, h, row, row_valid, g, oacc, M, L, 1.0f);
}

// ---------------------------------------------------------------- unit kernel
template <int D, bool QF32, bool OF32>
__global__ __launch_bounds__(kUnitWaves * 64, 1) void attn_unit_kernel(AttnArgs a) {
    constexpr int kThreads = kUnitWaves * 64;
    using T = Tile<D, kUnitWaves>;
    using P = Partial<D>;
    constexpr int KS = D / 16;  // k-steps of the QK^T contraction
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    // One LDS object only (with several, the compiler can no longer tell the tile DMA's LDS
    // writes from the fragment reads and waits for every DMA before reading a stage): the
    // two tile stages, the unit table and a few words of schedule state.
    using PP = Pipe<D>;
    __shared__ __attribute__((aligned(1024))) char smem[PP::BYTES + kTableBytes + 256];
    static_assert(5 * kMaxTiles <= PP::BYTES, "per-tile scratch of the table build must fit the stages");
    int* u_tile = reinterpret_cast<int*>(smem + PP::BYTES);  // [units]: first tile | partner << 30
    int* u_pre = u_tile + kMaxTiles + 1;                        // [units + 1]: prefix of unit iterations
    int* t_it = reinterpret_cast<int*>(smem);                   // per-tile scratch in the stages
    unsigned char* t_same = reinterpret_cast<unsigned char*>(smem + 4 * kMaxTiles);
    char* tail = smem + PP::BYTES + kTableBytes;
    int* s_pos = reinterpret_cast<int*>(tail + 64);   // [4]
    int& s_arrived = *reinterpret_cast<int*>(tail + 96);
    int& s_bad = *reinterpret_cast<int*>(tail + 100);
    int& s_units = *reinterpret_cast<int*>(tail + 104);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qi = lane & 31, g = lane >> 5;
    const int grp = wave / kTileWaves;  // query tile of the unit this wave works on
    const int G = gridDim.x;
    const int w = xcd_logical(blockIdx.x, G);

    const int32_t* plan = a.plan;
    const int nq = a.n_qtiles;
    // a plan that does not belong to this call (another magic, rule, tile size or tile count) is
    // not read out of bounds: NaN outputs instead
    if (plan[0] != (int32_t)VDIT_PLAN_MAGIC || plan[2] != a.plan_kind || plan[3] != a.plan_tile || plan[4] != nq ||
        nq > kMaxTiles) {
        poison_share<D, OF32>(a, blockIdx.x, G);
        return;
    }
    const int n_spans = plan[5];
    const int32_t* qtiles = plan + VDIT_PLAN_HEADER_WORDS;
    const int32_t* row_ptr = qtiles + 2 * nq;
    const int32_t* spans = row_ptr + nq + 1;

    // ---- unit table.  Every workgroup validates the plan and builds the same table: tile q
    // gets its key iteration count and whether its span list equals tile q - 1's.  Runs of
    // equal lists are cut into units of two tiles (one tile at an odd run end); the two
    // tiles of a unit share every K/V tile.  Units are numbered per head in tile order.
    if (tid == 0) s_bad = 0;
    if (tid < 4) s_pos[tid] = 0;  // set by the share lookup below
    int bad = tid == 0 && !plan_for_call(plan, a) ? 1 : 0;  // built for another query call
    for (int q = tid; q < nq; q += kThreads) {
        const int qs = qtiles[2 * q], ql = qtiles[2 * q + 1], b = row_ptr[q], e = row_ptr[q + 1];
        int n = 0, same = 0;
        if (qs < 0 || ql < 1 || ql > kBM || (long long)qs + ql > a.n_tokens || b < 0 || b > e || e > n_spans) {
            bad = 1;
        } else {
            for (int sp = b; sp < e; ++sp) {  // spans must lie inside the cache, 8-aligned
                const int k0 = spans[2 * sp], kl = spans[2 * sp + 1];
                if (k0 < 0 || (k0 & 7) || kl < 1 || (long long)k0 + kl > a.kv_rows) bad = 1;
                n += (kl + kBN - 1) / kBN;
            }
            if (q > 0) {
                const int pb = row_ptr[q - 1], pe = row_ptr[q];
                same = pb >= 0 && pe - pb == e - b;
                for (int i = 0; same && i < 2 * (e - b); ++i) same = spans[2 * pb + i] == spans[2 * b + i];
            }
        }
        if (n > (1 << 24)) bad = 1;
        t_it[q] = n;
        t_same[q] = (unsigned char)same;
    }
    __syncthreads();
    if (__any(bad) && lane == 0) s_bad = 1;
    __syncthreads();
    if (uniform(s_bad)) {
        poison_share<D, OF32>(a, blockIdx.x, G);
        return;
    }
    if (wave == 0) {
        // run starts (max-scan), unit heads (even offset in the run), partners, unit numbers
        // and the prefix of unit iterations
        int carry_rs = 0, carry_units = 0, carry_sum = 0;
        for (int base = 0; base < nq; base += 64) {
            const int q = base + lane;
            const bool in = q < nq;
            int rs = in && !t_same[q] ? q : -1;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(rs, off);
                if (lane >= off) rs = max(rs, t);
            }
            rs = max(rs, carry_rs);
            const bool head = in && ((q - rs) & 1) == 0;
            const bool partner = head && q + 1 < nq && t_same[q + 1];
            const int hc = head ? 1 : 0, c = head ? t_it[q] : 0;
            int incl_h = hc, incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int th = __shfl_up(incl_h, off), t = __shfl_up(incl, off);
                if (lane >= off) {
                    incl_h += th;
                    incl += t;
                }
            }
            if (head) {
                const int k = carry_units + incl_h - 1;
                u_tile[k] = q | (partner ? 1 << 30 : 0);
                u_pre[k] = carry_sum + incl - c;
            }
            carry_rs = __shfl(rs, 63);
            carry_units += __shfl(incl_h, 63);
            carry_sum += __shfl(incl, 63);
        }
        if (lane == 0) {
            u_pre[carry_units] = carry_sum;
            s_units = carry_units;
        }
    }
    __syncthreads();
    const int n_units = uniform(s_units);         // units per head
    const long long t_head = uniform(u_pre[n_units]);  // iterations per head
    const long long total = t_head * a.heads;
    auto unit_iters = [&](int k) { return uniform(u_pre[k + 1] - u_pre[k]); };
    auto unit_tile = [&](int k) { return uniform(u_tile[k]) & ((1 << 30) - 1); };
    auto unit_partner = [&](int k) { return (uniform(u_tile[k]) >> 30) != 0; };

    auto write_empty = [&](int h, int q) {  // a query tile without keys: O = 0, LSE = -inf
        const int qs = qtiles[2 * q], ql = qtiles[2 * q + 1];
        for (int i = tid; i < ql * (D / 4); i += kThreads) {
            const int r = qs + i / (D / 4), d = (i % (D / 4)) * 4;
            const int64_t off = (int64_t)r * a.o_st + (int64_t)h * a.o_sh + d;
            if constexpr (OF32) *reinterpret_cast<float4*>(static_cast<float*>(a.o) + off) = make_float4(0, 0, 0, 0);
            else *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off) = make_uint2(0, 0);
        }
        if (a.lse)
            for (int r = tid; r < ql; r += kThreads) a.lse[(int64_t)h * a.n_tokens + qs + r] = -INFINITY;
    };
    const int n_all = n_units * a.heads;  // units of the call, numbered head-major
    for (int j = w; j < n_all; j += G) {
        const int k = j % n_units;
        if (unit_iters(k) == 0) {
            write_empty(j / n_units, unit_tile(k));
            if (unit_partner(k)) write_empty(j / n_units, unit_tile(k) + 1);
        }
    }
    if (total == 0) return;

    // ---- schedule.  Rounds of whole units first (workgroup w takes unit r G + w of round r:
    // neighbouring workgroups, which share an XCD, work on neighbouring units with similar
    // key sets at the same time), then the units left over (fewer than G) as a stream:
    // their iterations laid end to end, every workgroup takes an equal contiguous share.
    // The stream balances the iterations exactly but splits units: a split costs a second
    // segment start, a partial result written and read back, and keys read out of step with
    // the neighbours.  So when the units do not fill whole rounds, the leftovers are taken as
    // one more round of whole units instead (workgroups without a unit in it are idle) if the
    // bound on a workgroup's work, the sum over rounds of the round's longest unit, exceeds
    // the balanced share by at most 3/16 of it and by at most 40 iterations.
    const int R = (n_all + G - 1) / G;
    bool whole = false;
    if (n_all % G != 0 && R <= PP::BYTES / 4) {
        int* s_rmax = reinterpret_cast<int*>(smem);  // [R], in the stages: free until the first segment
        int& s_whole = *reinterpret_cast<int*>(tail + 108);
        for (int r = tid; r < R; r += kThreads) s_rmax[r] = 0;
        __syncthreads();
        for (int j = tid; j < n_all; j += kThreads) {
            const int k = j % n_units;
            atomicMax(&s_rmax[j / G], u_pre[k + 1] - u_pre[k]);
        }
        __syncthreads();
        if (wave == 0) {
            long long m = 0;
            for (int r = lane; r < R; r += 64) m += s_rmax[r];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m += __shfl_xor(m, off);
            if (lane == 0) {
                const long long share = (total + G - 1) / G;
                s_whole = m <= share + min(share * 3 / 16, 40LL);
            }
        }
        __syncthreads();
        whole = uniform(s_whole) != 0;
    }
    const int rounds = whole ? R : n_all / G;
    const long long sk_base =
        whole ? total : (long long)(rounds * G / n_units) * t_head + u_pre[(rounds * G) % n_units];
    const long long sk_len = total - sk_base;
    const long long B = sk_base + (long long)w * sk_len / G, E = sk_base + (long long)(w + 1) * sk_len / G;

    // the units holding this workgroup's first and last stream iteration: the largest k with
    // u_pre[k] <= r (a unit with iterations, as u_pre[k + 1] > r)
    if (tid < 2 && B < E) {
        const int r = (int)((tid == 0 ? B : E - 1) % t_head);
        int lo = 0, hi = n_units - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (u_pre[mid] <= r) lo = mid;
            else hi = mid - 1;
        }
        s_pos[2 * tid] = lo;
        s_pos[2 * tid + 1] = r - u_pre[lo];
    }
    __syncthreads();
    // the share = [ib_b, ..) of unit b, whole units, [0, ie_l) of unit l (b == l: one segment)
    const int h_b = (int)(B / t_head), k_b = uniform(s_pos[0]), ib_b = uniform(s_pos[1]);
    const int h_l = (int)((E - 1) / t_head), k_l = uniform(s_pos[2]), ie_l = uniform(s_pos[3]) + 1;
    const long long ut_b = B - ib_b, ut_l = E - ie_l;  // global index of those units' first iteration
    const bool single = h_b == h_l && k_b == k_l;

    // the workgroup whose share holds stream iteration x, and the start of a share
    auto wg_begin = [&](int u) -> long long { return sk_base + (long long)u * sk_len / G; };
    auto wg_of = [&](long long x) -> int {
        int u = (int)((x - sk_base) * G / sk_len);
        while (u + 1 < G && wg_begin(u + 1) <= x) ++u;
        return u;
    };

    const float c = a.scale_log2;
    // the exponent base m_run and the merge below are in log2 units (Q carries c)
    const __amdgpu_buffer_rsrc_t rpart = head_rsrc(a.part, (uint32_t)((size_t)2 * G * P::SLOT * 4));
    const int wave_u = uniform(wave);
    const DmaLane<D / 8> kdl = dma_lane<D / 8>(wave_u, lane);
    const DmaLane<kBN / 8> vdl = dma_lane<kBN / 8>(wave_u, lane);
    const uint32_t head_bytes = (uint32_t)(a.kv_rows * D * 2);
    const uint32_t vpitch = (uint32_t)(a.kv_rows * 2);
    const PipeLane<D> pl = pipe_lane<D, 3>(qi, g);

    // Segment order of the stream share.  The unit l segment (from its first iteration) comes
    // first, then the whole units, each started at the iteration index equal to the stream
    // iterations done so far (mod its length) and wrapped around, then the unit b segment.  For units with equal
    // span lists (chunk-causal, dense) all workgroups then read the same K/V rows at about
    // the same time, up to a fixed offset ((n - share) mod n iterations), so those rows
    // are fetched into each XCD's L2 once.  Softmax accumulation is order-free.
    const int sk_phase = B == E ? 4 : single ? 2 : 0;
    int phase = rounds > 0 ? -1 : sk_phase;  // -1: rounds, 0: unit l, 1: whole units, 2: unit b
    int round = 0;
    int mh = h_b, mk = k_b;  // whole-unit walk of the stream share, starts at unit b
    long long mut = ut_b;
    long long elapsed = 0;  // stream iterations done
    for (;;) {
        int h, k, ib, ie, slot;
        long long ut;
        bool stream = true;
        if (phase == -1) {
            int j = round * G + w;
            if (whole && round == rounds - 1) {
                // the last round's L units in equal contiguous shares per XCD (the idle workgroups
                // spread over all XCDs); j = n_all: no unit
                constexpr int kXcd = 8;
                const int L = n_all - round * G, q = L / kXcd, r = L % kXcd;
                const int xcd = blockIdx.x % kXcd, idx = blockIdx.x / kXcd;
                j = idx < q + (xcd < r ? 1 : 0) ? round * G + xcd * q + min(xcd, r) + idx : n_all;
            }
            h = j / n_units, k = j % n_units, ut = 0, ib = 0, ie = j < n_all ? -1 : 0, slot = 0;
            stream = false;
            if (++round == rounds) phase = sk_phase;
        } else if (phase == 0) {
            h = h_l, k = k_l, ut = ut_l, ib = 0, ie = ie_l, slot = 1;
            phase = 1;
        } else if (phase == 1) {
            mut += unit_iters(mk);
            if (++mk == n_units) {
                mk = 0;
                ++mh;
            }
            if (mh == h_l && mk == k_l) {
                phase = 2;
                continue;
            }
            h = mh, k = mk, ut = mut, ib = 0, ie = -1, slot = 0;  // ie = n below
        } else if (phase == 2) {
            h = h_b, k = k_b, ut = ut_b, ib = ib_b, ie = single ? ie_l : -1, slot = 0;
            phase = 3;
        } else {
            break;
        }
        const int n = unit_iters(k);
        const int q = unit_tile(k);
        if (ie < 0) ie = n;
        if (ie > ib) {
            // ---- this wave's query tile of the unit (the second tile may not exist)
            const int my_tile = grp == 0 ? q : (unit_partner(k) ? q + 1 : -1);
            const int q_start = my_tile >= 0 ? plan_word(qtiles + 2 * my_tile) : 0;
            const int q_len = my_tile >= 0 ? plan_word(qtiles + 2 * my_tile + 1) : 1;
            // uniform per wave: the tile exists and holds some of the wave's 32 rows (a wave past
            // the end of a short tile keeps its share of the DMA and the barriers, nothing else);
            // read as a scalar so that its branches need no saved exec mask
            const bool active = uniform(my_tile >= 0 && uniform(wave % kTileWaves) * 32 < q_len ? 1 : 0) != 0;
            const int r_in = (wave % kTileWaves) * 32 + qi;
            const bool row_valid = active && r_in < q_len;
            const int row = q_start + (r_in < q_len ? r_in : q_len - 1);
            bf16x8 qreg[KS];
            f32x16 oacc[DB];
#pragma unroll
            for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
            // Running max of the raw scores used as the exponent base.  It is only raised when
            // a tile's max exceeds it by more than kLazy (in log2 units), so most tiles skip
            // the rescale of O; p = exp2((s - m) * c) then stays below 2^kLazy.
            float m_run = -INFINITY, l_run = 0.f;

            // first key tile of the segment: a whole unit starts at elapsed mod n and wraps
            const int sp_begin = plan_word(row_ptr + q), sp_end = plan_word(row_ptr + q + 1);
            int span = sp_begin, skip = stream && ib == 0 && ie == n ? (int)(elapsed % n) : ib;
            for (;;) {
                const int cnt = (plan_word(spans + 2 * span + 1) + kBN - 1) / kBN;
                if (skip < cnt) break;
                skip -= cnt;
                ++span;
            }
            const int span_k0 = plan_word(spans + 2 * span);
            int k0 = span_k0 + skip * kBN, kend = span_k0 + plan_word(spans + 2 * span + 1);
            const __amdgpu_buffer_rsrc_t rk = head_rsrc(a.kc + (int64_t)h * a.kv_rows * D, head_bytes);
            const __amdgpu_buffer_rsrc_t rv = head_rsrc(a.vt + (int64_t)h * D * a.kv_rows, head_bytes);
            // Key tiles of the segment: n (k0, kend), n + 1 (k1, kend1), and the span of the
            // furthest tile located so far.  A span ends in a ragged tile; whole units wrap
            // from the last span to the first.
            int left = ie - ib - 1;  // tiles after tile n
            int k1 = 0, kend1 = 0;
            auto advance = [&](int k, int ke, int& nk, int& nke) {
                nk = k + kBN;
                nke = ke;
                if (nk >= ke) {
                    span = span + 1 == sp_end ? sp_begin : span + 1;
                    nk = plan_word(spans + 2 * span);
                    nke = nk + plan_word(spans + 2 * span + 1);
                }
            };
            __syncthreads();  // the previous segment's LDS reads are done
            pipe_load<D, kUnitWaves, 3>(rk, rv, vpitch, k0, kend, wave_u, kdl, vdl, smem, 0, 0);
            if (left >= 1) {
                advance(k0, kend, k1, kend1);
                pipe_load<D, kUnitWaves, 3>(rk, rv, vpitch, k1, kend1, wave_u, kdl, vdl, smem, 1, 1);
            }
            // Q loads overlap the first K/V tiles; Q carries the softmax scale and log2(e)
            if (active) load_q_rows<D, QF32>(a, h, row, g, qreg, c);
            wait_tile_loads();
            __syncthreads();
            f32x16 sacc[2][2];
            f32x16 negm;
            if (active) {
                pipe_scores<D, 3>(smem, pl, 0, qreg, sacc[0]);
                pipe_first(sacc[0], k0 + kBN > kend, kend - k0 - g * 8, m_run, negm);
            }
            // Step n: tile n's V^T is in stage n mod 3 and tile n + 1's K in the next stage; the
            // loop is unrolled by 6 (three stages times two score buffers) so that stages and
            // buffers are constants.
            auto key_step = [&](auto stc, auto sbc) {  // returns false after the segment's last tile
                constexpr int ST = decltype(stc)::value, SB = decltype(sbc)::value;
                constexpr int ST1 = (ST + 1) % 3, ST2 = (ST + 2) % 3;
                // tile n + 1 has landed (every wave's share of its DMA) and stage ST2 is free:
                // every wave is done with tile n - 1
                wait_tile_loads();
                __syncthreads();
                int k2 = 0, kend2 = 0;
                if (left >= 2) {
                    advance(k1, kend1, k2, kend2);
                    pipe_load<D, kUnitWaves, 3>(rk, rv, vpitch, k2, kend2, wave_u, kdl, vdl, smem, ST2, ST2);
                }
                if (active) {
                    float mt;
                    pipe_step<D, 3, ST, ST1>(smem, pl, qreg, oacc, sacc[SB], sacc[SB ^ 1], negm, l_run, mt);
                    if (left >= 1)
                        pipe_fixup<D>(sacc[SB ^ 1], k1 + kBN > kend1, kend1 - k1 - g * 8, mt, m_run, l_run, oacc, negm);
                }
                if (left == 0) return false;
                --left;
                k0 = k1;
                kend = kend1;
                k1 = k2;
                kend1 = kend2;
                return true;
            };
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            while (key_step(I0{}, I0{}) && key_step(I1{}, I1{}) && key_step(I2{}, I0{}) && key_step(I0{}, I1{}) &&
                   key_step(I1{}, I0{}) && key_step(I2{}, I1{})) {
            }

            if (ib == 0 && ie == n) {
                if (active) store_rows<D, OF32>(a, h, row, row_valid, g, oacc, m_run, l_run, 1.0f);
            } else {
                // Split unit: leave the partial in this workgroup's slot (0: the first unit of
                // its share, 1: the last), then count in.
                const uint32_t pw = (uint32_t)(((2 * w + slot) * P::SLOT + wave * P::WAVE) * 4);
                if (active) partial_store<D>(rpart, pw, lane, oacc, m_run, l_run);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                int32_t* counter = a.cnt + (h * n_units + k);
                if (tid == 0) s_arrived = atomicAdd(counter, 1);
                __syncthreads();
                const int arrived = uniform(s_arrived);
                // the unit's segments = the non-empty shares that meet [ut, ut + n)
                const int u0 = wg_of(ut), u1 = wg_of(ut + n - 1);
                int nseg = 0;
                for (int u = u0; u <= u1; ++u) nseg += wg_begin(u + 1) > wg_begin(u);
                if (arrived == nseg - 1) {
                    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (active) {
                        // Segments are folded in descending share order, the same order
                        // whichever workgroup merges, all of them from the workspace (this
                        // workgroup's own partial too: O and its row state start empty here, so
                        // the accumulators of the key loop are free).
                        float M = -INFINITY, L = 0.f;
#pragma unroll
                        for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
                        for (int u = u1; u >= u0; --u) {
                            const long long ub = wg_begin(u);
                            if (wg_begin(u + 1) == ub) continue;
                            const uint32_t pu = (uint32_t)(((2 * u + (ub >= ut ? 0 : 1)) * P::SLOT + wave * P::WAVE) * 4);
                            // partial_fold written out: as a call, the register allocator spills
                            // inside the key loop
                            const u32x2 mlu =
                                __builtin_amdgcn_raw_buffer_load_b64(rpart, pu + P::O_FLOATS * 4 + lane * 8, 0, kSc1);
                            const float mu = __uint_as_float(mlu[0]), lu = __uint_as_float(mlu[1]);
                            const float mn = fmaxf(M, mu);
                            const float a1 = M == -INFINITY ? 0.f : fast_exp2(M - mn);
                            const float a2 = mu == -INFINITY ? 0.f : fast_exp2(mu - mn);
#pragma unroll
                            for (int db = 0; db < DB; ++db) {
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const u32x4 vu = __builtin_amdgcn_raw_buffer_load_b128(
                                        rpart, pu + lane * 16, (db * 4 + j) * 1024, kSc1);
#pragma unroll
                                    for (int e = 0; e < 4; ++e)
                                        oacc[db][4 * j + e] = oacc[db][4 * j + e] * a1 + __uint_as_float(vu[e]) * a2;
                                }
                                sched_fence();
                            }
                            L = L * a1 + lu * a2;
                            M = mn;
                        }
                        store_rows<D, OF32>(a, h, row, row_valid, g, oacc, M, L, 1.0f);
                    }
                }
            }
        }
        if (stream) elapsed += ie - ib;
        if (phase == 3) break;
    }
}

// Workspace layouts (caller-owned, see vdit_block_attn_workspace_bytes), every region 256-byte
// aligned.  Tile kernel on a dynamic plan: the item count, the item list, the arrival counters
// and the partial slots of split tiles; the schedule kernel writes all of them before the
// attention kernel reads any, so their contents between calls do not matter.  Unit kernel: the
// split-unit partials (two slots per workgroup, sized for head_dim 128 whatever the call's) from
// offset 0, then the per-tile arrival counters, above the largest dynamic-plan layout as well.
// A counter word is thus never used as anything else, by either kernel, and stays zero between
// calls (the last arriver of a tile resets it): the caller zeroes the workspace once.
constexpr size_t align256(size_t b) { return (b + 255) / 256 * 256; }

struct TileWs {
    size_t items, cnt, part, bytes;
};
constexpr TileWs tile_ws(int32_t n_qtiles, int32_t heads) {
    TileWs w{};
    w.items = 256;
    w.cnt = w.items + align256((size_t)tile_items_max(n_qtiles, heads) * sizeof(TileItem));
    w.part = w.cnt + align256((size_t)kSplitCap * 4);
    w.bytes = w.part + (size_t)kSplitCap * Partial<128, kTileWaves>::SLOT * 4;
    return w;
}

size_t partial_bytes(int grid) { return (size_t)2 * grid * Partial<128>::SLOT * 4; }

// the largest dynamic-plan layout (kMaxTiles query tiles, one head)
constexpr size_t kTileWsMax = tile_ws(kMaxTiles, 1).bytes;

}  // namespace

// Workgroups of the unit kernel: one per CU (its LDS admits no second), a multiple of 8 so
// that the XCD renumbering is exact.
hipError_t attn_unit_grid(int* grid) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    *grid = cus / 8 * 8 < 8 ? 8 : cus / 8 * 8;
    return hipSuccess;
}

size_t attn_workspace_bytes(int grid, int32_t heads, int32_t n_qtiles, bool unit_kernel, bool split) {
    if (unit_kernel) return attn_workspace_counter_offset(grid) + (size_t)heads * n_qtiles * 4;
    return split ? tile_ws(n_qtiles, heads).bytes : 0;
}

size_t attn_workspace_counter_offset(int grid) { return std::max(partial_bytes(grid), kTileWsMax); }

// Scratch of the allocation-free attention entry point: one array per GPU the library runs
// on, held until the process ends, shared by every call on that GPU.  Host code never uses
// its name as an address (that is a host-side stand-in): the device address comes from
// hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) char scratch[kAttnStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t attn_static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

namespace {

template <int D, bool QF, bool OF>
hipError_t launch_unit(AttnArgs a, char* ws, hipStream_t s) {
    int grid = 0;
    hipError_t e = attn_unit_grid(&grid);
    if (e != hipSuccess) return e;
    a.part = reinterpret_cast<float*>(ws);
    a.cnt = reinterpret_cast<int32_t*>(ws + attn_workspace_counter_offset(grid));
    attn_unit_kernel<D, QF, OF><<<grid, kUnitWaves * 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, bool QF, bool OF>
hipError_t launch_tile(AttnArgs a, bool split, char* ws, hipStream_t s) {
    unsigned blocks = (unsigned)(a.n_qtiles * a.heads);
    a.items = nullptr;
    a.n_items = nullptr;
    if (split) {  // dynamic plan: the work list first, on the same stream
        const TileWs w = tile_ws(a.n_qtiles, a.heads);
        int32_t* n_items = reinterpret_cast<int32_t*>(ws);
        TileItem* items = reinterpret_cast<TileItem*>(ws + w.items);
        a.cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
        a.part = reinterpret_cast<float*>(ws + w.part);
        tile_schedule_kernel<<<1, kSchedThreads, 0, s>>>(a.plan, a.n_qtiles, a.heads, a.kv_rows, items, n_items,
                                                         a.cnt);
        a.items = items;
        a.n_items = n_items;
        blocks = (unsigned)(tile_items_max(a.n_qtiles, a.heads) * a.heads);
    }
    attn_tile_kernel<D, QF, OF><<<blocks, kTileWaves * 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, bool QF, bool OF>
hipError_t launch_k(const AttnLaunch& L, const AttnArgs& a, hipStream_t s) {
    char* ws = static_cast<char*>(L.workspace);
    if (attn_uses_tile_kernel(L.mask_kind, L.unpaired)) return launch_tile<D, QF, OF>(a, L.unpaired, ws, s);
    return launch_unit<D, QF, OF>(a, ws, s);
}

template <int D>
hipError_t launch_d(const AttnLaunch& L, const AttnArgs& a, hipStream_t s) {
    bool qf = L.q.dtype == VDIT_DTYPE_FP32, of = L.o.dtype == VDIT_DTYPE_FP32;
    if (qf && of) return launch_k<D, true, true>(L, a, s);
    if (qf) return launch_k<D, true, false>(L, a, s);
    if (of) return launch_k<D, false, true>(L, a, s);
    return launch_k<D, false, false>(L, a, s);
}

}  // namespace

hipError_t launch_attn_fwd(const AttnLaunch& L, hipStream_t s) {
    AttnArgs a{};
    a.q = L.q.data;
    a.q_st = L.q.stride_token;
    a.q_sh = L.q.stride_head;
    a.o = L.o.data;
    a.o_st = L.o.stride_token;
    a.o_sh = L.o.stride_head;
    a.lse = L.lse;
    a.kc = static_cast<const uint16_t*>(L.kc);
    a.vt = static_cast<const uint16_t*>(L.vt);
    a.kv_rows = L.kv_rows;
    a.plan = L.plan;
    a.rope = L.rope;
    a.has_rope = L.has_rope ? 1 : 0;
    a.hw = L.hw;
    a.wf = L.wf;
    a.t0 = L.t0;
    a.n_tokens = L.n_tokens;
    a.heads = L.heads;
    a.n_qtiles = L.n_qtiles;
    a.plan_kind = L.plan_kind;
    a.plan_tile = L.plan_tile;
    a.scale_log2 = L.scale_log2;
    if (L.head_dim == 128) return launch_d<128>(L, a, s);
    return launch_d<64>(L, a, s);
}

}  // namespace vdit
