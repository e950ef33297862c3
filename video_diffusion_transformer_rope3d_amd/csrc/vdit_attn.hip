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
#include <map>
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
    float scale_log2;
    int32_t* cnt;  // per-tile arrival counters, zero between calls
    float* part;   // partial results, two slots per workgroup
    const int32_t* order;  // tile kernel: query tiles longest first (NULL: plan order)
};

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keeps the instruction scheduler from moving anything across this point, so that the
// fragment reads of one phase are not hoisted into the previous one (register pressure).
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
__device__ inline int plan_word(const int32_t* p) {
    return __builtin_amdgcn_readfirstlane(*(const const_i32_t*)p);
}

// Q rows of one wave (this lane's row), RoPE applied at the global position while loading.
// All row loads are issued first, then the table loads of half the chunks at a time (a
// bound on live registers), so the segment start waits for a few round trips instead of
// one per chunk.
template <int D, bool QF32>
__device__ __forceinline__ void load_q_rows(const AttnArgs& a, int h, int row, int g, bf16x8 (&qreg)[D / 16]) {
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
            qreg[ks] = __builtin_bit_cast(bf16x8, pack_bf16x8(x));
        }
    }
}

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

// ---------------------------------------------------------------- tile kernel
// One workgroup = one (query tile, head), 4 waves, two workgroups per CU; the grid covers
// all tiles of all heads.  Used where neighbouring query tiles have different span lists
// (log-radial), so that two tiles cannot share one K/V stream.
//
// Workgroups are dispatched round-robin over the 8 XCDs; renumber so that each XCD gets a
// contiguous range of (head, query tile) items, whose K/V then stream through its L2.
__device__ inline int xcd_remap(int bid, int total) {
    constexpr int kXcd = 8;
    int q = total / kXcd, r = total % kXcd;
    int xcd = bid % kXcd, idx = bid / kXcd;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

template <int D, bool QF32, bool OF32>
__global__ __launch_bounds__(kTileWaves * 64, 2) void attn_tile_kernel(AttnArgs a) {
    using T = Tile<D, kTileWaves>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qi = lane & 31, g = lane >> 5;
    int h, qt;
    if (a.order) {  // longest tiles first, all heads of a tile together
        qt = a.order[blockIdx.x / a.heads];
        h = blockIdx.x % a.heads;
    } else {
        const int item = xcd_remap(blockIdx.x, a.n_qtiles * a.heads);
        h = item / a.n_qtiles;
        qt = item % a.n_qtiles;
    }

    const int32_t* plan = a.plan;
    const int nq = plan[4];
    // a plan that does not belong to this call is ignored rather than read out of bounds
    if (plan[0] != (int32_t)VDIT_PLAN_MAGIC || nq != a.n_qtiles || qt >= nq) return;
    const int32_t* qtiles = plan + VDIT_PLAN_HEADER_WORDS;
    const int32_t* row_ptr = qtiles + 2 * nq;
    const int32_t* spans = row_ptr + nq + 1;
    const int q_start = plan_word(qtiles + 2 * qt), q_len = plan_word(qtiles + 2 * qt + 1);
    const int sp_begin = plan_word(row_ptr + qt), sp_end = plan_word(row_ptr + qt + 1);
    if (q_start < 0 || q_len < 1 || q_len > kBM || q_start + q_len > a.n_tokens || sp_begin < 0 ||
        sp_begin > sp_end || sp_end > plan[5])
        return;
    for (int sp = sp_begin; sp < sp_end; ++sp) {  // spans must lie inside the cache, 8-aligned
        const int k0 = spans[2 * sp], kl = spans[2 * sp + 1];
        if (k0 < 0 || (k0 & 7) || kl < 1 || (int64_t)k0 + kl > a.kv_rows) return;
    }

    const int r_in = wave * 32 + qi;
    const bool row_valid = r_in < q_len;
    const int row = q_start + (row_valid ? r_in : q_len - 1);
    // a wave whose 32 rows all lie past the tile's end (the short last tile of a frame) keeps
    // its share of the DMA and the barriers but skips the math
    const bool wave_rows = uniform(wave) * 32 < q_len;
    bf16x8 qreg[KS];
    if (wave_rows) load_q_rows<D, QF32>(a, h, row, g, qreg);

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    const float c = a.scale_log2;
    const float lazy_raw = kLazy / c;
    float m_run = -INFINITY, l_run = 0.f;

    if (sp_begin < sp_end) {
        int span = sp_begin;
        int k0 = plan_word(spans + 2 * span), kend = k0 + plan_word(spans + 2 * span + 1);
        // The words of the span after the current one, loaded when the current one starts with a
        // vector load (counted by vmcnt, so the tile waits cover it), so that crossing into the
        // next span does not wait for a plan read before the next tile's DMA is issued.
        const __amdgpu_buffer_rsrc_t rsp = head_rsrc(spans, (uint32_t)sp_end * 8);
        u32x2 pf = {0u, 0u};
        if (span + 1 < sp_end) pf = __builtin_amdgcn_raw_buffer_load_b64(rsp, (uint32_t)(span + 1) * 8, 0, 0);
        const int wave_u = uniform(wave);
        const DmaLane<D / 8> kdl = dma_lane<D / 8>(wave_u, lane);
        const DmaLane<kBN / 8> vdl = dma_lane<kBN / 8>(wave_u, lane);
        const uint32_t head_bytes = (uint32_t)(a.kv_rows * D * 2);
        const __amdgpu_buffer_rsrc_t rk = head_rsrc(a.kc + (int64_t)h * a.kv_rows * D, head_bytes);
        const __amdgpu_buffer_rsrc_t rv = head_rsrc(a.vt + (int64_t)h * D * a.kv_rows, head_bytes);
        const uint32_t vpitch = (uint32_t)(a.kv_rows * 2);
        FragLane fl;
        fl.qi = qi, fl.g = g, fl.krow = swap23(qi);
        fl.kswz = swz<T::KCH>(fl.krow), fl.vswz = swz<T::VCH>(qi);
        load_tile_lds<D, kTileWaves>(rk, rv, vpitch, k0, kend, wave_u, kdl, vdl, smem);
        wait_tile_loads();
        __syncthreads();
        // (not unrolled by stage as the unit kernel is: measured 2% slower here)
        int buf = 0;
        while (true) {
            int nk0 = k0 + kBN, nkend = kend, nspan = span;
            if (nk0 >= kend) {
                ++nspan;
                if (nspan < sp_end) {
                    nk0 = uniform((int)pf[0]);
                    nkend = nk0 + uniform((int)pf[1]);
                    if (nspan + 1 < sp_end)
                        pf = __builtin_amdgcn_raw_buffer_load_b64(rsp, (uint32_t)(nspan + 1) * 8, 0, 0);
                }
            }
            const bool has_next = nspan < sp_end;
            if (has_next)
                load_tile_lds<D, kTileWaves>(rk, rv, vpitch, nk0, nkend, wave_u, kdl, vdl,
                                             smem + (buf ^ 1) * T::STAGE);
            if (wave_rows)
                tile_step<D, kTileWaves>(smem + buf * T::STAGE, fl, qreg, oacc, m_run, l_run, c, lazy_raw, k0, kend);
            if (!has_next) break;
            wait_tile_loads();
            __syncthreads();
            buf ^= 1;
            k0 = nk0;
            kend = nkend;
            span = nspan;
        }
    }
    store_rows<D, OF32>(a, h, row, row_valid, g, oacc, m_run, l_run, c);
}

// ---------------------------------------------------------------- tile order
// Query tiles of a dynamic-threshold plan carry very different numbers of keys.  Workgroups
// start in grid order, so the tile kernel takes its (tile, head) items longest first (list
// scheduling: the long ones do not end up in the last wave of workgroups).  One workgroup
// sums each tile's span lengths (a wave per tile) and ranks the tiles by (count, lower tile
// first): a tile's rank is the number of tiles ahead of it, read from LDS by every thread in
// step (broadcast reads, no barriers).  A plan that does not belong to the call gives the
// plan order; the tile kernel rejects its items itself.
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void tile_order_kernel(const int32_t* plan, int32_t nq, int32_t* order) {
    __shared__ int32_t s_rp[kMaxTiles + 1];
    __shared__ int32_t s_cnt[kMaxTiles];
    const int tid = threadIdx.x;
    const bool ok = plan[0] == (int32_t)VDIT_PLAN_MAGIC && plan[4] == nq && nq <= kMaxTiles;
    const int n_spans = ok ? plan[5] : 0;
    const int32_t* row_ptr = plan + VDIT_PLAN_HEADER_WORDS + 2 * nq;
    const int32_t* spans = row_ptr + nq + 1;
    for (int t = tid; t <= nq; t += kOrderThreads) s_rp[t] = ok ? row_ptr[t] : 0;
    __syncthreads();
    // one wave per tile: lanes stride over the tile's spans, a shuffle tree adds them
    const int lane = tid & 63, wave = tid >> 6;
    for (int t = wave; t < nq; t += kOrderThreads / 64) {
        const int b = max(s_rp[t], 0), e = min(s_rp[t + 1], n_spans);
        int n = 0;
        for (int sp = b + lane; sp < e; sp += 64) n += max(spans[2 * sp + 1], 0);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
        if (lane == 0) s_cnt[t] = n;
    }
    __syncthreads();
    for (int t = tid; t < nq; t += kOrderThreads) {
        const unsigned c = (unsigned)s_cnt[t];
        int rank = 0;
        for (int u = 0; u < nq; ++u) {
            const unsigned cu = (unsigned)s_cnt[u];
            rank += cu > c || (cu == c && u < t);
        }
        order[rank] = t;
    }
}

// ---------------------------------------------------------------- unit kernel
constexpr int kSc1 = 16;  // cache-policy operand of the buffer builtins: device scope (sc1)

// Floats of one workgroup's partial result: per wave the O^T accumulators of its 64 lanes
// (DB * 16 floats each, stored float4-interleaved over lanes) and the lanes' (max, sum).
template <int D>
struct Partial {
    static constexpr int DB = D / 32;
    static constexpr int O_FLOATS = DB * 16 * 64;
    static constexpr int WAVE = O_FLOATS + 2 * 64;
    static constexpr int SLOT = kUnitWaves * WAVE;
};

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
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::STAGE + kTableBytes + 256];
    static_assert(5 * kMaxTiles <= 2 * T::STAGE, "per-tile scratch of the table build must fit the stages");
    int* u_tile = reinterpret_cast<int*>(smem + 2 * T::STAGE);  // [units]: first tile | partner << 30
    int* u_pre = u_tile + kMaxTiles + 1;                        // [units + 1]: prefix of unit iterations
    int* t_it = reinterpret_cast<int*>(smem);                   // per-tile scratch in the stages
    unsigned char* t_same = reinterpret_cast<unsigned char*>(smem + 4 * kMaxTiles);
    char* tail = smem + 2 * T::STAGE + kTableBytes;
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
    // a plan that does not belong to this call is ignored rather than read out of bounds
    if (plan[0] != (int32_t)VDIT_PLAN_MAGIC || plan[4] != nq || nq > kMaxTiles) return;
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
    int bad = 0;
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
    if (uniform(s_bad)) return;
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
    if (n_all % G != 0 && R <= 2 * T::STAGE / 4) {
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
    const float lazy_raw = kLazy / c;
    const __amdgpu_buffer_rsrc_t rpart = head_rsrc(a.part, (uint32_t)((size_t)2 * G * P::SLOT * 4));
    const int wave_u = uniform(wave);
    const DmaLane<D / 8> kdl = dma_lane<D / 8>(wave_u, lane);
    const DmaLane<kBN / 8> vdl = dma_lane<kBN / 8>(wave_u, lane);
    const uint32_t head_bytes = (uint32_t)(a.kv_rows * D * 2);
    const uint32_t vpitch = (uint32_t)(a.kv_rows * 2);
    FragLane fl;
    fl.qi = qi, fl.g = g, fl.krow = swap23(qi);
    fl.kswz = swz<T::KCH>(fl.krow), fl.vswz = swz<T::VCH>(qi);

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
            // the end of a short tile keeps its share of the DMA and the barriers, nothing else)
            const bool active = my_tile >= 0 && uniform(wave % kTileWaves) * 32 < q_len;
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
            __syncthreads();  // the previous segment's LDS reads are done
            load_tile_lds<D, kUnitWaves>(rk, rv, vpitch, k0, kend, wave_u, kdl, vdl, smem);
            // Q loads overlap the first K/V tile
            if (active) load_q_rows<D, QF32>(a, h, row, g, qreg);

            wait_tile_loads();
            __syncthreads();
            // The loop is unrolled by the two stages, so that each stage's LDS address is a
            // constant (the fragment reads take it as their immediate offset instead of
            // adding it per read).
            int left = ie - ib - 1;
            auto key_step = [&](auto bufc) {  // returns false after the segment's last tile
                constexpr int BUF = decltype(bufc)::value;
                int nk0 = k0 + kBN, nkend = kend;
                if (left > 0 && nk0 >= kend) {
                    span = span + 1 == sp_end ? sp_begin : span + 1;
                    nk0 = plan_word(spans + 2 * span);
                    nkend = nk0 + plan_word(spans + 2 * span + 1);
                }
                if (left > 0)
                    load_tile_lds<D, kUnitWaves>(rk, rv, vpitch, nk0, nkend, wave_u, kdl, vdl, smem + (BUF ^ 1) * T::STAGE);
                if (active)
                    tile_step<D, kUnitWaves>(smem + BUF * T::STAGE, fl, qreg, oacc, m_run, l_run, c, lazy_raw, k0, kend);
                if (left == 0) return false;
                wait_tile_loads();
                __syncthreads();
                --left;
                k0 = nk0;
                kend = nkend;
                return true;
            };
            while (key_step(std::integral_constant<int, 0>{}) && key_step(std::integral_constant<int, 1>{})) {
            }

            if (ib == 0 && ie == n) {
                if (active) store_rows<D, OF32>(a, h, row, row_valid, g, oacc, m_run, l_run, c);
            } else {
                // Split unit: leave the partial in this workgroup's slot (0: the first unit of
                // its share, 1: the last), then count in.  Partials are written and read with
                // device-scope (sc1) accesses, which go to the point of coherence of all XCDs, so
                // the per-XCD L2s need no write-back or invalidation; each wave waits for its
                // stores to complete before the workgroup counts in.
                const uint32_t pw = (uint32_t)(((2 * w + slot) * P::SLOT + wave * P::WAVE) * 4);
                if (active) {
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const u32x4 v = {__float_as_uint(oacc[db][4 * j]), __float_as_uint(oacc[db][4 * j + 1]),
                                             __float_as_uint(oacc[db][4 * j + 2]),
                                             __float_as_uint(oacc[db][4 * j + 3])};
                            __builtin_amdgcn_raw_buffer_store_b128(v, rpart, pw + ((db * 4 + j) * 64 + lane) * 16, 0,
                                                                   kSc1);
                        }
                    const u32x2 ml = {__float_as_uint(m_run), __float_as_uint(l_run)};
                    __builtin_amdgcn_raw_buffer_store_b64(ml, rpart, pw + P::O_FLOATS * 4 + lane * 8, 0, kSc1);
                }
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
                        // whichever workgroup merges.  The last arriver usually holds the last
                        // segment; its partial is then the first one folded, which leaves it
                        // unchanged, so it is taken from the registers instead of being re-read.
                        int ulast = u1;
                        while (wg_begin(ulast + 1) == wg_begin(ulast)) --ulast;
                        const bool own_first = ulast == w;
                        float M = own_first ? m_run : -INFINITY, L = own_first ? l_run : 0.f;
                        if (!own_first) {
#pragma unroll
                            for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
                        }
                        for (int u = own_first ? ulast - 1 : ulast; u >= u0; --u) {
                            const long long ub = wg_begin(u);
                            if (wg_begin(u + 1) == ub) continue;
                            const uint32_t pu = (uint32_t)(((2 * u + (ub >= ut ? 0 : 1)) * P::SLOT + wave * P::WAVE) * 4);
                            const u32x2 mlu =
                                __builtin_amdgcn_raw_buffer_load_b64(rpart, pu + P::O_FLOATS * 4 + lane * 8, 0, kSc1);
                            const float mu = __uint_as_float(mlu[0]), lu = __uint_as_float(mlu[1]);
                            const float mn = fmaxf(M, mu);
                            const float a1 = M == -INFINITY ? 0.f : fast_exp2((M - mn) * c);
                            const float a2 = mu == -INFINITY ? 0.f : fast_exp2((mu - mn) * c);
#pragma unroll
                            for (int db = 0; db < DB; ++db)
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const u32x4 vu = __builtin_amdgcn_raw_buffer_load_b128(
                                        rpart, pu + ((db * 4 + j) * 64 + lane) * 16, 0, kSc1);
#pragma unroll
                                    for (int e = 0; e < 4; ++e)
                                        oacc[db][4 * j + e] = oacc[db][4 * j + e] * a1 + __uint_as_float(vu[e]) * a2;
                                }
                            L = L * a1 + lu * a2;
                            M = mn;
                        }
                        store_rows<D, OF32>(a, h, row, row_valid, g, oacc, M, L, c);
                    }
                }
            }
        }
        if (stream) elapsed += ie - ib;
        if (phase == 3) break;
    }
}

// Workspace of one (device, stream).  Counters and partials are separate buffers: every
// word that has ever served as a counter is zero between calls (the last arriver of a tile
// resets its counter), which would not hold if the two regions shifted between calls.
struct Workspace {
    int32_t* cnt = nullptr;
    size_t cnt_words = 0;
    float* part = nullptr;
    size_t part_floats = 0;
    int32_t* order = nullptr;  // tile kernel order (rewritten by every call that uses it)
    size_t order_words = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

template <typename X>
hipError_t grow(X*& p, size_t& have, size_t need, bool zero, hipStream_t s) {
    if (have >= need) return hipSuccess;
    hipError_t e;
    if (p) {  // the old buffer may still be in use by this stream's previous launch
        if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
        if ((e = hipFree(p)) != hipSuccess) return e;
        p = nullptr;
        have = 0;
    }
    if ((e = hipMalloc(reinterpret_cast<void**>(&p), need * sizeof(X))) != hipSuccess) return e;
    if (zero) {
        if ((e = hipMemset(p, 0, need * sizeof(X))) != hipSuccess) return e;
        if ((e = hipDeviceSynchronize()) != hipSuccess) return e;  // zeroed before any stream uses it
    }
    have = need;
    return hipSuccess;
}

hipError_t workspace_for(hipStream_t s, size_t cnt_words, size_t part_floats, int32_t** cnt, float** part) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& w = g_ws[{dev, s}];
    if ((e = grow(w.cnt, w.cnt_words, cnt_words, true, s)) != hipSuccess) return e;
    if ((e = grow(w.part, w.part_floats, part_floats, false, s)) != hipSuccess) return e;
    *cnt = w.cnt;
    *part = w.part;
    return hipSuccess;
}

struct GridInfo {
    int cus = 0;
    int per_cu[2][2][2] = {};  // unit kernel, [D == 128][QF32][OF32]
};
std::mutex g_grid_mutex;
std::map<int, GridInfo> g_grid;

template <int D, bool QF, bool OF>
hipError_t launch_unit(AttnArgs a, int n_heads_tiles, hipStream_t s) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus, per_cu;
    {
        std::lock_guard<std::mutex> lock(g_grid_mutex);
        GridInfo& gi = g_grid[dev];
        if (gi.cus == 0 &&
            (e = hipDeviceGetAttribute(&gi.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return e;
        int& pc = gi.per_cu[D == 128][QF][OF];
        if (pc == 0 && (e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, attn_unit_kernel<D, QF, OF>,
                                                                         kUnitWaves * 64, 0)) != hipSuccess)
            return e;
        cus = gi.cus;
        per_cu = pc < 1 ? 1 : pc;
    }
    const int grid = ((cus * per_cu) / 8 < 1 ? 1 : (cus * per_cu) / 8) * 8;
    if ((e = workspace_for(s, (size_t)n_heads_tiles, (size_t)2 * grid * Partial<D>::SLOT, &a.cnt, &a.part)) !=
        hipSuccess)
        return e;
    attn_unit_kernel<D, QF, OF><<<grid, kUnitWaves * 64, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t order_workspace(hipStream_t s, size_t words, int32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& w = g_ws[{dev, s}];
    if ((e = grow(w.order, w.order_words, words, false, s)) != hipSuccess) return e;
    *out = w.order;
    return hipSuccess;
}

template <int D, bool QF, bool OF>
hipError_t launch_tile(AttnArgs a, bool longest_first, hipStream_t s) {
    const unsigned blocks = (unsigned)(a.n_qtiles * a.heads);
    a.order = nullptr;
    if (longest_first) {
        int32_t* order = nullptr;
        hipError_t e = order_workspace(s, (size_t)a.n_qtiles, &order);
        if (e != hipSuccess) return e;
        tile_order_kernel<<<1, kOrderThreads, 0, s>>>(a.plan, a.n_qtiles, order);
        a.order = order;
    }
    attn_tile_kernel<D, QF, OF><<<blocks, kTileWaves * 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, bool QF, bool OF>
hipError_t launch_k(const AttnLaunch& L, const AttnArgs& a, hipStream_t s) {
    // neighbouring log-radial tiles (and tiles of dynamic plans) do not share span lists:
    // one tile per workgroup
    if (is_radial(L.mask_kind) || L.unpaired) return launch_tile<D, QF, OF>(a, L.unpaired, s);
    return launch_unit<D, QF, OF>(a, L.n_qtiles * L.heads, s);
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
    a.scale_log2 = L.scale_log2;
    if (L.head_dim == 128) return launch_d<128>(L, a, s);
    return launch_d<64>(L, a, s);
}

}  // namespace vdit
