// Block-sparse flash-attention forward for CDNA4 (gfx950), bf16 MFMA with fp32 online
// softmax.  One workgroup = one (query tile of <= 128 rows, head); 4 waves of 32 query
// rows each.  The key loop walks the plan's spans in tiles of 64 keys; K and V^T tiles are
// double-buffered in LDS, the next tile's global loads are in flight while the current
// tile is computed.  Keys outside the spans are never loaded.
//
// Math per key tile (FlashAttention-style online softmax, exact up to rounding): the
// scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so every
// lane owns one query row and the row max / sum are in-lane except one exchange between
// the two 32-lane halves; O^T += V^T P^T keeps the output in the same lane-per-row layout,
// so the rescale by exp(m_old - m_new) is a per-lane scalar.  The key order inside an
// MFMA is chosen (bits 2 and 3 of the S row index swapped) so that the bf16 P operand is
// taken from the S accumulator registers as they are and V^T is read from LDS with one
// 16-byte read per lane.
#include <type_traits>

#include "vdit_bf16.hpp"
#include "vdit_internal.hpp"

namespace vdit {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 128;  // query rows per workgroup (= plan tile)
constexpr int kBN = 64;   // keys per iteration

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
template <int D>
struct Tile {
    static constexpr int KCH = D / 8;    // 16-byte chunks per K row
    static constexpr int VCH = kBN / 8;  // 16-byte chunks per V^T row
    static constexpr int K_BYTES = kBN * D * 2;
    static constexpr int V_BYTES = D * kBN * 2;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int K_LOADS = kBN * KCH / kThreads;  // direct loads per thread
    static constexpr int V_LOADS = D * VCH / kThreads;
};

template <int CH>
__device__ inline int swz(int r) {
    return CH == 16 ? (r & 15) : ((r >> 1) & 7);
}

// Per-lane constants of the tile DMA.  Load i of wave w fills 1 KB block b = 4 i + w of a
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
    // swz(b * RPB + rib) with b = 4 i + wave
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
template <int D>
__device__ inline void load_tile_lds(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t vpitch, int k0,
                                     int kend, int wave, const DmaLane<D / 8>& kl, const DmaLane<kBN / 8>& vl,
                                     char* stage) {
    using T = Tile<D>;
    constexpr int KRPB = 64 / T::KCH, VRPB = 64 / T::VCH;
    // every address stays inside the span: scalar offset = tile start k0 (< kend), the lane's
    // row delta is clamped to kend - 1 - k0 >= 0
    const int last = kend - 1 - k0;
#pragma unroll
    for (int i = 0; i < T::K_LOADS; ++i) {
        const int blk = i * kWaves + wave;
        const int rowd = min(blk * KRPB + kl.rib, last);
        const uint32_t voff = (uint32_t)rowd * (D * 2) + kl.chunk * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(stage + blk * 1024), 16, voff,
                                                 (uint32_t)k0 * (D * 2), 0, 0);
    }
    const int vkey = min(k0 + vl.chunk * 8, (kend - 1) & ~7);  // >= k0: k0 is a multiple of 8
    const uint32_t vcol = (uint32_t)(vkey - k0) * 2;
#pragma unroll
    for (int i = 0; i < T::V_LOADS; ++i) {
        const int blk = i * kWaves + wave;
        const uint32_t voff = (uint32_t)vl.rib * vpitch + vcol;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(stage + T::K_BYTES + blk * 1024), 16, voff,
                                                 (uint32_t)(blk * VRPB) * vpitch + (uint32_t)k0 * 2, 0, 0);
    }
}

__device__ inline void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Logical work item of this workgroup.  Workgroups are dispatched round-robin over the
// 8 XCDs; renumber so that each XCD gets a contiguous range of (head, query tile) items,
// i.e. mostly one head, whose K/V then stream through that XCD's L2 once.
__device__ inline int xcd_remap(int bid, int total) {
    constexpr int kXcd = 8;
    int q = total / kXcd, r = total % kXcd;
    int xcd = bid % kXcd, idx = bid / kXcd;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

template <int D, bool QF32, bool OF32>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs a) {
    using T = Tile<D>;
    constexpr int KS = D / 16;  // k-steps of the QK^T contraction
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qi = lane & 31, g = lane >> 5;

    const int item = xcd_remap(blockIdx.x, a.n_qtiles * a.heads);
    const int h = item / a.n_qtiles, qt = item % a.n_qtiles;

    const int32_t* plan = a.plan;
    const int nq = plan[4];
    // a plan that does not belong to this call is ignored rather than read out of bounds
    if (plan[0] != (int32_t)VDIT_PLAN_MAGIC || nq != a.n_qtiles || qt >= nq) return;
    const int32_t* qtiles = plan + VDIT_PLAN_HEADER_WORDS;
    const int32_t* row_ptr = qtiles + 2 * nq;
    const int32_t* spans = row_ptr + nq + 1;
    const int q_start = qtiles[2 * qt], q_len = qtiles[2 * qt + 1];
    const int sp_begin = row_ptr[qt], sp_end = row_ptr[qt + 1];
    if (q_start < 0 || q_len < 1 || q_len > kBM || q_start + q_len > a.n_tokens || sp_begin > sp_end ||
        sp_end > plan[5])
        return;
    for (int sp = sp_begin; sp < sp_end; ++sp) {  // spans must lie inside the cache, 8-aligned
        const int k0 = spans[2 * sp], kl = spans[2 * sp + 1];
        if (k0 < 0 || (k0 & 7) || kl < 1 || (int64_t)k0 + kl > a.kv_rows) return;
    }

    // ---- Q tile: this lane's row, RoPE at the global position while loading.
    const int r_in = wave * 32 + qi;
    const bool row_valid = r_in < q_len;
    const int row = q_start + (row_valid ? r_in : q_len - 1);
    bf16x8 qreg[KS];
    {
        const int f = row / a.hw, s = row % a.hw;
        const int pt = a.t0 + f, ph = s / a.wf, pw = s % a.wf;
        const int64_t qoff = (int64_t)row * a.q_st + (int64_t)h * a.q_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = ks * 16 + g * 8;
            float x[8];
            if constexpr (QF32) {
                const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qoff + d0);
                float4 u = p[0], v = p[1];
                x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
                x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
            } else {
                unpack_bf16x8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qoff + d0), x);
            }
            if (a.has_rope) rope_rotate8(a.rope, d0 / 2, pt, ph, pw, x);
            qreg[ks] = __builtin_bit_cast(bf16x8, pack_bf16x8(x));
        }
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    // Running max of the raw scores used as the exponent base.  It is only raised when a
    // tile's max exceeds it by more than kLazy (in log2 units), so most tiles skip the
    // rescale of O; p = exp2((s - m) * c) then stays below 2^kLazy.
    constexpr float kLazy = 8.0f;
    const float c = a.scale_log2;
    const float lazy_raw = kLazy / c;
    float m_run = -INFINITY, l_run = 0.f;

    if (sp_begin < sp_end) {
        int span = sp_begin;
        int k0 = spans[2 * span], kend = k0 + spans[2 * span + 1];
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        const DmaLane<D / 8> kl = dma_lane<D / 8>(wave_u, lane);
        const DmaLane<kBN / 8> vl = dma_lane<kBN / 8>(wave_u, lane);
        const uint32_t head_bytes = (uint32_t)(a.kv_rows * D * 2);
        const __amdgpu_buffer_rsrc_t rk = head_rsrc(a.kc + (int64_t)h * a.kv_rows * D, head_bytes);
        const __amdgpu_buffer_rsrc_t rv = head_rsrc(a.vt + (int64_t)h * D * a.kv_rows, head_bytes);
        const uint32_t vpitch = (uint32_t)(a.kv_rows * 2);
        load_tile_lds<D>(rk, rv, vpitch, k0, kend, wave_u, kl, vl, smem);
        wait_tile_loads();
        __syncthreads();
        int buf = 0;
        // per-lane fragment addresses (bytes inside a stage)
        const int krow = swap23(qi);  // S row qi holds key krow of each 32-key block
        const int kswz = swz<T::KCH>(krow);
        const int vswz = swz<T::VCH>(qi);

        auto body = [&]() {
            const char* kst = smem + buf * T::STAGE;
            const char* vst = kst + T::K_BYTES;
            auto read_k = [&](int ks, int kb) {
                return *reinterpret_cast<const bf16x8*>(kst + (kb * 32 + krow) * (T::KCH * 16) +
                                                        (((2 * ks + g) ^ kswz) * 16));
            };
            auto read_v = [&](int j, int db) {
                return *reinterpret_cast<const bf16x8*>(vst + (db * 32 + qi) * (T::VCH * 16) +
                                                        (((2 * j + g) ^ vswz) * 16));
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
            mt = fmaxf(mt, __shfl_xor(mt, 32));
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
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = fast_exp2(__builtin_fmaf(sacc[j >> 1][(j & 1) * 8 + e], c, mc));
                    l_run += p[e];
                }
                pk[j] = __builtin_bit_cast(bf16x8, pack_bf16x8(p));
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
        };

        while (true) {
            int nk0 = k0 + kBN, nkend = kend, nspan = span;
            if (nk0 >= kend) {
                ++nspan;
                if (nspan < sp_end) {
                    nk0 = spans[2 * nspan];
                    nkend = nk0 + spans[2 * nspan + 1];
                }
            }
            const bool has_next = nspan < sp_end;
            if (has_next) load_tile_lds<D>(rk, rv, vpitch, nk0, nkend, wave_u, kl, vl, smem + (buf ^ 1) * T::STAGE);
            body();
            if (!has_next) break;
            wait_tile_loads();
            __syncthreads();
            buf ^= 1;
            k0 = nk0;
            kend = nkend;
            span = nspan;
        }
    }

    // ---- epilogue: O = O^T / l, LSE
    const float l = l_run + __shfl_xor(l_run, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_valid) {
        const int64_t ooff = (int64_t)row * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
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
            a.lse[(int64_t)h * a.n_tokens + row] =
                l > 0.f ? (m_run * c + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
}

template <int D>
hipError_t launch_d(const AttnLaunch& L, const AttnArgs& a, hipStream_t s) {
    unsigned blocks = (unsigned)(L.n_qtiles * L.heads);
    bool qf = L.q.dtype == VDIT_DTYPE_FP32, of = L.o.dtype == VDIT_DTYPE_FP32;
    if (qf && of) attn_fwd_kernel<D, true, true><<<blocks, kThreads, 0, s>>>(a);
    else if (qf) attn_fwd_kernel<D, true, false><<<blocks, kThreads, 0, s>>>(a);
    else if (of) attn_fwd_kernel<D, false, true><<<blocks, kThreads, 0, s>>>(a);
    else attn_fwd_kernel<D, false, false><<<blocks, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnLaunch& L, hipStream_t s) {
    AttnArgs a;
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
