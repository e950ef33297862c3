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

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// swap bits 2 and 3
__device__ inline int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D>
struct Tile {
    static constexpr int KP = D + 8;    // LDS pitch of a K row (elements)
    static constexpr int VP = kBN + 8;  // LDS pitch of a V^T row
    static constexpr int K_ELEMS = kBN * KP;
    static constexpr int V_ELEMS = D * VP;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int K_LOADS = kBN * D / 8 / kThreads;  // 16-byte loads per thread
    static constexpr int V_LOADS = D * kBN / 8 / kThreads;
};

template <int D>
__device__ inline void load_tile(const AttnArgs& a, int h, int k0, int kend, int tid, u32x4* kr, u32x4* vr) {
    using T = Tile<D>;
    const uint16_t* kbase = a.kc + (int64_t)h * a.kv_rows * D;
#pragma unroll
    for (int r = 0; r < T::K_LOADS; ++r) {
        int c = tid + kThreads * r;
        int row = c / (D / 8), col = c % (D / 8);
        int key = k0 + row;
        key = key < kend ? key : kend - 1;
        kr[r] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * D + col * 8);
    }
    const uint16_t* vbase = a.vt + (int64_t)h * D * a.kv_rows;
#pragma unroll
    for (int r = 0; r < T::V_LOADS; ++r) {
        int c = tid + kThreads * r;
        int drow = c / (kBN / 8), col = c % (kBN / 8);
        int key = k0 + col * 8;
        key = key < kend ? key : ((kend - 1) & ~7);
        vr[r] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)drow * a.kv_rows + key);
    }
}

template <int D>
__device__ inline void store_tile(uint16_t* stage, int tid, const u32x4* kr, const u32x4* vr) {
    using T = Tile<D>;
#pragma unroll
    for (int r = 0; r < T::K_LOADS; ++r) {
        int c = tid + kThreads * r;
        int row = c / (D / 8), col = c % (D / 8);
        *reinterpret_cast<u32x4*>(stage + row * T::KP + col * 8) = kr[r];
    }
    uint16_t* vs = stage + T::K_ELEMS;
#pragma unroll
    for (int r = 0; r < T::V_LOADS; ++r) {
        int c = tid + kThreads * r;
        int drow = c / (kBN / 8), col = c % (kBN / 8);
        *reinterpret_cast<u32x4*>(vs + drow * T::VP + col * 8) = vr[r];
    }
}

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
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];

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
    float m_run = -1e30f, l_run = 0.f;

    if (sp_begin < sp_end) {
        int span = sp_begin;
        int k0 = spans[2 * span], kend = k0 + spans[2 * span + 1];
        u32x4 kr[T::K_LOADS], vr[T::V_LOADS];
        load_tile<D>(a, h, k0, kend, tid, kr, vr);
        store_tile<D>(smem, tid, kr, vr);
        __syncthreads();
        int buf = 0;
        const int krow_lane = swap23(qi);
        while (true) {
            // next tile
            int nk0 = k0 + kBN, nkend = kend, nspan = span;
            if (nk0 >= kend) {
                ++nspan;
                if (nspan < sp_end) {
                    nk0 = spans[2 * nspan];
                    nkend = nk0 + spans[2 * nspan + 1];
                }
            }
            const bool has_next = nspan < sp_end;
            if (has_next) load_tile<D>(a, h, nk0, nkend, tid, kr, vr);

            const uint16_t* ks_lds = smem + buf * T::STAGE;
            const uint16_t* vs_lds = ks_lds + T::K_ELEMS;
            // S^T = K Q^T for 2 blocks of 32 keys
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x16{};
                const uint16_t* kp = ks_lds + (kb * 32 + krow_lane) * T::KP + g * 8;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    bf16x8 kv = *reinterpret_cast<const bf16x8*>(kp + ks * 16);
                    sacc[kb] = mfma32(kv, qreg[ks], sacc[kb]);
                }
            }
            // online softmax (log2 domain)
            float mt = -INFINITY;
            const bool tail = k0 + kBN > kend;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = sacc[kb][r] * a.scale_log2;
                    if (tail) {
                        int key = k0 + kb * 32 + (r >> 3) * 16 + g * 8 + (r & 7);
                        x = key < kend ? x : -INFINITY;
                    }
                    sacc[kb][r] = x;
                    mt = fmaxf(mt, x);
                }
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            float rs = 0.f;
            bf16x8 pk[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        p[e] = fast_exp2(sacc[kb][hh * 8 + e] - m_new);
                        rs += p[e];
                    }
                    pk[kb][hh] = __builtin_bit_cast(bf16x8, pack_bf16x8(p));
                }
            }
            l_run = l_run * alpha + rs;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t* vp = vs_lds + (db * 32 + qi) * T::VP + g * 8;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        bf16x8 vv = *reinterpret_cast<const bf16x8*>(vp + kb * 32 + hh * 16);
                        oacc[db] = mfma32(vv, pk[kb][hh], oacc[db]);
                    }
                }
            }
            if (!has_next) break;
            store_tile<D>(smem + (buf ^ 1) * T::STAGE, tid, kr, vr);
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
            a.lse[(int64_t)h * a.n_tokens + row] = l > 0.f ? (m_run + __log2f(l)) * 0.69314718055994531f : -INFINITY;
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
