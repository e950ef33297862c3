// Dynamic-threshold block plan ("DynamicRad: Content-Adaptive Sparse Attention for Long
// Video Diffusion", section 2, dual-mode strategy, mode 2): the pre-softmax logits of
// (query tile, key tile) pairs serve as importance proxies and an adaptive threshold keeps
// a part of the candidates the static rule of the call allows.
//
// Proxy of query tile i and key tile j (the mean logit of the tile pair, summed over heads
// so that one plan serves every head): scale * sum_h <mean of the tile's rotated queries,
// mean of the tile's rotated keys>.  Key tiles are the tile-token pieces of each cache slot.
// Kept: candidates with proxy p, p - m >= (1 - tau) (M - m), M and m the largest and
// smallest candidate proxies of the query tile.  The kept tiles become maximal runs of
// physical key indices in the usual plan words.
//
// Four launches: one that pools the queries [nq][H*D] and the keys (transposed, [H*D][nk])
// side by side, the partial proxies [nq][nk] (a small fp32 product, its channels split over
// slices), then per query tile the proxies summed, the threshold and the run count, and per
// query tile its offset (a sum over the counts before it) and its runs.
#include <algorithm>
#include <utility>

#include "vdit_bf16.hpp"
#include "vdit_internal.hpp"

namespace vdit {

namespace {

constexpr int kDynThreads = 256;
constexpr int kScoreQ = 16;    // query tiles per score workgroup
constexpr int kScoreK = 64;    // key tiles per score workgroup (one per lane)
constexpr int kScoreC = 256;   // channels of the pooled queries staged in LDS at a time
constexpr int kMaxKeyTiles = kDynMaxKeyTiles;

// The table of one channel pair p (0 .. D/2 - 1): its axis (0 = t, 1 = h, 2 = w), the
// table, its row length and the pair's column; the angle of position (t, h, w) is then
// tab[coord(axis) * pitch + col].
struct PairTab {
    const float2* tab;
    int32_t axis, pitch, col;
};
__device__ inline PairTab pair_tab(const RopeDev& r, int p) {
    if (p < r.pairs_t) return {r.tab_t, 0, r.pairs_t, p};
    if (p < r.pairs_t + r.pairs_h) return {r.tab_h, 1, r.pairs_h, p - r.pairs_t};
    return {r.tab_w, 2, r.pairs_w, p - r.pairs_t - r.pairs_h};
}
__device__ inline void rotate(float2 cs, float& x0, float& x1) {
    const float a = x0, b = x1;
    x0 = a * cs.x - b * cs.y;
    x1 = a * cs.y + b * cs.x;
}

// eight consecutive channels of one row as floats
template <bool F32>
__device__ inline void load8(const void* base, int64_t off, float (&x)[8]) {
    if constexpr (F32) {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
        x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(w[k] << 16);
            x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
}

// Column sums of a [rows][D] block held by the workgroup: thread t holds channels
// 8 (t % (D/8)) .. +7 of row group t / (D/8); returns the sum of channel t (t < D) in lane t.
template <int D>
__device__ inline float reduce_rows(float* red, const float (&acc)[8]) {
    constexpr int LPR = D / 8, RPS = kDynThreads / LPR;
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 8; ++k) red[(t / LPR) * D + (t % LPR) * 8 + k] = acc[k];
    __syncthreads();
    float sum = 0.f;
    if (t < D) {
#pragma unroll 8
        for (int r = 0; r < RPS; ++r) sum += red[r * D + t];
    }
    return sum;
}

// Mean of the rotated queries of query tile i, head h.  Each thread loads 16 or 32 bytes
// (eight channels) of a row per step; D/8 threads cover a row.
template <int D, bool QF32>
__device__ __forceinline__ void pool_q_tile(float* red, int i, PlanGeom g, const void* q, int64_t q_st, int64_t q_sh,
                                            RopeDev r, bool has_rope, int32_t width, float* qbar) {
    constexpr int LPR = D / 8, RPS = kDynThreads / LPR;
    const int h = blockIdx.y, heads = gridDim.y, t = threadIdx.x;
    const QTile qt = plan_qtile(g, i);
    const int c0 = (t % LPR) * 8;
    PairTab pt[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) pt[p] = pair_tab(r, c0 / 2 + p);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = t / LPR; k < qt.q_len; k += RPS) {
        const int row = qt.q_start + k;
        float x[8];
        load8<QF32>(q, (int64_t)row * q_st + (int64_t)h * q_sh + c0, x);
        if (has_rope) {
            const int f = row / g.hw, sp = row - f * g.hw;
            const int hh = sp / width, ww = sp - hh * width;
            const int tt = g.t0 + f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int coord = pt[p].axis == 0 ? tt : (pt[p].axis == 1 ? hh : ww);
                rotate(pt[p].tab[coord * pt[p].pitch + pt[p].col], x[2 * p], x[2 * p + 1]);
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += x[c];
    }
    const float sum = reduce_rows<D>(red, acc);
    if (t < D) qbar[((size_t)i * heads + h) * D + t] = sum * (1.f / (float)qt.q_len);
}

// Mean of the cached (rotated) keys of key tile j = slot * tiles_per_frame + piece, head h,
// written transposed: kbar_t[(h * D + d) * nk + j]; empty slots give zeros.
template <int D>
__device__ __forceinline__ void pool_k_tile(float* red, int j, PlanGeom g, const int32_t* slot_frame,
                                            const uint16_t* kc, int64_t kv_rows, int32_t nk, float* kbar_t) {
    constexpr int LPR = D / 8, RPS = kDynThreads / LPR;
    const int h = blockIdx.y, t = threadIdx.x;
    const int tpf = ceil_div(g.hw, g.tile);
    const int slot = j / tpf, s0 = (j - slot * tpf) * g.tile;
    const int len = min(g.tile, g.hw - s0);
    const int c0 = (t % LPR) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (slot_frame[slot] >= 0) {
        const int64_t row0 = (int64_t)h * kv_rows + (int64_t)slot * g.frame_stride + s0;
#pragma unroll 4
        for (int k = t / LPR; k < len; k += RPS) {
            float x[8];
            load8<false>(kc, (row0 + k) * D + c0, x);
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] += x[c];
        }
    }
    const float sum = reduce_rows<D>(red, acc);
    if (t < D) kbar_t[((size_t)h * D + t) * nk + j] = sum * (1.f / (float)len);
}

// Both poolings in one launch (they are independent): workgroups [0, nq) pool query tiles,
// [nq, nq + nk) key tiles.
template <int D, bool QF32>
__global__ __launch_bounds__(kDynThreads) void dyn_pool_kernel(PlanGeom g, const void* q, int64_t q_st, int64_t q_sh,
                                                               RopeDev r, bool has_rope, int32_t width, float* qbar,
                                                               int32_t nq, const int32_t* slot_frame,
                                                               const uint16_t* kc, int64_t kv_rows, int32_t nk,
                                                               float* kbar_t) {
    __shared__ float red[(kDynThreads / (D / 8)) * D];
    const int b = blockIdx.x;
    if (b < nq) pool_q_tile<D, QF32>(red, b, g, q, q_st, q_sh, r, has_rope, width, qbar);
    else pool_k_tile<D>(red, b - nq, g, slot_frame, kc, kv_rows, nk, kbar_t);
}

// Partial proxies over the channel range [z * cps, (z + 1) * cps) of grid slice z, for 16
// query tiles x 64 key tiles per workgroup: lane = key tile, wave = a quarter of each staged
// chunk of channels, the four wave sums added in wave order.
// part[(z * nq + i) * nk + j] = <qbar[i], kbar[j]> over the slice's channels.
__global__ __launch_bounds__(kDynThreads) void dyn_score_kernel(const float* qbar, const float* kbar_t, int32_t hd,
                                                                int32_t cps, int32_t nq, int32_t nk, float* part) {
    __shared__ float sq[kScoreC * kScoreQ];  // [channel][query tile]
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int j = blockIdx.x * kScoreK + lane, i0 = blockIdx.y * kScoreQ;
    const int c_lo = blockIdx.z * cps, c_hi = min(hd, c_lo + cps);
    const bool jv = j < nk;
    float acc[kScoreQ];
#pragma unroll
    for (int a = 0; a < kScoreQ; ++a) acc[a] = 0.f;
    for (int cb = c_lo; cb < c_hi; cb += kScoreC) {
        const int cn = min(kScoreC, c_hi - cb), per = (cn + 3) / 4;
        __syncthreads();
        for (int idx = t; idx < kScoreC * kScoreQ; idx += kDynThreads) {
            const int ii = idx / kScoreC, c = idx % kScoreC;
            sq[c * kScoreQ + ii] = (c < cn && i0 + ii < nq) ? qbar[(size_t)(i0 + ii) * hd + cb + c] : 0.f;
        }
        __syncthreads();
        const int ce = min(cn, (wave + 1) * per);
#pragma unroll 8
        for (int c = wave * per; c < ce; ++c) {
            const float kv = jv ? kbar_t[(size_t)(cb + c) * nk + j] : 0.f;
            const float4* qv = reinterpret_cast<const float4*>(sq + c * kScoreQ);
#pragma unroll
            for (int a = 0; a < kScoreQ / 4; ++a) {
                const float4 qq = qv[a];
                acc[4 * a] += qq.x * kv;
                acc[4 * a + 1] += qq.y * kv;
                acc[4 * a + 2] += qq.z * kv;
                acc[4 * a + 3] += qq.w * kv;
            }
        }
    }
    __syncthreads();
    float* red = sq;  // [wave][query tile][lane]
#pragma unroll
    for (int a = 0; a < kScoreQ; ++a) red[(wave * kScoreQ + a) * 64 + lane] = acc[a];
    __syncthreads();
    for (int idx = t; idx < kScoreQ * 64; idx += kDynThreads) {
        const int a = idx / 64, l = idx % 64;
        const int i = i0 + a, jj = blockIdx.x * kScoreK + l;
        if (i >= nq || jj >= nk) continue;
        float v = red[a * 64 + l];
#pragma unroll
        for (int w = 1; w < 4; ++w) v += red[(w * kScoreQ + a) * 64 + l];
        part[((size_t)blockIdx.z * nq + i) * nk + jj] = v;
    }
}

// Key tile j of the cache: physical start and length, and whether query tile qt may see it
// under the static rule (the rule's ranges are whole tiles or whole frames).
struct KeyTile {
    int32_t start, len;
    bool cand;
};
__device__ inline KeyTile key_tile(const PlanGeom& g, const int32_t* sf, const QTile& qt, int32_t j) {
    const int tpf = ceil_div(g.hw, g.tile);
    const int slot = j / tpf, s0 = (j - slot * tpf) * g.tile, e = min(s0 + g.tile, g.hw);
    int32_t a, b;
    const bool vis = plan_slot_range(g, qt, sf[slot], &a, &b) && s0 >= a && e <= b;
    return {slot * g.frame_stride + s0, e - s0, vis};
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ inline float wave_min(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off));
    return v;
}
template <class T>
__device__ inline T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Kept flags of query tile i into s_keep[nk] (0 / 1) and the flags of run starts and run
// ends (a kept tile not physically continued by its kept neighbour) into s_start / s_end.
// Returns, in every thread, the number of runs and of kept keys.  s_red: 16 words of LDS.
__device__ inline void kept_runs(const PlanGeom& g, const int32_t* sf, const QTile& qt, const float* prow,
                                 int32_t nk, float keep_frac, uint8_t* s_keep, float* s_red, int32_t* runs,
                                 int32_t* keys) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float big = -INFINITY, small = INFINITY;
    for (int j = t; j < nk; j += kDynThreads) {
        const KeyTile kt = key_tile(g, sf, qt, j);
        if (kt.cand) {
            const float p = prow[j];
            big = fmaxf(big, p);
            small = fminf(small, p);
        }
    }
    big = wave_max(big);
    small = wave_min(small);
    if (lane == 0) {
        s_red[wave] = big;
        s_red[4 + wave] = small;
    }
    __syncthreads();
    big = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    small = fminf(fminf(s_red[4], s_red[5]), fminf(s_red[6], s_red[7]));
    const float cut = keep_frac * (big - small);
    for (int j = t; j < nk; j += kDynThreads) {
        const KeyTile kt = key_tile(g, sf, qt, j);
        s_keep[j] = kt.cand && (prow[j] - small >= cut);
    }
    __syncthreads();
    int32_t nr = 0, nkeys = 0;
    for (int j = t; j < nk; j += kDynThreads) {
        if (!s_keep[j]) continue;
        const KeyTile kt = key_tile(g, sf, qt, j);
        nkeys += kt.len;
        bool joined = false;
        if (j > 0 && s_keep[j - 1]) {
            const KeyTile pv = key_tile(g, sf, qt, j - 1);
            joined = pv.start + pv.len == kt.start;
        }
        nr += !joined;
    }
    nr = wave_sum(nr);
    nkeys = wave_sum(nkeys);
    __syncthreads();
    if (lane == 0) {
        reinterpret_cast<int32_t*>(s_red)[8 + wave] = nr;
        reinterpret_cast<int32_t*>(s_red)[12 + wave] = nkeys;
    }
    __syncthreads();
    const int32_t* si = reinterpret_cast<const int32_t*>(s_red);
    *runs = si[8] + si[9] + si[10] + si[11];
    *keys = si[12] + si[13] + si[14] + si[15];
}

// Pass 1, one workgroup per query tile: its proxies (the partial sums of the channel
// slices added in slice order, times the scale), the number of runs and of (query, key) pairs.
__global__ __launch_bounds__(kDynThreads) void dyn_count_kernel(PlanGeom g, const int32_t* slot_frame,
                                                                const float* part, int32_t slices, int32_t nq,
                                                                int32_t nk, float scale, float keep_frac,
                                                                float* prox, int32_t* n_runs, long long* n_pairs) {
    __shared__ float s_p[kMaxKeyTiles];
    __shared__ uint8_t s_keep[kMaxKeyTiles];
    __shared__ float s_red[16];
    const int i = blockIdx.x;
    const QTile qt = plan_qtile(g, i);
    for (int j = threadIdx.x; j < nk; j += kDynThreads) {
        float v = part[(size_t)i * nk + j];
        for (int z = 1; z < slices; ++z) v += part[((size_t)z * nq + i) * nk + j];
        v *= scale;
        s_p[j] = v;
        prox[(size_t)i * nk + j] = v;
    }
    __syncthreads();
    int32_t runs, keys;
    kept_runs(g, slot_frame, qt, s_p, nk, keep_frac, s_keep, s_red, &runs, &keys);
    if (threadIdx.x == 0) {
        n_runs[i] = runs;
        n_pairs[i] = (long long)keys * qt.q_len;
    }
}

// Sum of v[0 .. n) over the workgroup, in every thread.
template <class T>
__device__ inline T block_sum(const T* v, int32_t n, T* s_part) {
    T acc = 0;
    for (int k = threadIdx.x; k < n; k += kDynThreads) acc += v[k];
    acc = wave_sum(acc);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
    __syncthreads();
    return s_part[0] + s_part[1] + s_part[2] + s_part[3];
}

// Pass 2, one workgroup per query tile: its offset (runs of the tiles before it), its
// query tile, row pointer and runs; workgroup 0 also writes the header.
__global__ __launch_bounds__(kDynThreads) void dyn_write_kernel(PlanGeom g, const int32_t* slot_frame,
                                                                const float* prox, int32_t nk, float keep_frac,
                                                                int32_t nq, const int32_t* n_runs,
                                                                const long long* n_pairs, int32_t* plan) {
    __shared__ float s_p[kMaxKeyTiles];
    __shared__ uint8_t s_keep[kMaxKeyTiles];
    __shared__ int32_t s_first[kMaxKeyTiles];  // physical start of each run of this tile
    __shared__ float s_red[16];
    __shared__ int32_t s_scan[kDynThreads];
    __shared__ long long s_ll[4];
    const int i = blockIdx.x, t = threadIdx.x;
    int32_t* qtiles = plan + VDIT_PLAN_HEADER_WORDS;
    int32_t* row_ptr = qtiles + 2 * nq;
    int32_t* spans = row_ptr + nq + 1;
    const QTile qt = plan_qtile(g, i);
    const int32_t offset = block_sum(n_runs, i, reinterpret_cast<int32_t*>(s_red));
    if (i == 0) {
        const int32_t total = block_sum(n_runs, nq, reinterpret_cast<int32_t*>(s_red));
        const long long pairs = block_sum(n_pairs, nq, s_ll);
        if (t == 0) {
            const unsigned long long tot = (unsigned long long)pairs;
            row_ptr[0] = 0;
            plan[0] = (int32_t)VDIT_PLAN_MAGIC;
            plan[1] = VDIT_PLAN_VERSION;
            plan[2] = g.kind | VDIT_MASK_FLAG_DYNAMIC;
            plan[3] = g.tile;
            plan[4] = nq;
            plan[5] = total;
            plan[6] = (int32_t)(uint32_t)(tot & 0xFFFFFFFFull);
            plan[7] = (int32_t)(uint32_t)(tot >> 32);
            plan_set_call(plan, g);
        }
    }
    for (int j = t; j < nk; j += kDynThreads) s_p[j] = prox[(size_t)i * nk + j];
    __syncthreads();
    int32_t runs, keys;
    kept_runs(g, slot_frame, qt, s_p, nk, keep_frac, s_keep, s_red, &runs, &keys);
    if (t == 0) {
        qtiles[2 * i] = qt.q_start;
        qtiles[2 * i + 1] = qt.q_len;
        row_ptr[i + 1] = offset + runs;
    }
    // thread t owns key tiles [t * per, (t + 1) * per): its run starts, scanned over threads
    const int per = ceil_div(nk, kDynThreads), j0 = t * per, j1 = min(j0 + per, nk);
    auto starts_run = [&](int j, KeyTile& kt) {
        if (!s_keep[j]) return false;
        kt = key_tile(g, slot_frame, qt, j);
        if (j == 0 || !s_keep[j - 1]) return true;
        const KeyTile pv = key_tile(g, slot_frame, qt, j - 1);
        return pv.start + pv.len != kt.start;
    };
    int32_t mine = 0;
    for (int j = j0; j < j1; ++j) {
        KeyTile kt;
        mine += starts_run(j, kt);
    }
    s_scan[t] = mine;
    __syncthreads();
    for (int off = 1; off < kDynThreads; off <<= 1) {
        const int32_t v = t >= off ? s_scan[t - off] : 0;
        __syncthreads();
        s_scan[t] += v;
        __syncthreads();
    }
    int32_t r = s_scan[t] - mine;  // runs that start before j0
    for (int j = j0; j < j1; ++j) {
        KeyTile kt;
        if (starts_run(j, kt)) s_first[r++] = kt.start;
    }
    __syncthreads();
    // the end of run k is the k-th kept tile not continued by its kept successor
    r = s_scan[t] - mine;
    for (int j = j0; j < j1; ++j) {
        KeyTile kt;
        if (starts_run(j, kt)) ++r;  // the run that holds j is run r - 1
        if (!s_keep[j]) continue;
        kt = key_tile(g, slot_frame, qt, j);
        bool cont = false;
        if (j + 1 < nk && s_keep[j + 1]) {
            const KeyTile nx = key_tile(g, slot_frame, qt, j + 1);
            cont = kt.start + kt.len == nx.start;
        }
        if (!cont) {
            const int32_t k = r - 1, first = s_first[k];
            spans[2 * (offset + k)] = first;
            spans[2 * (offset + k) + 1] = kt.start + kt.len - first;
        }
    }
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Partial proxies are kept under this many bytes: the channels are split over as many
// slices (whole heads) as fit, at most one per head.
constexpr size_t kPartBytes = size_t(64) << 20;

// Sizes of the workspace regions: pooled queries, pooled keys (transposed), partial proxies,
// proxies (when the caller does not take them), run and pair counts per query tile.
struct DynSizes {
    int32_t cps, slices;
    size_t qbar, kbar, part, prox, runs, pairs;
    size_t total() const { return qbar + kbar + part + prox + runs + pairs; }
};

DynSizes dyn_sizes(const PlanGeom& g, int32_t nq, int32_t heads, int32_t head_dim) {
    const int32_t hd = heads * head_dim;
    const int32_t nk = g.capacity * ceil_div(g.hw, g.tile);
    const size_t one = (size_t)nq * nk * 4;
    const int32_t want = (int32_t)std::max<size_t>(1, std::min<size_t>((size_t)heads, kPartBytes / one));
    DynSizes z;
    z.cps = ceil_div(heads, want) * head_dim;
    z.slices = ceil_div(hd, z.cps);
    z.qbar = align256((size_t)nq * hd * 4);
    z.kbar = align256((size_t)hd * nk * 4);
    z.part = align256(one * z.slices);
    z.prox = align256(one);
    z.runs = align256((size_t)nq * 4);
    z.pairs = align256((size_t)nq * 8);
    return z;
}

template <int D>
hipError_t launch_dyn_d(const DynLaunch& L, hipStream_t s) {
    const PlanGeom& g = L.geom;
    const int32_t nq = L.n_qtiles, heads = L.heads, hd = heads * D;
    const int32_t nk = g.capacity * ceil_div(g.hw, g.tile);
    const DynSizes z = dyn_sizes(g, nq, heads, D);
    const int32_t cps = z.cps, slices = z.slices;
    const size_t b_qbar = z.qbar, b_kbar = z.kbar, b_part = z.part, b_prox = z.prox, b_runs = z.runs,
                 b_pairs = z.pairs;
    char* ws = static_cast<char*>(L.workspace);
    char* at = ws;
    auto take = [&](size_t b) {
        char* p = at;
        at += b;
        return p;
    };
    float* qbar = reinterpret_cast<float*>(take(b_qbar));
    float* kbar_t = reinterpret_cast<float*>(take(b_kbar));
    float* part = reinterpret_cast<float*>(take(b_part));
    float* prox = reinterpret_cast<float*>(take(b_prox));
    if (L.proxies) prox = L.proxies;
    int32_t* runs = reinterpret_cast<int32_t*>(take(b_runs));
    long long* pairs = reinterpret_cast<long long*>(take(b_pairs));
    const uint16_t* kc = static_cast<const uint16_t*>(L.kc);
    if (L.q.dtype == VDIT_DTYPE_FP32)
        dyn_pool_kernel<D, true><<<dim3(nq + nk, heads), kDynThreads, 0, s>>>(
            g, L.q.data, L.q.stride_token, L.q.stride_head, L.rope, L.has_rope, L.width, qbar, nq, L.slot_frame, kc,
            L.kv_rows, nk, kbar_t);
    else
        dyn_pool_kernel<D, false><<<dim3(nq + nk, heads), kDynThreads, 0, s>>>(
            g, L.q.data, L.q.stride_token, L.q.stride_head, L.rope, L.has_rope, L.width, qbar, nq, L.slot_frame, kc,
            L.kv_rows, nk, kbar_t);
    dyn_score_kernel<<<dim3(ceil_div(nk, kScoreK), ceil_div(nq, kScoreQ), slices), kDynThreads, 0, s>>>(
        qbar, kbar_t, hd, cps, nq, nk, part);
    dyn_count_kernel<<<nq, kDynThreads, 0, s>>>(g, L.slot_frame, part, slices, nq, nk, L.scale, L.keep_frac, prox,
                                                runs, pairs);
    dyn_write_kernel<<<nq, kDynThreads, 0, s>>>(g, L.slot_frame, prox, nk, L.keep_frac, nq, runs, pairs, L.plan);
    return hipGetLastError();
}

}  // namespace

size_t dyn_workspace_bytes(const PlanGeom& g, int32_t n_qtiles, int32_t heads, int32_t head_dim) {
    return dyn_sizes(g, n_qtiles, heads, head_dim).total();
}

hipError_t launch_plan_dynamic(const DynLaunch& L, hipStream_t s) {
    if (L.head_dim == 128) return launch_dyn_d<128>(L, s);
    return launch_dyn_d<64>(L, s);
}

}  // namespace vdit
