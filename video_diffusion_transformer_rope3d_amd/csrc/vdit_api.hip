// Host side of the C ABI: argument validation, RoPE tables, the host plan builder and
// kernel launches.  See include/vdit.h for the contract of every entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "vdit_internal.hpp"

using namespace vdit;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return VDIT_OK;
}

int device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(VDIT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

int check_grid(const vdit_grid& g) {
    if (g.frames < 0 || g.height <= 0 || g.width <= 0)
        return fail(VDIT_ERR_INVALID_ARG, "grid (%d, %d, %d): frames must be >= 0, height and width > 0", g.frames,
                    g.height, g.width);
    if ((int64_t)g.frames * g.height * g.width > INT32_MAX)
        return fail(VDIT_ERR_INVALID_ARG, "grid has more than 2^31-1 tokens");
    return VDIT_OK;
}

int check_rope_dims(const vdit_rope_cfg* r) {
    if (!r) return fail(VDIT_ERR_INVALID_ARG, "rope cfg is NULL");
    if (r->dim_t < 0 || r->dim_h < 0 || r->dim_w < 0 || (r->dim_t & 1) || (r->dim_h & 1) || (r->dim_w & 1))
        return fail(VDIT_ERR_INVALID_ARG, "rope widths (%d, %d, %d) must be even and >= 0", r->dim_t, r->dim_h,
                    r->dim_w);
    if (r->dim_t + r->dim_h + r->dim_w != r->head_dim)
        return fail(VDIT_ERR_INVALID_ARG, "rope widths %d + %d + %d != head_dim %d", r->dim_t, r->dim_h, r->dim_w,
                    r->head_dim);
    if (!(r->theta > 0.0)) return fail(VDIT_ERR_INVALID_ARG, "rope theta must be > 0");
    if (r->max_t <= 0 || r->max_h <= 0 || r->max_w <= 0)
        return fail(VDIT_ERR_INVALID_ARG, "rope table rows (%d, %d, %d) must be > 0", r->max_t, r->max_h, r->max_w);
    if (r->reserved != 0) return fail(VDIT_ERR_INVALID_ARG, "rope cfg reserved field must be 0");
    return VDIT_OK;
}

// Rope cfg usable by a kernel: dims valid, device table present, positions covered.
int check_rope_use(const vdit_rope_cfg* r, int32_t head_dim, const vdit_grid& g, int32_t t0) {
    int st = check_rope_dims(r);
    if (st) return st;
    if (r->head_dim != head_dim)
        return fail(VDIT_ERR_INVALID_ARG, "rope head_dim %d != tensor head_dim %d", r->head_dim, head_dim);
    if (!r->table) return fail(VDIT_ERR_INVALID_ARG, "rope cfg has no device table");
    if ((int64_t)t0 + g.frames > r->max_t)
        return fail(VDIT_ERR_INVALID_ARG, "global frames up to %lld exceed the rope table (%d rows)",
                    (long long)t0 + g.frames - 1, r->max_t);
    if (g.height > r->max_h || g.width > r->max_w)
        return fail(VDIT_ERR_INVALID_ARG, "grid %dx%d exceeds the rope table (%d x %d)", g.height, g.width, r->max_h,
                    r->max_w);
    return VDIT_OK;
}

RopeDev rope_dev(const vdit_rope_cfg* r) {
    RopeDev d;
    const float* p = r->table;
    d.pairs_t = r->dim_t / 2;
    d.pairs_h = r->dim_h / 2;
    d.pairs_w = r->dim_w / 2;
    d.tab_t = reinterpret_cast<const float2*>(p);
    d.tab_h = reinterpret_cast<const float2*>(p + (size_t)r->max_t * r->dim_t);
    d.tab_w = reinterpret_cast<const float2*>(p + (size_t)r->max_t * r->dim_t + (size_t)r->max_h * r->dim_h);
    return d;
}

int check_tensor(const vdit_tensor& x, const char* name, int32_t n_tokens, int32_t heads, int32_t head_dim) {
    if (!x.data) return fail(VDIT_ERR_INVALID_ARG, "%s: data is NULL", name);
    if (x.dtype != VDIT_DTYPE_BF16 && x.dtype != VDIT_DTYPE_FP32)
        return fail(VDIT_ERR_UNSUPPORTED, "%s: dtype %d is not bf16 or fp32", name, x.dtype);
    if (x.reserved != 0) return fail(VDIT_ERR_INVALID_ARG, "%s: reserved field must be 0", name);
    int64_t align = x.dtype == VDIT_DTYPE_BF16 ? 8 : 4;
    if (((uintptr_t)x.data & 15) != 0) return fail(VDIT_ERR_INVALID_ARG, "%s: base pointer not 16-byte aligned", name);
    if (x.stride_token % align || x.stride_head % align)
        return fail(VDIT_ERR_INVALID_ARG, "%s: strides must be multiples of %lld elements", name, (long long)align);
    if (x.stride_token < 0 || x.stride_head < 0) return fail(VDIT_ERR_INVALID_ARG, "%s: negative stride", name);
    if (heads > 1 && x.stride_head < head_dim)
        return fail(VDIT_ERR_INVALID_ARG, "%s: head stride %lld < head_dim %d", name, (long long)x.stride_head,
                    head_dim);
    if (n_tokens > 1 && x.stride_token < head_dim)
        return fail(VDIT_ERR_INVALID_ARG, "%s: token stride %lld < head_dim %d", name, (long long)x.stride_token,
                    head_dim);
    return VDIT_OK;
}

int check_cache(const vdit_kv_cache* c) {
    if (!c) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (c->capacity <= 0 || c->tokens_per_frame <= 0 || c->heads <= 0)
        return fail(VDIT_ERR_INVALID_ARG, "cache capacity %d, tokens_per_frame %d, heads %d must be > 0",
                    c->capacity, c->tokens_per_frame, c->heads);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(VDIT_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", c->head_dim);
    // one head's K (or V^T) slice is addressed with 32-bit buffer offsets
    if ((int64_t)c->capacity * frame_stride_of(c->tokens_per_frame) * c->head_dim * 2 > INT32_MAX)
        return fail(VDIT_ERR_UNSUPPORTED, "one head of the cache exceeds 2 GiB");
    return VDIT_OK;
}

int check_mask(const vdit_mask_cfg* m) {
    if (!m) return fail(VDIT_ERR_INVALID_ARG, "mask cfg is NULL");
    if (m->kind != VDIT_MASK_DENSE && m->kind != VDIT_MASK_CHUNK_CAUSAL && !is_radial(m->kind))
        return fail(VDIT_ERR_INVALID_ARG, "mask kind %d", m->kind);
    if (m->tile != 128) return fail(VDIT_ERR_UNSUPPORTED, "mask tile %d (supported: 128)", m->tile);
    if ((m->kind == VDIT_MASK_CHUNK_CAUSAL || m->kind == VDIT_MASK_LOG_RADIAL_CAUSAL) && m->chunk_frames < 1)
        return fail(VDIT_ERR_INVALID_ARG, "chunk_frames %d must be >= 1", m->chunk_frames);
    if (is_radial(m->kind) &&
        (m->radial_w0 < 0 || m->radial_decay_log2 < 0 || m->long_range_period < 0))
        return fail(VDIT_ERR_INVALID_ARG, "log-radial parameters must be >= 0");
    return VDIT_OK;
}

PlanGeom make_geom(const vdit_mask_cfg* m, const vdit_grid& g, int32_t t0, const vdit_kv_cache* c) {
    PlanGeom pg;
    pg.kind = m->kind;
    pg.chunk_frames =
        m->kind == VDIT_MASK_CHUNK_CAUSAL || m->kind == VDIT_MASK_LOG_RADIAL_CAUSAL ? m->chunk_frames : 1;
    pg.tile = m->tile;
    pg.w0 = m->radial_w0;
    pg.decay_log2 = m->radial_decay_log2;
    pg.period = m->long_range_period;
    pg.frames = g.frames;
    pg.hw = g.height * g.width;
    pg.t0 = t0;
    pg.capacity = c ? c->capacity : 0;
    pg.frame_stride = c ? frame_stride_of(c->tokens_per_frame) : 0;
    return pg;
}

int check_plan_args(const vdit_mask_cfg* mask, const vdit_grid& g, int32_t t0, const vdit_kv_cache* c) {
    int st = check_mask(mask);
    if (st) return st;
    if ((st = check_grid(g))) return st;
    if (t0 < 0) return fail(VDIT_ERR_INVALID_ARG, "t0 %d must be >= 0", t0);
    if ((int64_t)t0 + g.frames > INT32_MAX / 2) return fail(VDIT_ERR_INVALID_ARG, "t0 too large");
    if (c) {
        if ((st = check_cache(c))) return st;
        if (g.height * g.width != c->tokens_per_frame)
            return fail(VDIT_ERR_INVALID_ARG, "query grid has %d tokens per frame, cache %d", g.height * g.width,
                        c->tokens_per_frame);
    }
    return VDIT_OK;
}

// Arguments of an append; fills *r (the rotation tables) when rope is given.
int check_append(const vdit_kv_cache* c, const vdit_rope_cfg* rope, vdit_grid grid, int32_t t0, vdit_tensor k,
                 vdit_tensor v, RopeDev* r) {
    int st = check_cache(c);
    if (st) return st;
    if (!c->k || !c->v || !c->slot_frame_dev || !c->slot_frame_host)
        return fail(VDIT_ERR_INVALID_ARG, "cache buffers must be set");
    if ((st = check_grid(grid))) return st;
    if (grid.height * grid.width != c->tokens_per_frame)
        return fail(VDIT_ERR_INVALID_ARG, "grid has %d tokens per frame, cache %d", grid.height * grid.width,
                    c->tokens_per_frame);
    if (grid.frames < 1 || grid.frames > c->capacity)
        return fail(VDIT_ERR_INVALID_ARG, "frames %d must be in [1, capacity %d]", grid.frames, c->capacity);
    if (t0 < 0 || (int64_t)t0 + grid.frames > INT32_MAX / 2) return fail(VDIT_ERR_INVALID_ARG, "t0 %d out of range", t0);
    int32_t n = grid.frames * c->tokens_per_frame;
    if ((st = check_tensor(k, "k", n, c->heads, c->head_dim))) return st;
    if ((st = check_tensor(v, "v", n, c->heads, c->head_dim))) return st;
    if (k.dtype != v.dtype) return fail(VDIT_ERR_INVALID_ARG, "k and v must have the same dtype");
    *r = RopeDev{};
    if (rope) {
        if ((st = check_rope_use(rope, c->head_dim, grid, t0))) return st;
        *r = rope_dev(rope);
    }
    return VDIT_OK;
}

}  // namespace

extern "C" {

int vdit_abi_version(void) { return VDIT_ABI_VERSION; }

const char* vdit_last_error(void) { return g_last_error.c_str(); }

const char* vdit_status_string(int status) {
    switch (status) {
        case VDIT_OK: return "ok";
        case VDIT_ERR_INVALID_ARG: return "invalid argument";
        case VDIT_ERR_BUFFER_TOO_SMALL: return "buffer too small";
        case VDIT_ERR_UNSUPPORTED: return "unsupported";
        case VDIT_ERR_DEVICE: return "device error";
        default: return "unknown status";
    }
}

int vdit_token_positions(vdit_grid grid, int32_t t0, int32_t where, int32_t* out, void* stream) {
    int st = check_grid(grid);
    if (st) return st;
    if (t0 < 0) return fail(VDIT_ERR_INVALID_ARG, "t0 %d must be >= 0", t0);
    if (!out) return fail(VDIT_ERR_INVALID_ARG, "out is NULL");
    if (where == VDIT_WHERE_HOST) {
        int32_t hw = grid.height * grid.width, n = grid.frames * hw;
        for (int32_t i = 0; i < n; ++i) {
            int32_t s = i % hw;
            out[3 * i + 0] = t0 + i / hw;
            out[3 * i + 1] = s / grid.width;
            out[3 * i + 2] = s % grid.width;
        }
        return ok();
    }
    if (where != VDIT_WHERE_DEVICE) return fail(VDIT_ERR_INVALID_ARG, "where %d", where);
    return device_status(launch_positions(grid, t0, out, (hipStream_t)stream), "positions kernel");
}

int vdit_rope_table_build(const vdit_rope_cfg* cfg, float* host_out, size_t cap_floats, size_t* needed_floats) {
    int st = check_rope_dims(cfg);
    if (st) return st;
    size_t need = (size_t)cfg->max_t * cfg->dim_t + (size_t)cfg->max_h * cfg->dim_h + (size_t)cfg->max_w * cfg->dim_w;
    if (needed_floats) *needed_floats = need;
    if (!host_out || cap_floats < need)
        return fail(VDIT_ERR_BUFFER_TOO_SMALL, "rope table needs %zu floats, have %zu", need, cap_floats);
    const int32_t dims[3] = {cfg->dim_t, cfg->dim_h, cfg->dim_w};
    const int32_t rows[3] = {cfg->max_t, cfg->max_h, cfg->max_w};
    float* p = host_out;
    for (int a = 0; a < 3; ++a) {
        int32_t pairs = dims[a] / 2;
        for (int32_t r = 0; r < rows[a]; ++r) {
            for (int32_t j = 0; j < pairs; ++j) {
                double w = pow(cfg->theta, -2.0 * (double)j / (double)dims[a]);
                double ang = (double)r * w;
                *p++ = (float)cos(ang);
                *p++ = (float)sin(ang);
            }
        }
    }
    return ok();
}

int vdit_rope3d_qk(const vdit_rope_cfg* cfg, vdit_grid grid, int32_t t0, int32_t heads, vdit_tensor q,
                   vdit_tensor k, void* stream) {
    int st = check_grid(grid);
    if (st) return st;
    if (t0 < 0) return fail(VDIT_ERR_INVALID_ARG, "t0 %d must be >= 0", t0);
    if (heads <= 0) return fail(VDIT_ERR_INVALID_ARG, "heads %d must be > 0", heads);
    if (!cfg) return fail(VDIT_ERR_INVALID_ARG, "rope cfg is NULL");
    if (cfg->head_dim != 64 && cfg->head_dim != 128)
        return fail(VDIT_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", cfg->head_dim);
    if ((st = check_rope_use(cfg, cfg->head_dim, grid, t0))) return st;
    int32_t n = grid.frames * grid.height * grid.width;
    if (q.data && (st = check_tensor(q, "q", n, heads, cfg->head_dim))) return st;
    if (k.data && (st = check_tensor(k, "k", n, heads, cfg->head_dim))) return st;
    if (n == 0) return ok();
    RopeDev r = rope_dev(cfg);
    hipStream_t s = (hipStream_t)stream;
    // Q and K in one launch when they have one dtype and their address ranges are disjoint;
    // otherwise one launch after the other, so that elements they share are rotated in order.
    auto range_end = [&](const vdit_tensor& x) {
        const int64_t es = x.dtype == VDIT_DTYPE_FP32 ? 4 : 2;
        return (uintptr_t)x.data + (uintptr_t)(((int64_t)(n - 1) * x.stride_token + (int64_t)(heads - 1) * x.stride_head +
                                                cfg->head_dim) * es);
    };
    if (q.data && k.data && q.dtype == k.dtype &&
        (range_end(q) <= (uintptr_t)k.data || range_end(k) <= (uintptr_t)q.data))
        return device_status(launch_rope_inplace(r, grid, t0, heads, cfg->head_dim, q, &k, s), "rope kernel (q, k)");
    if (q.data) {
        if ((st = device_status(launch_rope_inplace(r, grid, t0, heads, cfg->head_dim, q, nullptr, s),
                                "rope kernel (q)")))
            return st;
    }
    if (k.data)
        return device_status(launch_rope_inplace(r, grid, t0, heads, cfg->head_dim, k, nullptr, s), "rope kernel (k)");
    return ok();
}

int vdit_kv_cache_bytes(int32_t capacity, int32_t tokens_per_frame, int32_t heads, int32_t head_dim,
                        size_t* k_bytes, size_t* v_bytes) {
    vdit_kv_cache c{};
    c.capacity = capacity;
    c.tokens_per_frame = tokens_per_frame;
    c.heads = heads;
    c.head_dim = head_dim;
    int st = check_cache(&c);
    if (st) return st;
    size_t b = (size_t)heads * capacity * frame_stride_of(tokens_per_frame) * head_dim * 2;
    if (k_bytes) *k_bytes = b;
    if (v_bytes) *v_bytes = b;
    return ok();
}

int vdit_kv_cache_reset(vdit_kv_cache* c, void* stream) {
    int st = check_cache(c);
    if (st) return st;
    if (!c->slot_frame_dev || !c->slot_frame_host) return fail(VDIT_ERR_INVALID_ARG, "slot tables must be set");
    for (int32_t i = 0; i < c->capacity; ++i) c->slot_frame_host[i] = -1;
    return device_status(launch_fill_i32(c->slot_frame_dev, -1, c->capacity, (hipStream_t)stream), "fill kernel");
}

int vdit_kv_append(vdit_kv_cache* c, const vdit_rope_cfg* rope, vdit_grid grid, int32_t t0, vdit_tensor k,
                   vdit_tensor v, void* stream) {
    RopeDev r;
    int st = check_append(c, rope, grid, t0, k, v, &r);
    if (st) return st;
    hipError_t e = launch_kv_append(*c, rope ? &r : nullptr, grid, t0, k, v, (hipStream_t)stream);
    if (e != hipSuccess) return device_status(e, "kv append kernel");
    for (int32_t f = 0; f < grid.frames; ++f) c->slot_frame_host[(t0 + f) % c->capacity] = t0 + f;
    return ok();
}

int vdit_kv_append_plan(vdit_kv_cache* c, const vdit_rope_cfg* rope, vdit_grid grid, int32_t t0, vdit_tensor k,
                        vdit_tensor v, const vdit_mask_cfg* mask, int32_t* plan_dev, size_t cap_words,
                        size_t* used_words, void* stream) {
    RopeDev r;
    int st = check_append(c, rope, grid, t0, k, v, &r);
    if (st) return st;
    if ((st = check_plan_args(mask, grid, t0, c))) return st;
    if (!plan_dev) return fail(VDIT_ERR_INVALID_ARG, "plan_dev is NULL");
    const PlanGeom g = make_geom(mask, grid, t0, c);
    const int32_t nq = plan_qtile_count(g);
    const size_t bound = plan_bound_words(nq, c->capacity);
    if (cap_words < bound)
        return fail(VDIT_ERR_BUFFER_TOO_SMALL, "device plan needs %zu words, have %zu", bound, cap_words);
    if (used_words) *used_words = bound;
    hipError_t e =
        launch_kv_append_plan(*c, rope ? &r : nullptr, grid, t0, k, v, g, nq, plan_dev, (hipStream_t)stream);
    if (e != hipSuccess) return device_status(e, "kv append + plan kernel");
    for (int32_t f = 0; f < grid.frames; ++f) c->slot_frame_host[(t0 + f) % c->capacity] = t0 + f;
    return ok();
}

int vdit_plan_qtiles(const vdit_mask_cfg* mask, vdit_grid q_grid, int32_t q_t0, int32_t* n_qtiles) {
    int st = check_plan_args(mask, q_grid, q_t0, nullptr);
    if (st) return st;
    if (!n_qtiles) return fail(VDIT_ERR_INVALID_ARG, "n_qtiles is NULL");
    PlanGeom g = make_geom(mask, q_grid, q_t0, nullptr);
    *n_qtiles = plan_qtile_count(g);
    return ok();
}

int vdit_plan_bound(const vdit_mask_cfg* mask, vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache,
                    size_t* max_words) {
    int st = check_plan_args(mask, q_grid, q_t0, cache);
    if (st) return st;
    if (!cache) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (!max_words) return fail(VDIT_ERR_INVALID_ARG, "max_words is NULL");
    PlanGeom g = make_geom(mask, q_grid, q_t0, cache);
    *max_words = plan_bound_words(plan_qtile_count(g), cache->capacity);
    return ok();
}

int vdit_plan_mask(const vdit_mask_cfg* mask, vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache,
                   int32_t where, int32_t* plan_out, size_t cap_words, size_t* used_words, void* stream) {
    int st = check_plan_args(mask, q_grid, q_t0, cache);
    if (st) return st;
    if (!cache) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (!plan_out) return fail(VDIT_ERR_INVALID_ARG, "plan_out is NULL");
    PlanGeom g = make_geom(mask, q_grid, q_t0, cache);
    int32_t nq = plan_qtile_count(g);
    size_t bound = plan_bound_words(nq, cache->capacity);
    if (where == VDIT_WHERE_DEVICE) {
        if (!cache->slot_frame_dev) return fail(VDIT_ERR_INVALID_ARG, "cache has no device slot table");
        if (cap_words < bound)
            return fail(VDIT_ERR_BUFFER_TOO_SMALL, "device plan needs %zu words, have %zu", bound, cap_words);
        if (used_words) *used_words = bound;
        return device_status(launch_plan_build(g, cache->slot_frame_dev, nq, plan_out, (hipStream_t)stream),
                             "plan kernel");
    }
    if (where != VDIT_WHERE_HOST) return fail(VDIT_ERR_INVALID_ARG, "where %d", where);
    if (!cache->slot_frame_host) return fail(VDIT_ERR_INVALID_ARG, "cache has no host slot table");
    // exact size first, so that a short buffer is reported before anything is written
    int64_t n_spans = 0;
    for (int32_t i = 0; i < nq; ++i) {
        QTile qt = plan_qtile(g, i);
        plan_tile_spans(g, cache->slot_frame_host, qt, [&](int32_t, int32_t) { ++n_spans; });
    }
    size_t need = (size_t)VDIT_PLAN_HEADER_WORDS + 3 * (size_t)nq + 1 + 2 * (size_t)n_spans;
    if (used_words) *used_words = need;
    if (cap_words < need) return fail(VDIT_ERR_BUFFER_TOO_SMALL, "plan needs %zu words, have %zu", need, cap_words);
    int32_t* qtiles = plan_out + VDIT_PLAN_HEADER_WORDS;
    int32_t* row_ptr = qtiles + 2 * nq;
    int32_t* spans = row_ptr + nq + 1;
    int64_t pairs = 0;
    int32_t k = 0;
    row_ptr[0] = 0;
    for (int32_t i = 0; i < nq; ++i) {
        QTile qt = plan_qtile(g, i);
        qtiles[2 * i] = qt.q_start;
        qtiles[2 * i + 1] = qt.q_len;
        int64_t keys = 0;
        plan_tile_spans(g, cache->slot_frame_host, qt, [&](int32_t s0, int32_t len) {
            spans[2 * k] = s0;
            spans[2 * k + 1] = len;
            ++k;
            keys += len;
        });
        row_ptr[i + 1] = k;
        pairs += keys * qt.q_len;
    }
    plan_out[0] = (int32_t)VDIT_PLAN_MAGIC;
    plan_out[1] = VDIT_PLAN_VERSION;
    plan_out[2] = mask->kind;
    plan_out[3] = mask->tile;
    plan_out[4] = nq;
    plan_out[5] = k;
    plan_out[6] = (int32_t)(uint32_t)((uint64_t)pairs & 0xFFFFFFFFu);
    plan_out[7] = (int32_t)(uint32_t)((uint64_t)pairs >> 32);
    plan_set_call(plan_out, g);
    return ok();
}

int vdit_plan_dynamic_bound(const vdit_mask_cfg* base, vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache,
                            size_t* max_words) {
    int st = check_plan_args(base, q_grid, q_t0, cache);
    if (st) return st;
    if (!cache) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (!max_words) return fail(VDIT_ERR_INVALID_ARG, "max_words is NULL");
    PlanGeom g = make_geom(base, q_grid, q_t0, cache);
    // every key tile of every slot may form its own run
    *max_words = plan_bound_words(plan_qtile_count(g), cache->capacity * ceil_div(g.hw, g.tile));
    return ok();
}

int vdit_plan_dynamic_workspace_bytes(const vdit_mask_cfg* base, vdit_grid q_grid, int32_t q_t0,
                                      const vdit_kv_cache* cache, size_t* bytes) {
    int st = check_plan_args(base, q_grid, q_t0, cache);
    if (st) return st;
    if (!cache) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (!bytes) return fail(VDIT_ERR_INVALID_ARG, "bytes is NULL");
    PlanGeom g = make_geom(base, q_grid, q_t0, cache);
    *bytes = dyn_workspace_bytes(g, plan_qtile_count(g), cache->heads, cache->head_dim);
    return ok();
}

int vdit_plan_dynamic(const vdit_mask_cfg* base, const vdit_dynamic_cfg* dyn, vdit_tensor q, const vdit_rope_cfg* rope,
                      vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache, int32_t* plan_dev, size_t cap_words,
                      float* proxies_dev, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_plan_args(base, q_grid, q_t0, cache);
    if (st) return st;
    if (!cache) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (!cache->k || !cache->v || !cache->slot_frame_dev) return fail(VDIT_ERR_INVALID_ARG, "cache buffers must be set");
    if (!dyn) return fail(VDIT_ERR_INVALID_ARG, "dynamic cfg is NULL");
    if (!(dyn->tau >= 0.f && dyn->tau <= 1.f)) return fail(VDIT_ERR_INVALID_ARG, "tau %g outside [0, 1]", dyn->tau);
    if (!plan_dev) return fail(VDIT_ERR_INVALID_ARG, "plan is NULL");
    int32_t n = q_grid.frames * q_grid.height * q_grid.width;
    if ((st = check_tensor(q, "q", n, cache->heads, cache->head_dim))) return st;
    PlanGeom g = make_geom(base, q_grid, q_t0, cache);
    const int32_t nq = plan_qtile_count(g);
    if ((int64_t)cache->capacity * ceil_div(g.hw, g.tile) > kDynMaxKeyTiles)
        return fail(VDIT_ERR_UNSUPPORTED, "%d key tiles in the cache; the dynamic plan weighs at most %d",
                    cache->capacity * ceil_div(g.hw, g.tile), kDynMaxKeyTiles);
    const size_t need = plan_bound_words(nq, cache->capacity * ceil_div(g.hw, g.tile));
    if (cap_words < need)
        return fail(VDIT_ERR_BUFFER_TOO_SMALL, "plan buffer holds %zu words, the bound is %zu", cap_words, need);
    const size_t ws_need = dyn_workspace_bytes(g, nq, cache->heads, cache->head_dim);
    if (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 255))
        return fail(VDIT_ERR_BUFFER_TOO_SMALL, "workspace %p of %zu bytes; the call needs %zu bytes, 256-byte aligned",
                    workspace, workspace_bytes, ws_need);
    DynLaunch a{};
    a.workspace = workspace;
    if (rope) {
        if ((st = check_rope_use(rope, cache->head_dim, q_grid, q_t0))) return st;
        a.rope = rope_dev(rope);
        a.has_rope = true;
    }
    float scale = dyn->softmax_scale > 0.f ? dyn->softmax_scale : 1.0f / sqrtf((float)cache->head_dim);
    a.geom = g;
    a.q = q;
    a.width = q_grid.width;
    a.heads = cache->heads;
    a.head_dim = cache->head_dim;
    a.n_qtiles = nq;
    a.slot_frame = cache->slot_frame_dev;
    a.kc = cache->k;
    a.kv_rows = (int64_t)cache->capacity * frame_stride_of(cache->tokens_per_frame);
    a.scale = scale;
    a.keep_frac = 1.0f - dyn->tau;
    a.proxies = proxies_dev;
    a.plan = plan_dev;
    if (n == 0 || nq == 0) return ok();
    return device_status(launch_plan_dynamic(a, (hipStream_t)stream), "dynamic plan kernels");
}

namespace {
// The rule of an attention call: a plan from vdit_plan_dynamic is marked in the kind, and the
// geometry is the base rule's.
struct AttnRule {
    vdit_mask_cfg base{};
    const vdit_mask_cfg* mask = nullptr;
    bool dynamic = false;
};
AttnRule attn_rule(const vdit_mask_cfg* mask_in) {
    AttnRule r;
    r.mask = mask_in;
    if (mask_in && (mask_in->kind & VDIT_MASK_FLAG_DYNAMIC)) {
        r.base = *mask_in;
        r.base.kind &= ~VDIT_MASK_FLAG_DYNAMIC;
        r.mask = &r.base;
        r.dynamic = true;
    }
    return r;
}

// Workspace bytes of an attention call on the current device (arguments already checked).
int attn_ws_need(const vdit_mask_cfg* mask, bool dynamic, int32_t heads, int32_t n_qtiles, size_t* need) {
    const bool unit = !attn_uses_tile_kernel(mask->kind, dynamic);
    int grid = 0;
    if (unit) {
        hipError_t e = attn_unit_grid(&grid);
        if (e != hipSuccess) return device_status(e, "device attribute query");
    }
    *need = attn_workspace_bytes(grid, heads, n_qtiles, unit, dynamic);
    return VDIT_OK;
}
}  // namespace

int vdit_block_attn_workspace_bytes(const vdit_mask_cfg* mask_in, vdit_grid q_grid, int32_t q_t0,
                                    const vdit_kv_cache* cache, size_t* bytes) {
    const AttnRule r = attn_rule(mask_in);
    int st = check_plan_args(r.mask, q_grid, q_t0, cache);
    if (st) return st;
    if (!cache) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (!bytes) return fail(VDIT_ERR_INVALID_ARG, "bytes is NULL");
    PlanGeom g = make_geom(r.mask, q_grid, q_t0, cache);
    if ((st = attn_ws_need(r.mask, r.dynamic, cache->heads, plan_qtile_count(g), bytes))) return st;
    return ok();
}

namespace {
// vdit_block_attn_fwd with the caller's workspace, or (static_scratch) with the library's
// static scratch array of this device.
int attn_fwd_impl(vdit_tensor q, const vdit_rope_cfg* rope, vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache,
                  const vdit_mask_cfg* mask_in, const int32_t* plan_dev, float softmax_scale, vdit_tensor o, float* lse,
                  void* workspace, size_t workspace_bytes, bool static_scratch, void* stream) {
    const AttnRule rule = attn_rule(mask_in);
    const vdit_mask_cfg* mask = rule.mask;
    const bool unpaired = rule.dynamic;
    int st = check_plan_args(mask, q_grid, q_t0, cache);
    if (st) return st;
    if (!cache) return fail(VDIT_ERR_INVALID_ARG, "cache is NULL");
    if (!cache->k || !cache->v) return fail(VDIT_ERR_INVALID_ARG, "cache buffers must be set");
    if (!plan_dev) return fail(VDIT_ERR_INVALID_ARG, "plan is NULL");
    int32_t n = q_grid.frames * q_grid.height * q_grid.width;
    if ((st = check_tensor(q, "q", n, cache->heads, cache->head_dim))) return st;
    if ((st = check_tensor(o, "o", n, cache->heads, cache->head_dim))) return st;
    if (lse && ((uintptr_t)lse & 3)) return fail(VDIT_ERR_INVALID_ARG, "lse not 4-byte aligned");
    AttnLaunch a{};
    if (rope) {
        if ((st = check_rope_use(rope, cache->head_dim, q_grid, q_t0))) return st;
        a.rope = rope_dev(rope);
        a.has_rope = true;
    }
    if (!(softmax_scale > 0.0f)) softmax_scale = 1.0f / sqrtf((float)cache->head_dim);
    PlanGeom g = make_geom(mask, q_grid, q_t0, cache);
    a.q = q;
    a.o = o;
    a.lse = lse;
    a.kc = cache->k;
    a.vt = cache->v;
    a.kv_rows = (int64_t)cache->capacity * frame_stride_of(cache->tokens_per_frame);
    a.plan = plan_dev;
    a.hw = cache->tokens_per_frame;
    a.wf = q_grid.width;
    a.t0 = q_t0;
    a.n_tokens = n;
    a.heads = cache->heads;
    a.head_dim = cache->head_dim;
    a.n_qtiles = plan_qtile_count(g);
    a.mask_kind = mask->kind;
    a.plan_kind = mask_in->kind;  // the dynamic flag included
    a.plan_tile = g.tile;
    a.unpaired = unpaired;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    if (n == 0 || a.n_qtiles == 0) return ok();
    if (a.n_qtiles > kAttnMaxQTiles)
        return fail(VDIT_ERR_UNSUPPORTED, "%d query tiles in one call; at most %d (split the call by frames)",
                    a.n_qtiles, kAttnMaxQTiles);
    size_t ws_need = 0;
    if ((st = attn_ws_need(mask, unpaired, cache->heads, a.n_qtiles, &ws_need))) return st;
    if (static_scratch) {
        if (ws_need > kAttnStaticScratchBytes)
            return fail(VDIT_ERR_UNSUPPORTED, "the call needs %zu bytes of scratch; the static scratch holds %zu",
                        ws_need, kAttnStaticScratchBytes);
        hipError_t e = attn_static_scratch(&workspace);
        if (e != hipSuccess) return device_status(e, "static scratch address");
        workspace_bytes = kAttnStaticScratchBytes;
        // the unit kernel's arrival counters must start at zero: the array keeps whatever the
        // last call on this device left there
        if (!attn_uses_tile_kernel(mask->kind, unpaired)) {
            int grid = 0;
            if ((e = attn_unit_grid(&grid)) != hipSuccess) return device_status(e, "device attribute query");
            const size_t off = attn_workspace_counter_offset(grid);
            e = launch_fill_i32(reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + off), 0,
                                (int64_t)cache->heads * a.n_qtiles, (hipStream_t)stream);
            if (e != hipSuccess) return device_status(e, "fill kernel");
        }
    }
    if (ws_need > 0 && (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 255)))
        return fail(VDIT_ERR_BUFFER_TOO_SMALL, "workspace %p of %zu bytes; the call needs %zu bytes, 256-byte aligned",
                    workspace, workspace_bytes, ws_need);
    a.workspace = workspace;
    return device_status(launch_attn_fwd(a, (hipStream_t)stream), "attention kernel");
}

}  // namespace

int vdit_block_attn_fwd(vdit_tensor q, const vdit_rope_cfg* rope, vdit_grid q_grid, int32_t q_t0,
                        const vdit_kv_cache* cache, const vdit_mask_cfg* mask, const int32_t* plan_dev,
                        float softmax_scale, vdit_tensor o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
    return attn_fwd_impl(q, rope, q_grid, q_t0, cache, mask, plan_dev, softmax_scale, o, lse, workspace,
                         workspace_bytes, false, stream);
}

int vdit_block_attn_fwd_static(vdit_tensor q, const vdit_rope_cfg* rope, vdit_grid q_grid, int32_t q_t0,
                               const vdit_kv_cache* cache, const vdit_mask_cfg* mask, const int32_t* plan_dev,
                               float softmax_scale, vdit_tensor o, float* lse, void* stream) {
    return attn_fwd_impl(q, rope, q_grid, q_t0, cache, mask, plan_dev, softmax_scale, o, lse, nullptr, 0, true,
                         stream);
}

int vdit_block_rel_l1_workspace_bytes(int32_t n_blocks, int64_t block_elems, size_t* bytes) {
    if (!bytes) return fail(VDIT_ERR_INVALID_ARG, "bytes is NULL");
    if (n_blocks < 1 || n_blocks > 65535) return fail(VDIT_ERR_INVALID_ARG, "n_blocks %d outside [1, 65535]", n_blocks);
    if (block_elems < 0) return fail(VDIT_ERR_INVALID_ARG, "block_elems %lld < 0", (long long)block_elems);
    *bytes = rel_l1_workspace_bytes(n_blocks, block_elems);
    return ok();
}

int vdit_block_rel_l1(const void* cur, const void* prev, int32_t dtype, int32_t n_blocks, int64_t block_elems,
                      int64_t block_stride, float* out_dev, void* workspace, size_t workspace_bytes, void* stream) {
    if (!out_dev) return fail(VDIT_ERR_INVALID_ARG, "out is NULL");
    if (block_elems > 0 && (!cur || !prev)) return fail(VDIT_ERR_INVALID_ARG, "cur and prev must be set");
    if (dtype != VDIT_DTYPE_BF16 && dtype != VDIT_DTYPE_FP32)
        return fail(VDIT_ERR_UNSUPPORTED, "dtype %d is not bf16 or fp32", dtype);
    if (n_blocks < 1 || n_blocks > 65535) return fail(VDIT_ERR_INVALID_ARG, "n_blocks %d outside [1, 65535]", n_blocks);
    if (block_elems < 0 || block_stride < block_elems)
        return fail(VDIT_ERR_INVALID_ARG, "block_elems %lld, block_stride %lld", (long long)block_elems,
                    (long long)block_stride);
    const int64_t align = dtype == VDIT_DTYPE_BF16 ? 8 : 4;
    if (block_stride % align) return fail(VDIT_ERR_INVALID_ARG, "block_stride must be a multiple of %lld", (long long)align);
    if (((uintptr_t)cur & 15) || ((uintptr_t)prev & 15))
        return fail(VDIT_ERR_INVALID_ARG, "feature pointers must be 16-byte aligned");
    if (((uintptr_t)out_dev & 3)) return fail(VDIT_ERR_INVALID_ARG, "out not 4-byte aligned");
    const size_t ws_need = rel_l1_workspace_bytes(n_blocks, block_elems);
    if (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 15))
        return fail(VDIT_ERR_BUFFER_TOO_SMALL, "workspace %p of %zu bytes; the call needs %zu bytes, 16-byte aligned",
                    workspace, workspace_bytes, ws_need);
    return device_status(launch_rel_l1(cur, prev, dtype == VDIT_DTYPE_FP32, n_blocks, block_elems, block_stride,
                                       out_dev, workspace, (hipStream_t)stream),
                         "relative L1 kernels");
}

int vdit_reuse_decide(const vdit_reuse_cfg* cfg, int32_t step, float mean_rel_l1, int32_t* first_reuse, int32_t* run,
                      uint8_t* reuse_out) {
    if (!cfg || !first_reuse || !run || !reuse_out) return fail(VDIT_ERR_INVALID_ARG, "NULL argument");
    if (cfg->n_blocks < 1 || cfg->reuse_interval < 1 || cfg->total_steps < 1)
        return fail(VDIT_ERR_INVALID_ARG, "n_blocks %d, reuse_interval %d, total_steps %d must be >= 1",
                    cfg->n_blocks, cfg->reuse_interval, cfg->total_steps);
    if (step < 0 || step >= cfg->total_steps)
        return fail(VDIT_ERR_INVALID_ARG, "step %d outside [0, %d)", step, cfg->total_steps);
    const int32_t k = *first_reuse;
    const bool protected_tail = k >= 0 && step >= cfg->total_steps - k / 2;
    bool can = step > 0 && mean_rel_l1 < cfg->delta && !protected_tail;
    // a first reuse here would put this very step inside its own protected tail
    if (can && k < 0 && step >= cfg->total_steps - step / 2) can = false;
    bool any = false;
    for (int32_t b = 0; b < cfg->n_blocks; ++b) {
        const bool r = can && run[b] + 1 < cfg->reuse_interval;
        reuse_out[b] = r ? 1 : 0;
        any = any || r;
    }
    if (any && k < 0) *first_reuse = step;
    for (int32_t b = 0; b < cfg->n_blocks; ++b) run[b] = reuse_out[b] ? run[b] + 1 : 0;
    return ok();
}

int vdit_qkv_rope_append(vdit_tensor x, int32_t hidden, const void* w_qkv, int64_t w_stride, const float* b_qkv,
                         const vdit_rope_cfg* rope, vdit_grid grid, int32_t t0, vdit_kv_cache* c, vdit_tensor q_out,
                         void* stream) {
    int st = check_cache(c);
    if (st) return st;
    if (!c->k || !c->v || !c->slot_frame_dev || !c->slot_frame_host)
        return fail(VDIT_ERR_INVALID_ARG, "cache buffers must be set");
    if ((st = check_grid(grid))) return st;
    if (grid.height * grid.width != c->tokens_per_frame)
        return fail(VDIT_ERR_INVALID_ARG, "grid has %d tokens per frame, cache %d", grid.height * grid.width,
                    c->tokens_per_frame);
    if (grid.frames < 1 || grid.frames > c->capacity)
        return fail(VDIT_ERR_INVALID_ARG, "frames %d must be in [1, capacity %d]", grid.frames, c->capacity);
    if (t0 < 0 || (int64_t)t0 + grid.frames > INT32_MAX / 2) return fail(VDIT_ERR_INVALID_ARG, "t0 %d out of range", t0);
    if (hidden < 64 || hidden % 64) return fail(VDIT_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 64", hidden);
    if ((c->heads * c->head_dim) % 128)
        return fail(VDIT_ERR_UNSUPPORTED, "heads x head_dim %d must be a multiple of 128", c->heads * c->head_dim);
    if (!w_qkv || ((uintptr_t)w_qkv & 15)) return fail(VDIT_ERR_INVALID_ARG, "w_qkv NULL or not 16-byte aligned");
    if (w_stride < hidden || w_stride % 8) return fail(VDIT_ERR_INVALID_ARG, "w_stride %lld", (long long)w_stride);
    if (b_qkv && ((uintptr_t)b_qkv & 3)) return fail(VDIT_ERR_INVALID_ARG, "b_qkv not 4-byte aligned");
    const int32_t n = grid.frames * c->tokens_per_frame;
    if (!x.data || x.dtype != VDIT_DTYPE_BF16 || x.reserved)
        return fail(x.data && x.dtype != VDIT_DTYPE_BF16 ? VDIT_ERR_UNSUPPORTED : VDIT_ERR_INVALID_ARG,
                    "x must be bf16 device data");
    if (((uintptr_t)x.data & 15) || x.stride_token < hidden || x.stride_token % 8)
        return fail(VDIT_ERR_INVALID_ARG, "x: 16-byte aligned rows of at least hidden elements, stride a multiple of 8");
    if ((st = check_tensor(q_out, "q_out", n, c->heads, c->head_dim))) return st;
    if (q_out.dtype != VDIT_DTYPE_BF16) return fail(VDIT_ERR_UNSUPPORTED, "q_out must be bf16");
    const int64_t w_bytes = ((int64_t)3 * c->heads * c->head_dim - 1) * w_stride * 2 + (int64_t)hidden * 2;
    const int64_t x_bytes = ((int64_t)n - 1) * x.stride_token * 2 + (int64_t)hidden * 2;
    if (w_bytes >= ((int64_t)1 << 32) || x_bytes >= ((int64_t)1 << 32))
        return fail(VDIT_ERR_UNSUPPORTED, "x or w_qkv span 4 GiB or more");
    ProjLaunch L{};
    if (rope) {
        if ((st = check_rope_use(rope, c->head_dim, grid, t0))) return st;
        L.rope = rope_dev(rope);
        L.has_rope = true;
    }
    L.x = x.data;
    L.x_st = x.stride_token;
    L.n_tokens = n;
    L.hidden = hidden;
    L.w = w_qkv;
    L.w_st = w_stride;
    L.bias = b_qkv;
    L.heads = c->heads;
    L.head_dim = c->head_dim;
    L.hw = c->tokens_per_frame;
    L.wf = grid.width;
    L.t0 = t0;
    L.q = q_out.data;
    L.q_st = q_out.stride_token;
    L.q_sh = q_out.stride_head;
    L.kc = c->k;
    L.vt = c->v;
    L.frame_stride = frame_stride_of(c->tokens_per_frame);
    L.kv_rows = (int64_t)c->capacity * L.frame_stride;
    L.capacity = c->capacity;
    L.slot_frame = c->slot_frame_dev;
    L.frames = grid.frames;
    hipError_t e = launch_qkv_rope_append(L, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_kv_zero_pad(*c, grid, t0, (hipStream_t)stream);
    if (e != hipSuccess) return device_status(e, "projection kernels");
    for (int32_t f = 0; f < grid.frames; ++f) c->slot_frame_host[(t0 + f) % c->capacity] = t0 + f;
    return ok();
}

}  // extern "C"
