/*
 * vdit.h - C ABI of the MI355X (gfx950) RoPE3D + block-sparse KV-cache attention library.
 *
 * One attention call of a video diffusion transformer's denoising chunk: the chunk's
 * queries, rotated by a 3D rotary encoding whose time coordinate is the global frame
 * index (start frame t0 + local frame), attend to a ring-buffer KV cache of earlier
 * frames under a chunk-causal, log-radial or dense visibility rule, computed as a
 * tiled flash-attention forward pass that never touches invisible key tiles.
 *
 * Conventions for every entry point
 * - Return value: VDIT_OK (0) or a VDIT_ERR_* status.  All arguments are validated
 *   before anything is enqueued: on error nothing was launched and no output was
 *   touched.  vdit_last_error() returns a message for the calling thread's last error.
 *   Faults inside a kernel surface at the caller's next synchronisation; a launch the
 *   runtime rejects returns VDIT_ERR_DEVICE.
 * - Memory: every buffer passed in is allocated and owned by the caller, the scratch
 *   workspaces of vdit_block_attn_fwd, vdit_plan_dynamic and vdit_block_rel_l1 included
 *   (each has a *_workspace_bytes size query).  Pointers documented "device" must be device
 *   memory of the current HIP device, "host" plain host memory.  The library allocates no
 *   memory and keeps no global state besides a per-thread error string, except the one entry
 *   point for callers that cannot allocate (vdit_block_attn_fwd_static), whose static device
 *   scratch array is documented there.
 * - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).  Device
 *   work is only enqueued; no call synchronises the device or a stream.  Calls that may run
 *   at the same time must not share a workspace.
 * - Tensors [tokens][heads][channels]: vdit_tensor gives the base pointer, dtype and the
 *   token / head strides in ELEMENTS; channels are contiguous.  Base pointers must be
 *   16-byte aligned and strides multiples of 8 (bf16) or 4 (fp32) elements.
 * - Token order inside a call: frame-major, then row h, then column w.
 */
#ifndef VDIT_H
#define VDIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VDIT_ABI_VERSION 2

/* status codes */
#define VDIT_OK 0
#define VDIT_ERR_INVALID_ARG 1
#define VDIT_ERR_BUFFER_TOO_SMALL 2
#define VDIT_ERR_UNSUPPORTED 3
#define VDIT_ERR_DEVICE 4

/* element types of Q / K / V / O */
#define VDIT_DTYPE_BF16 0
#define VDIT_DTYPE_FP32 1

/* visibility rules */
#define VDIT_MASK_DENSE 0
#define VDIT_MASK_CHUNK_CAUSAL 1
#define VDIT_MASK_LOG_RADIAL 2
#define VDIT_MASK_LOG_RADIAL_CAUSAL 3
/* OR-ed into the kind of the mask given to vdit_block_attn_fwd when its plan comes from
 * vdit_plan_dynamic (also set in such a plan's header kind word) */
#define VDIT_MASK_FLAG_DYNAMIC 0x100

/* where a plan or position list is produced */
#define VDIT_WHERE_HOST 0
#define VDIT_WHERE_DEVICE 1

/* plan word layout (int32): header, then query tiles, row pointers and spans */
#define VDIT_PLAN_MAGIC 0x54494456 /* 'V' 'D' 'I' 'T' */
#define VDIT_PLAN_VERSION 2
#define VDIT_PLAN_HEADER_WORDS 12

typedef struct {
    void* data;           /* device */
    int32_t dtype;        /* VDIT_DTYPE_* */
    int32_t reserved;     /* must be 0 */
    int64_t stride_token; /* elements between consecutive tokens */
    int64_t stride_head;  /* elements between consecutive heads */
} vdit_tensor;

typedef struct {
    int32_t frames, height, width; /* latent frames of height x width tokens */
} vdit_grid;

/* 3D rotary encoding.  Channels are split [t | h | w] with widths dim_t, dim_h, dim_w
 * (each even, summing to head_dim).  Pair (2j, 2j+1) of an axis group of width d is
 * rotated by p * theta^(-2j/d), p being the token's coordinate on that axis. */
typedef struct {
    int32_t head_dim, dim_t, dim_h, dim_w;
    double theta;
    int32_t max_t, max_h, max_w; /* table rows per axis: t < max_t, h < max_h, w < max_w */
    int32_t reserved;            /* must be 0 */
    const float* table;          /* device copy of vdit_rope_table_build's output (may be
                                    NULL for vdit_rope_table_build itself) */
} vdit_rope_cfg;

/* Ring-buffer KV cache of `capacity` frames of tokens_per_frame tokens.  Frame t lives in
 * slot t mod capacity.  Slot pitch frame_stride = tokens_per_frame rounded up to 8;
 * the physical key index of token s of slot j is j * frame_stride + s, and
 * kv_rows = capacity * frame_stride.
 *   k: device bf16 [heads][kv_rows][head_dim], keys already rotated at their global
 *      position;
 *   v: device bf16 [heads][head_dim][kv_rows] (values stored transposed, keys contiguous);
 *   slot_frame_dev / slot_frame_host: int32 [capacity], the global frame held by each
 *      slot or -1; the host array mirrors the device array and is updated synchronously
 *      by vdit_kv_append. */
typedef struct {
    void* k;
    void* v;
    int32_t* slot_frame_dev;
    int32_t* slot_frame_host;
    int32_t capacity, tokens_per_frame, heads, head_dim;
} vdit_kv_cache;

/* Visibility rule.  tile = 128 (query and key tile length of the plan).
 * CHUNK_CAUSAL: query at global frame tq sees key frame tk iff
 *   floor(tk / chunk_frames) <= floor(tq / chunk_frames).
 * LOG_RADIAL: with d = |tq - tk| and spatial tile indices (within-frame index / tile),
 *   a key is visible iff d == 0, or long_range_period > 0 and d % long_range_period == 0,
 *   or |tile_q - tile_k| <= W(d) = ceil(radial_w0 * 2^(-radial_decay_log2 * d))
 *   ("DynamicRad ...", section 2, log-radial window; the full clip, symmetric in time).
 * LOG_RADIAL_CAUSAL: streaming log-radial, the LOG_RADIAL rule at the global frame distance
 *   and, in addition, floor(tk / chunk_frames) <= floor(tq / chunk_frames) (block-causal
 *   chunks of the Wave Forcing page against the ring cache).  Query tiles are per frame, as
 *   for LOG_RADIAL. */
typedef struct {
    int32_t kind;
    int32_t chunk_frames;
    int32_t tile;
    int32_t radial_w0;
    int32_t radial_decay_log2;
    int32_t long_range_period;
} vdit_mask_cfg;

/* ---- informational -------------------------------------------------------------- */
int vdit_abi_version(void);
const char* vdit_last_error(void);
const char* vdit_status_string(int status);

/* ---- positions: "Accelerating Video Generation Inference with Sequential-Parallel 3D
 * Positional Encoding Using a Global Time Index", section 2.B (Causal-RoPE SP): a token's
 * global time index is its local frame plus the block's start frame.
 * Writes int32 [frames*height*width][3] = (t0 + f, h, w).  where = VDIT_WHERE_HOST: `out`
 * is host memory, filled before return (stream ignored); VDIT_WHERE_DEVICE: `out` is
 * device memory, written by a kernel on `stream`.  Errors: negative sizes or t0,
 * NULL out -> INVALID_ARG. */
int vdit_token_positions(vdit_grid grid, int32_t t0, int32_t where, int32_t* out, void* stream);

/* ---- RoPE tables: same page, section 2.C ("Pre-calculo do RoPE"): frequencies are
 * precomputed once into contiguous tensors instead of a dynamic cache.
 * Number of floats of the table: max_t*dim_t + max_h*dim_h + max_w*dim_w.
 * Layout: per axis in the order t, h, w, [rows][dim_a/2] pairs of (cos, sin) as float,
 * computed in double precision on the host and rounded to float.
 * host_out is host memory; the caller copies it to the device and stores the device
 * pointer in cfg->table.  Errors: odd or negative widths, widths not summing to
 * head_dim, theta <= 0, non-positive table rows -> INVALID_ARG; cap_floats too small
 * -> BUFFER_TOO_SMALL (*needed_floats is still set). */
int vdit_rope_table_build(const vdit_rope_cfg* cfg, float* host_out, size_t cap_floats,
                          size_t* needed_floats);

/* ---- RoPE3D in place: "Timeripple: Accelerating vDiTs by Understanding the
 * Spatio-Temporal Correlations in Latent Space", Metodologia 1 (RoPE channel groups
 * for time and the two spatial axes) with the global time index above.
 * Rotates q and/or k ([frames*height*width][heads][head_dim], bf16 or fp32, device) in
 * place at positions (t0 + f, h, w); fp32 arithmetic, one rounding to the tensor's
 * dtype.  A tensor with data == NULL is skipped.  q and k of one dtype whose address
 * ranges are disjoint are rotated in one launch; otherwise q is rotated first, then k (an
 * element that both hold is rotated twice).  Errors: coordinates beyond the table rows,
 * head_dim not 64 or 128, bad strides -> INVALID_ARG / UNSUPPORTED. */
int vdit_rope3d_qk(const vdit_rope_cfg* cfg, vdit_grid grid, int32_t t0, int32_t heads,
                   vdit_tensor q, vdit_tensor k, void* stream);

/* ---- KV cache: "Accelerating Video Generation Inference ...", section 2.A (KV cache of
 * causal chunk inference) and the Wave Forcing / WaveRT page (cache refresh once a
 * block is denoised).
 * vdit_kv_cache_bytes: sizes of the caller-allocated k and v buffers.
 * vdit_kv_cache_reset: marks every slot empty (-1) in both slot tables; the device table
 *   is written by a kernel on `stream`. */
int vdit_kv_cache_bytes(int32_t capacity, int32_t tokens_per_frame, int32_t heads, int32_t head_dim,
                        size_t* k_bytes, size_t* v_bytes);
int vdit_kv_cache_reset(vdit_kv_cache* cache, void* stream);

/* vdit_kv_append: writes `grid.frames` frames starting at global frame t0.  Frame t0+f
 * goes to slot (t0+f) mod capacity, evicting what the slot held.  k and v are
 * [frames*tokens_per_frame][heads][head_dim] (bf16 or fp32, device).  If rope is not NULL
 * the keys are rotated at their global positions (t0+f, h, w) before the write (fp32
 * arithmetic, one rounding to bf16); with rope == NULL they are stored as given.  Values
 * are rounded to bf16 and stored transposed.  The padding tokens of each written slot
 * (tokens_per_frame .. frame_stride-1) are zeroed.  Both slot tables are updated (the host
 * one before return).  Errors: grid.height*grid.width != tokens_per_frame, frames < 1 or
 * > capacity, t0 < 0, coordinates beyond the rope table, shape mismatch -> INVALID_ARG. */
int vdit_kv_append(vdit_kv_cache* cache, const vdit_rope_cfg* rope, vdit_grid grid, int32_t t0,
                   vdit_tensor k, vdit_tensor v, void* stream);

/* ---- block plan: Wave Forcing / WaveRT page (block-causal attention);
 * "DynamicRad: Content-Adaptive Sparse Attention for Long Video Diffusion", section 2
 * (log-radial window, long-range factor, static-ratio mode).
 * The query rows of a call are cut into query tiles: consecutive `tile`-row pieces of
 * each mask unit (the whole call for DENSE, the call frames of one causal chunk for
 * CHUNK_CAUSAL, one frame for LOG_RADIAL), so that all rows of a tile see the same keys.
 * For every tile the plan lists the maximal ascending runs ("spans") of visible physical
 * key indices of the cache's occupied slots.
 * Words (int32): header[12] = {VDIT_PLAN_MAGIC, VDIT_PLAN_VERSION, kind, tile, n_qtiles,
 * n_spans, pairs_lo, pairs_hi, q_t0, q_frames, tokens per frame, 0} where pairs = sum over
 * tiles of q_len * (sum of span lengths) and q_t0, q_frames and the tokens per frame are the
 * query call the plan was built for (vdit_block_attn_fwd rejects it for another call); then
 * {q_start, q_len}[n_qtiles]; row_ptr[n_qtiles + 1]; {k_start, k_len}[n_spans].
 * vdit_plan_qtiles: number of query tiles (depends on the rule and grid only).
 * vdit_plan_bound: upper bound on the plan size in words for this cache.
 * vdit_plan_mask: where = VDIT_WHERE_HOST reads slot_frame_host and writes host memory
 *   before return (*used_words = exact size); VDIT_WHERE_DEVICE reads slot_frame_dev and
 *   writes device memory from a kernel on `stream` (*used_words = the bound).  Host and
 *   device plans are identical word for word.  Errors: grid tokens per frame differing
 *   from the cache's, tile != 128, chunk_frames < 1, radial parameters < 0 -> INVALID_ARG;
 *   cap_words below the bound -> BUFFER_TOO_SMALL. */
int vdit_plan_qtiles(const vdit_mask_cfg* mask, vdit_grid q_grid, int32_t q_t0, int32_t* n_qtiles);
int vdit_plan_bound(const vdit_mask_cfg* mask, vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache,
                    size_t* max_words);
int vdit_plan_mask(const vdit_mask_cfg* mask, vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache,
                   int32_t where, int32_t* plan_out, size_t cap_words, size_t* used_words, void* stream);

/* vdit_kv_append_plan: vdit_kv_append(cache, rope, grid, t0, k, v, stream) followed by
 * vdit_plan_mask(mask, grid, t0, cache, VDIT_WHERE_DEVICE, plan_dev, cap_words, used_words,
 * stream): the device plan of the appended chunk as the query call, in one launch.  One
 * extra workgroup builds the plan from the slot table with this append's frames in their
 * slots, while the others append (two launches when capacity > 1024).  The cache contents,
 * both slot tables and the plan words are those of the two calls.  Errors: those of the two
 * calls, all checked before anything is launched. */
int vdit_kv_append_plan(vdit_kv_cache* cache, const vdit_rope_cfg* rope, vdit_grid grid, int32_t t0,
                        vdit_tensor k, vdit_tensor v, const vdit_mask_cfg* mask, int32_t* plan_dev,
                        size_t cap_words, size_t* used_words, void* stream);

/* ---- dynamic-threshold block plan: "DynamicRad: Content-Adaptive Sparse Attention for
 * Long Video Diffusion", section 2, dual-mode strategy, mode 2 (pre-softmax attention logits
 * as importance proxies, an adaptive threshold inside the static rule's candidates).
 * Key tiles: the `tile`-token pieces of each cache slot (the last piece of a frame ragged),
 * numbered j = slot * ceil(tokens_per_frame / tile) + piece.  Proxy of query tile i and key
 * tile j: scale * sum over heads of <mean rotated query of the tile, mean cached key of the
 * tile> (the mean pre-softmax logit of the tile pair summed over heads; one plan serves all
 * heads).  Candidates: the key tiles `base` (a static rule) lets the query tile see.  Kept:
 * candidates with proxy p, p - m >= (1 - tau) * (M - m), M and m the largest and smallest
 * candidate proxies of the query tile (tau = 1 keeps every candidate, tau = 0 the best).
 * The plan has the usual words (query tiles of `base`, maximal runs of kept keys), its
 * header kind is base->kind | VDIT_MASK_FLAG_DYNAMIC; attention on it takes a mask whose
 * kind has that flag.
 * q, rope: as for vdit_block_attn_fwd (the proxies use fp32 rotated queries).
 * plan_dev: device, cap_words >= vdit_plan_dynamic_bound.  proxies_dev: NULL or device fp32
 * [n_qtiles][capacity * ceil(tokens_per_frame / tile)] (written; empty slots give 0).
 * workspace: device scratch of at least vdit_plan_dynamic_workspace_bytes(base, q_grid, q_t0,
 *   cache) bytes (pooled queries and keys, partial proxies, run counts), fully rewritten by
 *   every call; its contents need no initialisation.
 * Errors: as vdit_plan_mask and vdit_block_attn_fwd; tau outside [0, 1] -> INVALID_ARG;
 *   more than 4096 key tiles (capacity * ceil(tokens_per_frame / tile)) -> UNSUPPORTED;
 *   workspace NULL or below the size query -> BUFFER_TOO_SMALL. */
typedef struct {
    float tau;
    float softmax_scale; /* scale of the proxy logits; <= 0 selects 1/sqrt(head_dim) */
} vdit_dynamic_cfg;
int vdit_plan_dynamic_bound(const vdit_mask_cfg* base, vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache,
                            size_t* max_words);
int vdit_plan_dynamic_workspace_bytes(const vdit_mask_cfg* base, vdit_grid q_grid, int32_t q_t0,
                                      const vdit_kv_cache* cache, size_t* bytes);
int vdit_plan_dynamic(const vdit_mask_cfg* base, const vdit_dynamic_cfg* dyn, vdit_tensor q, const vdit_rope_cfg* rope,
                      vdit_grid q_grid, int32_t q_t0, const vdit_kv_cache* cache, int32_t* plan_dev, size_t cap_words,
                      float* proxies_dev, void* workspace, size_t workspace_bytes, void* stream);

/* ---- attention forward: the full spatiotemporal softmax attention of "DynamicRad ..."
 * section 1 and "Accelerating Video Generation Inference ..." section 1, restricted to
 * the visible keys of the plan, as a tiled (FlashAttention-style) pass that skips the
 * invisible tiles.
 * q: [frames*height*width][heads][head_dim] bf16 or fp32 (device); if rope != NULL the
 *   queries are rotated at (q_t0 + f, h, w) while they are loaded (fp32 arithmetic, one
 *   rounding to bf16); with rope == NULL they are used as given (rounded to bf16).
 * plan_dev: device plan built for this rule, grid, q_t0 and the cache's current slots
 *   (by vdit_plan_mask, or by vdit_plan_dynamic with base = this rule, in which case
 *   mask->kind carries VDIT_MASK_FLAG_DYNAMIC).  The plan is read on the device only: the
 *   kernels check its magic, its kind (flag included) and tile against this call's rule, its
 *   tile count against this grid, and every span against the cache (inside it, 8-aligned,
 *   non-empty).  What fails is not computed: the outputs it would have written are NaN
 *   (all of them for a bad header; the query tile's rows for a bad span under the
 *   log-radial and dynamic rules) and the call still returns VDIT_OK.  A plan of the same
 *   rule and tile count built for another q_t0 or slot table is not detected.
 * softmax_scale <= 0 selects 1/sqrt(head_dim).
 * o: same shape as q, bf16 or fp32 (device).  lse: NULL or device fp32 [heads][tokens],
 *   natural-log log-sum-exp of each row's scaled logits (-inf for a row with no visible
 *   key, whose output is 0).
 * Arithmetic: bf16 products with fp32 accumulation, fp32 online softmax, P rounded to
 * bf16 before the P.V product; the softmax scale (times log2 e) is applied to Q before its
 * bf16 rounding.  A query tile's keys may be split over several workgroups, whose partial
 * results are merged in a fixed order: outputs are deterministic for a given device.
 * workspace: device scratch of at least vdit_block_attn_workspace_bytes(mask, q_grid, q_t0,
 *   cache) bytes, asked on the device that runs the call (0 for static log-radial plans,
 *   which need none).  CHUNK_CAUSAL and DENSE plans: partial results (two 135 KB slots per
 *   CU, so the size depends on the device's CU count) and, above them and above every
 *   dynamic-plan layout, per-tile arrival counters (4 bytes per head and query tile), which
 *   must be zero before the workspace's first use and which every call leaves zero.  Dynamic
 *   plans (host arithmetic: 256 + align256((n_qtiles + 1024 / heads) * 32) + 4096 +
 *   1024 * 67584 bytes, about 69 MB): the call's work list (query tiles with many kept keys
 *   are cut into chunks of near-equal length, listed longest first) and the chunks' partial
 *   results, all rewritten by every call.  The caller zeroes a new workspace once (all bytes)
 *   and may pass it to any later call on the same device whose size query does not exceed
 *   its size.  Calls that may run at the same time need separate workspaces.
 * Errors: head counts or head_dim differing from the cache's, head_dim not 64 or 128 ->
 * INVALID_ARG / UNSUPPORTED; more than 4096 query tiles in one call -> UNSUPPORTED (split the
 * call by frames); workspace NULL or below the size query -> BUFFER_TOO_SMALL. */
int vdit_block_attn_workspace_bytes(const vdit_mask_cfg* mask, vdit_grid q_grid, int32_t q_t0,
                                    const vdit_kv_cache* cache, size_t* bytes);
int vdit_block_attn_fwd(vdit_tensor q, const vdit_rope_cfg* rope, vdit_grid q_grid, int32_t q_t0,
                        const vdit_kv_cache* cache, const vdit_mask_cfg* mask, const int32_t* plan_dev,
                        float softmax_scale, vdit_tensor o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/* vdit_block_attn_fwd_static: vdit_block_attn_fwd with no workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It allocates nothing: its scratch is a static device array of
 * 72 MiB on each GPU the library runs on, held until the process ends.  Before each call it
 * clears the part that must start at zero (the arrival counters) with a small fill kernel on
 * `stream`.  Every call on a GPU shares that GPU's array: calls that may overlap on one GPU
 * (other streams, other host threads) race and must not be issued.  Arguments and results
 * as for vdit_block_attn_fwd; a call whose workspace size query exceeds 72 MiB (a grid of
 * far more CUs, or more than about 1.5 million head x query-tile counters) -> UNSUPPORTED. */
int vdit_block_attn_fwd_static(vdit_tensor q, const vdit_rope_cfg* rope, vdit_grid q_grid, int32_t q_t0,
                               const vdit_kv_cache* cache, const vdit_mask_cfg* mask, const int32_t* plan_dev,
                               float softmax_scale, vdit_tensor o, float* lse, void* stream);

/* ---- fused QKV projection + RoPE3D + K/V append ("Accelerating Video Generation Inference ...",
 * section 2.C, the QKV projection and the rotary embedding as one kernel with precomputed
 * tables; section 2.B, global positions; section 2.A, the KV cache).
 * qkv = x W^T + b for the call's frames*height*width tokens; the Q part is rotated at
 * (t0 + f, h, w) and written to q_out; the K part is rotated and the V part copied into the
 * ring slots t mod capacity, exactly as vdit_kv_append would store them (slot tables and the
 * zeroed pad tokens included).  One rounding to bf16 after the fp32 accumulation, bias and
 * rotation.
 * x: device bf16, row n = token n of the call (frame-major, then h, w), hidden elements per
 *   row, rows stride_token elements apart (a multiple of 8); stride_head and reserved unused / 0.
 * w_qkv: device bf16 [3 * heads * head_dim][w_stride] (row pitch w_stride >= hidden, a multiple
 *   of 8): rows 0 .. HD-1 give Q, HD .. 2HD-1 K, 2HD .. 3HD-1 V, each block head-major (row
 *   h * head_dim + d), HD = heads * head_dim of the cache.
 * b_qkv: NULL or device fp32 [3 * heads * head_dim].
 * q_out: bf16 [tokens][heads][head_dim] (device).  rope: as for vdit_kv_append (NULL: no
 *   rotation).
 * Errors: as vdit_kv_append; hidden not a positive multiple of 64, heads * head_dim not a
 *   multiple of 128, x / q_out not bf16, x or W spanning 4 GiB or more -> UNSUPPORTED; bad
 *   strides or alignment -> INVALID_ARG. */
int vdit_qkv_rope_append(vdit_tensor x, int32_t hidden, const void* w_qkv, int64_t w_stride, const float* b_qkv,
                         const vdit_rope_cfg* rope, vdit_grid grid, int32_t t0, vdit_kv_cache* cache, vdit_tensor q_out,
                         void* stream);

/* ---- block-wise feature reuse ("BWCache: Accelerating Video Diffusion Transformers through
 * Block-Wise Caching", section 2): the dynamic similarity indicator and the reuse decision.
 *
 * vdit_block_rel_l1: for every block b < n_blocks, the relative L1 distance
 *   r_b = sum |cur_b - prev_b| / sum |prev_b| over the block's block_elems elements (0 when
 *   both sums are 0, +inf when only the denominator is), and their mean.
 * cur, prev: device, [n_blocks][block_stride] elements of `dtype` (VDIT_DTYPE_BF16 or _FP32),
 *   the block's features first in each row; base pointers 16-byte aligned (NULL allowed when
 *   block_elems == 0), block_stride >= block_elems and a multiple of 8 (bf16) or 4 (fp32).
 * out_dev: device fp32 [n_blocks + 1]: r_0 .. r_{n_blocks-1}, then the mean.
 * Arithmetic: fp32 sums over chunks of 32768 elements, chunk sums added in fp64 in chunk
 *   order (deterministic).
 * workspace: device scratch of at least vdit_block_rel_l1_workspace_bytes(n_blocks,
 *   block_elems) bytes (8 per chunk and block), fully rewritten by every call.
 * Errors: NULL pointers, n_blocks outside [1, 65535], block_elems < 0, bad stride or alignment
 *   -> INVALID_ARG; other dtypes -> UNSUPPORTED; workspace NULL or below the size query ->
 *   BUFFER_TOO_SMALL. */
int vdit_block_rel_l1_workspace_bytes(int32_t n_blocks, int64_t block_elems, size_t* bytes);
int vdit_block_rel_l1(const void* cur, const void* prev, int32_t dtype, int32_t n_blocks, int64_t block_elems,
                      int64_t block_stride, float* out_dev, void* workspace, size_t workspace_bytes, void* stream);

/* vdit_reuse_decide (host only): the reuse flags of every block at diffusion step `step`
 * (0-based, < total_steps) given the latest indicator (the mean from vdit_block_rel_l1).
 *   - The first step computes every block (nothing is cached).
 *   - Otherwise every block reuses its cached features when mean_rel_l1 < delta, except a
 *     block already reused reuse_interval - 1 times in a row, which is recomputed (periodic
 *     recomputation; reuse_interval = 1 never reuses).
 *   - When the first reuse happens at step k, the last floor(k / 2) steps recompute every
 *     block; a first reuse that would fall inside its own protected tail does not happen.
 * State (caller-owned, host): *first_reuse (-1 before any reuse) and run[n_blocks] (the
 *   blocks' current runs of reuses, zero at the start); both are updated.
 * reuse_out: host uint8 [n_blocks], 1 = reuse.
 * Errors: NULL pointers, n_blocks < 1, reuse_interval < 1, step outside [0, total_steps) ->
 *   INVALID_ARG. */
typedef struct {
    float delta;            /* reuse threshold on the mean relative L1 distance */
    int32_t reuse_interval; /* R: at most R - 1 consecutive reuses of a block */
    int32_t total_steps;    /* diffusion steps of the run */
    int32_t n_blocks;
} vdit_reuse_cfg;
int vdit_reuse_decide(const vdit_reuse_cfg* cfg, int32_t step, float mean_rel_l1, int32_t* first_reuse, int32_t* run,
                      uint8_t* reuse_out);

#ifdef __cplusplus
}
#endif

#endif /* VDIT_H */
