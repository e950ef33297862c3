"""ctypes binding of libvdit (include/vdit.h): same names, argument marshalling only.

Tensors are torch tensors (device memory and streams come from torch); every step of
the computation runs in the library's HIP kernels.  Loading fails loudly when the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvdit.so")

VDIT_OK, VDIT_ERR_INVALID_ARG, VDIT_ERR_BUFFER_TOO_SMALL, VDIT_ERR_UNSUPPORTED, VDIT_ERR_DEVICE = range(5)
VDIT_DTYPE_BF16, VDIT_DTYPE_FP32 = 0, 1
VDIT_MASK_DENSE, VDIT_MASK_CHUNK_CAUSAL, VDIT_MASK_LOG_RADIAL, VDIT_MASK_LOG_RADIAL_CAUSAL = 0, 1, 2, 3
VDIT_MASK_FLAG_DYNAMIC = 0x100
VDIT_WHERE_HOST, VDIT_WHERE_DEVICE = 0, 1
VDIT_PLAN_MAGIC = 0x54494456
PLAN_HEADER_WORDS = 12  # VDIT_PLAN_HEADER_WORDS
MASK_KINDS = {"dense": VDIT_MASK_DENSE, "chunk_causal": VDIT_MASK_CHUNK_CAUSAL, "log_radial": VDIT_MASK_LOG_RADIAL,
              "log_radial_causal": VDIT_MASK_LOG_RADIAL_CAUSAL}

# every function declared in include/vdit.h
EXPORTS = (
    "vdit_abi_version", "vdit_last_error", "vdit_status_string", "vdit_token_positions",
    "vdit_rope_table_build", "vdit_rope3d_qk", "vdit_kv_cache_bytes", "vdit_kv_cache_reset",
    "vdit_kv_append", "vdit_kv_append_plan", "vdit_plan_qtiles", "vdit_plan_bound", "vdit_plan_mask", "vdit_plan_dynamic_bound",
    "vdit_plan_dynamic", "vdit_block_attn_fwd", "vdit_block_rel_l1", "vdit_reuse_decide", "vdit_qkv_rope_append",
    "vdit_block_attn_workspace_bytes", "vdit_plan_dynamic_workspace_bytes", "vdit_block_rel_l1_workspace_bytes",
    "vdit_block_attn_fwd_static",
)


class VditReuseCfg(ctypes.Structure):
    _fields_ = [("delta", ctypes.c_float), ("reuse_interval", ctypes.c_int32), ("total_steps", ctypes.c_int32),
                ("n_blocks", ctypes.c_int32)]


class VditTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("stride_token", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class VditGrid(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("height", ctypes.c_int32), ("width", ctypes.c_int32)]


class VditRopeCfg(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("dim_t", ctypes.c_int32), ("dim_h", ctypes.c_int32),
                ("dim_w", ctypes.c_int32), ("theta", ctypes.c_double), ("max_t", ctypes.c_int32),
                ("max_h", ctypes.c_int32), ("max_w", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("table", ctypes.c_void_p)]


class VditKVCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("slot_frame_dev", ctypes.c_void_p),
                ("slot_frame_host", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class VditMaskCfg(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("chunk_frames", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("radial_w0", ctypes.c_int32), ("radial_decay_log2", ctypes.c_int32),
                ("long_range_period", ctypes.c_int32)]


class VditDynamicCfg(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("softmax_scale", ctypes.c_float)]


class VditError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"vdit status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m video_diffusion_transformer_rope3d_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pS = ctypes.POINTER(ctypes.c_size_t)
        sig = {
            "vdit_abi_version": (I32, []),
            "vdit_last_error": (ctypes.c_char_p, []),
            "vdit_status_string": (ctypes.c_char_p, [I32]),
            "vdit_token_positions": (I32, [VditGrid, I32, I32, P, P]),
            "vdit_rope_table_build": (I32, [ctypes.POINTER(VditRopeCfg), P, SZ, pS]),
            "vdit_rope3d_qk": (I32, [ctypes.POINTER(VditRopeCfg), VditGrid, I32, I32, VditTensor, VditTensor, P]),
            "vdit_kv_cache_bytes": (I32, [I32, I32, I32, I32, pS, pS]),
            "vdit_kv_cache_reset": (I32, [ctypes.POINTER(VditKVCache), P]),
            "vdit_kv_append": (I32, [ctypes.POINTER(VditKVCache), ctypes.POINTER(VditRopeCfg), VditGrid, I32,
                                     VditTensor, VditTensor, P]),
            "vdit_kv_append_plan": (I32, [ctypes.POINTER(VditKVCache), ctypes.POINTER(VditRopeCfg), VditGrid, I32,
                                          VditTensor, VditTensor, ctypes.POINTER(VditMaskCfg), P, SZ, pS, P]),
            "vdit_plan_qtiles": (I32, [ctypes.POINTER(VditMaskCfg), VditGrid, I32, ctypes.POINTER(I32)]),
            "vdit_plan_bound": (I32, [ctypes.POINTER(VditMaskCfg), VditGrid, I32, ctypes.POINTER(VditKVCache), pS]),
            "vdit_plan_mask": (I32, [ctypes.POINTER(VditMaskCfg), VditGrid, I32, ctypes.POINTER(VditKVCache), I32,
                                     P, SZ, pS, P]),
            "vdit_plan_dynamic_bound": (I32, [ctypes.POINTER(VditMaskCfg), VditGrid, I32,
                                              ctypes.POINTER(VditKVCache), pS]),
            "vdit_plan_dynamic": (I32, [ctypes.POINTER(VditMaskCfg), ctypes.POINTER(VditDynamicCfg), VditTensor,
                                        ctypes.POINTER(VditRopeCfg), VditGrid, I32, ctypes.POINTER(VditKVCache),
                                        P, SZ, P, P, SZ, P]),
            "vdit_plan_dynamic_workspace_bytes": (I32, [ctypes.POINTER(VditMaskCfg), VditGrid, I32,
                                                        ctypes.POINTER(VditKVCache), pS]),
            "vdit_block_attn_fwd": (I32, [VditTensor, ctypes.POINTER(VditRopeCfg), VditGrid, I32,
                                          ctypes.POINTER(VditKVCache), ctypes.POINTER(VditMaskCfg), P,
                                          ctypes.c_float, VditTensor, P, P, SZ, P]),
            "vdit_block_attn_workspace_bytes": (I32, [ctypes.POINTER(VditMaskCfg), VditGrid, I32,
                                                      ctypes.POINTER(VditKVCache), pS]),
            "vdit_block_attn_fwd_static": (I32, [VditTensor, ctypes.POINTER(VditRopeCfg), VditGrid, I32,
                                                 ctypes.POINTER(VditKVCache), ctypes.POINTER(VditMaskCfg), P,
                                                 ctypes.c_float, VditTensor, P, P]),
            "vdit_qkv_rope_append": (I32, [VditTensor, I32, P, ctypes.c_int64, P, ctypes.POINTER(VditRopeCfg),
                                           VditGrid, I32, ctypes.POINTER(VditKVCache), VditTensor, P]),
            "vdit_block_rel_l1": (I32, [P, P, I32, I32, ctypes.c_int64, ctypes.c_int64, P, P, SZ, P]),
            "vdit_block_rel_l1_workspace_bytes": (I32, [I32, ctypes.c_int64, pS]),
            "vdit_reuse_decide": (I32, [ctypes.POINTER(VditReuseCfg), I32, ctypes.c_float, ctypes.POINTER(I32),
                                        P, P]),
        }
        for name in EXPORTS:
            fn = getattr(L, name)
            fn.restype, fn.argtypes = sig[name]
        _lib = L
    return _lib


def _check(status):
    if status != VDIT_OK:
        raise VditError(status, lib().vdit_last_error().decode())


# ---------------------------------------------------------------- marshalling helpers
def grid(frames, height, width) -> VditGrid:
    return VditGrid(frames, height, width)


def mask_cfg(kind, chunk_frames=1, tile=128, radial_w0=13, radial_decay_log2=1, long_range_period=8) -> VditMaskCfg:
    k = MASK_KINDS[kind] if isinstance(kind, str) else int(kind)
    return VditMaskCfg(k, chunk_frames, tile, radial_w0, radial_decay_log2, long_range_period)


def tensor(x) -> VditTensor:
    """[tokens][heads][channels] torch tensor (bf16 / fp32, channels contiguous)."""
    import torch
    if x is None:
        return VditTensor(None, 0, 0, 0, 0)
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("expected a [tokens][heads][channels] tensor with contiguous channels")
    dt = {torch.bfloat16: VDIT_DTYPE_BF16, torch.float32: VDIT_DTYPE_FP32}.get(x.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {x.dtype}")
    return VditTensor(x.data_ptr(), dt, 0, x.stride(0), x.stride(1))


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


# ---------------------------------------------------------------- entry points
def vdit_abi_version() -> int:
    return lib().vdit_abi_version()


def vdit_status_string(status: int) -> str:
    return lib().vdit_status_string(status).decode()


def vdit_last_error() -> str:
    return lib().vdit_last_error().decode()


def vdit_token_positions(g: VditGrid, t0: int, where: int = VDIT_WHERE_HOST, out=None, stream=None):
    n = g.frames * g.height * g.width
    if where == VDIT_WHERE_HOST:
        out = np.zeros((n, 3), np.int32) if out is None else out
        _check(lib().vdit_token_positions(g, t0, where, out.ctypes.data, None))
        return out
    import torch
    out = torch.empty((n, 3), dtype=torch.int32, device="cuda") if out is None else out
    _check(lib().vdit_token_positions(g, t0, where, out.data_ptr(), _stream(stream)))
    return out


def rope_cfg(head_dim, dims, theta, max_t, max_h, max_w, table=None) -> VditRopeCfg:
    return VditRopeCfg(head_dim, dims[0], dims[1], dims[2], float(theta), max_t, max_h, max_w, 0,
                       None if table is None else table.data_ptr())


def vdit_rope_table_build(cfg: VditRopeCfg) -> np.ndarray:
    need = ctypes.c_size_t(0)
    st = lib().vdit_rope_table_build(ctypes.byref(cfg), None, 0, ctypes.byref(need))
    if st not in (VDIT_OK, VDIT_ERR_BUFFER_TOO_SMALL):
        _check(st)
    out = np.zeros(need.value, np.float32)
    _check(lib().vdit_rope_table_build(ctypes.byref(cfg), out.ctypes.data, out.size, ctypes.byref(need)))
    return out


class Rope:
    """RoPE configuration plus its device table (built on the host, copied once)."""

    def __init__(self, head_dim, dims, theta, max_t, max_h, max_w, device="cuda"):
        import torch
        cfg = rope_cfg(head_dim, dims, theta, max_t, max_h, max_w)
        self.host_table = vdit_rope_table_build(cfg)
        self.table = torch.from_numpy(self.host_table).to(device)
        self.cfg = rope_cfg(head_dim, dims, theta, max_t, max_h, max_w, self.table)


def vdit_rope3d_qk(rope: Rope, g: VditGrid, t0: int, heads: int, q=None, k=None, stream=None):
    _check(lib().vdit_rope3d_qk(ctypes.byref(rope.cfg), g, t0, heads, tensor(q), tensor(k), _stream(stream)))


def vdit_kv_cache_bytes(capacity, tokens_per_frame, heads, head_dim):
    kb, vb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().vdit_kv_cache_bytes(capacity, tokens_per_frame, heads, head_dim, ctypes.byref(kb), ctypes.byref(vb)))
    return kb.value, vb.value


class KVCache:
    """Caller-side allocation of the ring cache (torch device memory) and its descriptor."""

    def __init__(self, capacity, tokens_per_frame, heads, head_dim, device="cuda", stream=None):
        import torch
        kb, vb = vdit_kv_cache_bytes(capacity, tokens_per_frame, heads, head_dim)
        self.frame_stride = (tokens_per_frame + 7) // 8 * 8
        self.kv_rows = capacity * self.frame_stride
        self.k = torch.empty(kb // 2, dtype=torch.bfloat16, device=device)
        self.v = torch.empty(vb // 2, dtype=torch.bfloat16, device=device)
        self.slot_dev = torch.empty(capacity, dtype=torch.int32, device=device)
        self.slot_host = np.full(capacity, -1, np.int32)
        self.desc = VditKVCache(self.k.data_ptr(), self.v.data_ptr(), self.slot_dev.data_ptr(),
                                self.slot_host.ctypes.data, capacity, tokens_per_frame, heads, head_dim)
        vdit_kv_cache_reset(self, stream)

    def k_view(self):
        """Keys as [heads][kv_rows][head_dim]."""
        d = self.desc
        return self.k.view(d.heads, self.kv_rows, d.head_dim)

    def v_view(self):
        """Values as stored: [heads][head_dim][kv_rows]."""
        d = self.desc
        return self.v.view(d.heads, d.head_dim, self.kv_rows)


def vdit_kv_cache_reset(cache: KVCache, stream=None):
    _check(lib().vdit_kv_cache_reset(ctypes.byref(cache.desc), _stream(stream)))


def vdit_kv_append(cache: KVCache, rope, g: VditGrid, t0: int, k, v, stream=None):
    rp = ctypes.byref(rope.cfg) if rope is not None else None
    _check(lib().vdit_kv_append(ctypes.byref(cache.desc), rp, g, t0, tensor(k), tensor(v), _stream(stream)))


def vdit_kv_append_plan(cache: KVCache, rope, g: VditGrid, t0: int, k, v, mask: VditMaskCfg, out=None,
                        stream=None):
    """Append of the chunk and the device plan of the same chunk as the query call, in one
    launch; writes `out` (or a new int32 device tensor of the bound size) and returns it."""
    import torch
    bound = vdit_plan_bound(mask, g, t0, cache)
    buf = torch.empty(bound, dtype=torch.int32, device="cuda") if out is None else out
    rp = ctypes.byref(rope.cfg) if rope is not None else None
    used = ctypes.c_size_t(0)
    _check(lib().vdit_kv_append_plan(ctypes.byref(cache.desc), rp, g, t0, tensor(k), tensor(v), ctypes.byref(mask),
                                     buf.data_ptr(), buf.numel(), ctypes.byref(used), _stream(stream)))
    return buf


def vdit_plan_qtiles(mask: VditMaskCfg, g: VditGrid, q_t0: int) -> int:
    n = ctypes.c_int32(0)
    _check(lib().vdit_plan_qtiles(ctypes.byref(mask), g, q_t0, ctypes.byref(n)))
    return n.value


def vdit_plan_bound(mask: VditMaskCfg, g: VditGrid, q_t0: int, cache: KVCache) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vdit_plan_bound(ctypes.byref(mask), g, q_t0, ctypes.byref(cache.desc), ctypes.byref(n)))
    return n.value


def vdit_plan_mask(mask: VditMaskCfg, g: VditGrid, q_t0: int, cache: KVCache, where=VDIT_WHERE_HOST,
                   out=None, stream=None):
    """Host: returns the exact plan (numpy int32).  Device: writes `out` (or a new int32
    device tensor of the bound size) and returns it."""
    bound = vdit_plan_bound(mask, g, q_t0, cache)
    used = ctypes.c_size_t(0)
    if where == VDIT_WHERE_HOST:
        buf = np.zeros(bound, np.int32) if out is None else out
        _check(lib().vdit_plan_mask(ctypes.byref(mask), g, q_t0, ctypes.byref(cache.desc), where,
                                    buf.ctypes.data, buf.size, ctypes.byref(used), None))
        return buf[:used.value]
    import torch
    buf = torch.empty(bound, dtype=torch.int32, device="cuda") if out is None else out
    _check(lib().vdit_plan_mask(ctypes.byref(mask), g, q_t0, ctypes.byref(cache.desc), where,
                                buf.data_ptr(), buf.numel(), ctypes.byref(used), _stream(stream)))
    return buf


def vdit_plan_dynamic_bound(base: VditMaskCfg, g: VditGrid, q_t0: int, cache: KVCache) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vdit_plan_dynamic_bound(ctypes.byref(base), g, q_t0, ctypes.byref(cache.desc), ctypes.byref(n)))
    return n.value


class Workspace:
    """Caller-owned device scratch for the calls that need one (torch memory).  A buffer is
    zeroed when it is allocated, which the attention call's counters require, and is only
    replaced by a larger, zeroed one."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, stream=None):
        """The buffer, replaced by a zeroed one of at least nbytes if it is smaller; a new buffer
        is allocated and zeroed on `stream` (torch's current stream when None), the stream of the
        call that uses it."""
        import torch
        if self.buf is None or self.buf.numel() < nbytes:
            if stream is None:
                st = torch.cuda.current_stream()
            elif isinstance(stream, torch.cuda.Stream):
                st = stream
            else:
                st = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))
            with torch.cuda.stream(st):
                self.buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
        return self.buf

    def ptr_size(self, nbytes: int, stream=None):
        if nbytes == 0:
            return None, 0
        b = self.get(nbytes, stream)
        return b.data_ptr(), b.numel()


def vdit_plan_dynamic_workspace_bytes(base: VditMaskCfg, g: VditGrid, q_t0: int, cache: KVCache) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vdit_plan_dynamic_workspace_bytes(ctypes.byref(base), g, q_t0, ctypes.byref(cache.desc),
                                                   ctypes.byref(n)))
    return n.value


def vdit_plan_dynamic(base: VditMaskCfg, tau: float, q, rope, g: VditGrid, q_t0: int, cache: KVCache,
                      softmax_scale: float = 0.0, out=None, proxies=None, stream=None, workspace=None):
    """Dynamic-threshold plan on the device (int32 tensor of the bound size; `out` reused if
    given); `proxies`: optional fp32 device tensor [n_qtiles][key tiles] that receives them.
    `workspace`: a Workspace (a new one for this call when None)."""
    import torch
    bound = vdit_plan_dynamic_bound(base, g, q_t0, cache)
    buf = torch.empty(bound, dtype=torch.int32, device="cuda") if out is None else out
    dyn = VditDynamicCfg(tau, softmax_scale)
    rp = ctypes.byref(rope.cfg) if rope is not None else None
    ws = Workspace() if workspace is None else workspace
    wp, wn = ws.ptr_size(vdit_plan_dynamic_workspace_bytes(base, g, q_t0, cache), stream)
    _check(lib().vdit_plan_dynamic(ctypes.byref(base), ctypes.byref(dyn), tensor(q), rp, g, q_t0,
                                   ctypes.byref(cache.desc), buf.data_ptr(), buf.numel(),
                                   None if proxies is None else proxies.data_ptr(), wp, wn, _stream(stream)))
    return buf


def dynamic_mask(base: VditMaskCfg) -> VditMaskCfg:
    """The mask to give vdit_block_attn_fwd for a plan made by vdit_plan_dynamic from `base`."""
    m = VditMaskCfg.from_buffer_copy(base)
    m.kind = base.kind | VDIT_MASK_FLAG_DYNAMIC
    return m


def vdit_block_attn_workspace_bytes(mask: VditMaskCfg, g: VditGrid, q_t0: int, cache: KVCache) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vdit_block_attn_workspace_bytes(ctypes.byref(mask), g, q_t0, ctypes.byref(cache.desc),
                                                 ctypes.byref(n)))
    return n.value


def vdit_block_attn_fwd(q, rope, g: VditGrid, q_t0: int, cache: KVCache, mask: VditMaskCfg, plan_dev,
                        softmax_scale: float = 0.0, o=None, lse=None, stream=None, workspace=None):
    """`workspace`: a Workspace (a new, zeroed one for this call when None)."""
    import torch
    o = torch.empty_like(q) if o is None else o
    rp = ctypes.byref(rope.cfg) if rope is not None else None
    ws = Workspace() if workspace is None else workspace
    wp, wn = ws.ptr_size(vdit_block_attn_workspace_bytes(mask, g, q_t0, cache), stream)
    _check(lib().vdit_block_attn_fwd(tensor(q), rp, g, q_t0, ctypes.byref(cache.desc), ctypes.byref(mask),
                                     plan_dev.data_ptr(), ctypes.c_float(softmax_scale), tensor(o),
                                     None if lse is None else lse.data_ptr(), wp, wn, _stream(stream)))
    return o


def vdit_block_attn_fwd_static(q, rope, g: VditGrid, q_t0: int, cache: KVCache, mask: VditMaskCfg, plan_dev,
                               softmax_scale: float = 0.0, o=None, lse=None, stream=None):
    """vdit_block_attn_fwd on the library's static scratch (no workspace, nothing allocated by
    the library; `o` is allocated here when None)."""
    import torch
    o = torch.empty_like(q) if o is None else o
    rp = ctypes.byref(rope.cfg) if rope is not None else None
    _check(lib().vdit_block_attn_fwd_static(tensor(q), rp, g, q_t0, ctypes.byref(cache.desc), ctypes.byref(mask),
                                            plan_dev.data_ptr(), ctypes.c_float(softmax_scale), tensor(o),
                                            None if lse is None else lse.data_ptr(), _stream(stream)))
    return o


def plan_fields(plan):
    """Split plan words (numpy) into (header, qtiles [n,2], row_ptr [n+1], spans [m,2])."""
    p = np.asarray(plan)
    nq, ns, hw = int(p[4]), int(p[5]), PLAN_HEADER_WORDS
    qt = p[hw:hw + 2 * nq].reshape(nq, 2)
    rp = p[hw + 2 * nq:hw + 3 * nq + 1]
    sp = p[hw + 3 * nq + 1:hw + 3 * nq + 1 + 2 * ns].reshape(ns, 2)
    return p[:hw], qt, rp, sp


def vdit_block_rel_l1_workspace_bytes(n_blocks: int, block_elems: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vdit_block_rel_l1_workspace_bytes(n_blocks, block_elems, ctypes.byref(n)))
    return n.value


def vdit_block_rel_l1(cur, prev, out=None, stream=None, workspace=None):
    """Relative L1 distance of every block between two feature sets ([blocks][...] device
    tensors, bf16 or fp32, rows contiguous) and their mean: fp32 tensor [blocks + 1].
    `workspace`: a Workspace (a new one for this call when None)."""
    import torch
    if cur.shape != prev.shape or cur.dtype != prev.dtype:
        raise ValueError("cur and prev must have one shape and dtype")
    nb = cur.shape[0]
    cur2, prev2 = cur.reshape(nb, -1), prev.reshape(nb, -1)
    if cur2.stride(1) != 1 or prev2.stride(1) != 1 or cur2.stride(0) != prev2.stride(0):
        raise ValueError("blocks must be rows with contiguous elements and one stride")
    dt = {torch.bfloat16: VDIT_DTYPE_BF16, torch.float32: VDIT_DTYPE_FP32}.get(cur.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {cur.dtype}")
    out = torch.empty(nb + 1, dtype=torch.float32, device=cur.device) if out is None else out
    stride = cur2.stride(0) if cur2.shape[1] > 0 else 0  # empty blocks: nothing is read
    ws = Workspace(cur.device) if workspace is None else workspace
    b = ws.get(vdit_block_rel_l1_workspace_bytes(nb, cur2.shape[1]), stream)
    _check(lib().vdit_block_rel_l1(cur2.data_ptr(), prev2.data_ptr(), dt, nb, cur2.shape[1], stride,
                                   out.data_ptr(), b.data_ptr(), b.numel(), _stream(stream)))
    return out


class ReuseState:
    """Caller-side state of vdit_reuse_decide: the first reuse step and per-block runs."""

    def __init__(self, n_blocks: int, delta: float, reuse_interval: int, total_steps: int):
        self.cfg = VditReuseCfg(delta, reuse_interval, total_steps, n_blocks)
        self.first_reuse = ctypes.c_int32(-1)
        self.run = (ctypes.c_int32 * n_blocks)()
        self._out = (ctypes.c_uint8 * n_blocks)()

    def decide(self, step: int, mean_rel_l1: float):
        _check(lib().vdit_reuse_decide(ctypes.byref(self.cfg), step, ctypes.c_float(mean_rel_l1),
                                       ctypes.byref(self.first_reuse), ctypes.addressof(self.run),
                                       ctypes.addressof(self._out)))
        return [bool(x) for x in self._out]


def vdit_qkv_rope_append(x, w_qkv, b_qkv, rope, g: VditGrid, t0: int, cache: "KVCache", q_out=None, stream=None):
    """x [tokens][hidden] bf16, w_qkv [3 H D][hidden] bf16, b_qkv fp32 [3 H D] or None (device
    tensors): Q rotated (returned, [tokens][H][D] bf16); K, V appended to `cache`."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1 or w_qkv.dim() != 2 or w_qkv.stride(1) != 1:
        raise ValueError("x and w_qkv must be 2-D with contiguous rows")
    d = cache.desc
    q_out = torch.empty((x.shape[0], d.heads, d.head_dim), dtype=torch.bfloat16, device=x.device) \
        if q_out is None else q_out
    xt = VditTensor(x.data_ptr(), VDIT_DTYPE_BF16 if x.dtype == torch.bfloat16 else -1, 0, x.stride(0), 0)
    rp = ctypes.byref(rope.cfg) if rope is not None else None
    _check(lib().vdit_qkv_rope_append(xt, x.shape[1], w_qkv.data_ptr(), w_qkv.stride(0),
                                      None if b_qkv is None else b_qkv.data_ptr(), rp, g, t0,
                                      ctypes.byref(d), tensor(q_out), _stream(stream)))
    return q_out

