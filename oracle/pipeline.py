"""One attention call of a workload, end to end, float64.

positions (global time index) -> RoPE on Q and on K as it enters the ring ->
ring cache after all appends -> element mask -> masked softmax attention.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention
from .masks import allowed_mask, frame_stride_for, plan_from_mask, query_tiles, serialize_plan
from .ring import RingCache
from .rope3d import rope3d, token_positions


class State:
    pass


def build_state(w, inputs) -> State:
    """Replay the workload's appends (history, then the chunk's own K/V) into a ring."""
    st = State()
    st.w = w
    st.ring = RingCache(w.capacity, w.frame_h, w.frame_w, w.heads, w.head_dim)
    for t0, f, hk, hv in inputs["history"]:
        st.ring.append(hk, hv, f, t0, w.rope_dims, w.theta)
    st.ring.append(inputs["k"], inputs["v"], w.q_frames, w.q_t0, w.rope_dims, w.theta)
    st.q = np.asarray(inputs["q"])
    st.q_pos = token_positions(w.q_frames, w.frame_h, w.frame_w, w.q_t0)
    st.frame_stride = frame_stride_for(w.tokens_per_frame)
    st.k_phys, st.k_t, st.k_s, st.k, st.v = st.ring.keys(st.frame_stride)
    return st


def build_layout(w) -> State:
    """Slot table and key layout only (replays the append schedule without data)."""
    st = State()
    st.w = w
    st.ring = RingCache(w.capacity, w.frame_h, w.frame_w, w.heads, w.head_dim)
    for t0, f in w.appends():
        st.ring.append(None, None, f, t0, w.rope_dims, w.theta)
    st.q_pos = token_positions(w.q_frames, w.frame_h, w.frame_w, w.q_t0)
    st.frame_stride = frame_stride_for(w.tokens_per_frame)
    st.k_phys, st.k_t, st.k_s = st.ring.key_layout(st.frame_stride)
    return st


def q_within_frame(st) -> np.ndarray:
    return np.arange(st.w.n_q, dtype=np.int64) % st.w.tokens_per_frame


def attention_rows(st, head: int, rows=None, scale=None, block: int = 512):
    """O [len(rows), D] and LSE [len(rows)] of one head for the given query rows."""
    w = st.w
    rows = np.arange(w.n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = w.head_dim ** -0.5 if scale is None else scale
    q_rot = rope3d(st.q[rows][:, head:head + 1, :], st.q_pos[rows], w.rope_dims, w.theta)[:, 0, :]
    k = st.k[:, head, :]
    v = st.v[:, head, :]
    q_s = q_within_frame(st)[rows]
    q_t = st.q_pos[rows, 0]
    outs, lses = [], []
    for b in range(0, len(rows), block):
        sl = slice(b, b + block)
        allowed = allowed_mask(w.mask, q_t[sl, None], q_s[sl, None], st.k_t[None, :], st.k_s[None, :])
        o, lse = masked_attention(q_rot[sl], k, v, allowed, scale)
        outs.append(o)
        lses.append(lse)
    if not outs:
        return np.zeros((0, w.head_dim)), np.zeros(0)
    return np.concatenate(outs), np.concatenate(lses)


def plan_for(st) -> np.ndarray:
    """Serialized block plan of the call (int32 words)."""
    w = st.w
    tiles = query_tiles(w.mask, w.q_frames, w.tokens_per_frame, w.q_t0)
    spans = plan_from_mask(w.mask, st.q_pos[:, 0], q_within_frame(st), tiles, st.k_phys, st.k_t, st.k_s)
    return serialize_plan(w.mask, tiles, spans, w.q_t0, w.q_frames, w.tokens_per_frame)
