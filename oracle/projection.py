"""Fused QKV projection with RoPE at the global time index and the K/V cache append, float64.
Test infrastructure only (see oracle/__init__.py).

Source: "Accelerating Video Generation Inference with Sequential-Parallel 3D Positional
Encoding Using a Global Time Index", section 2.C: the QKV projection and the rotary
embedding are one fused operation, with precomputed rotary tables; section 2.B: positions
use the global frame index; section 2.A: keys and values go to the KV cache.

Definition (readings where the page is silent are marked):
* qkv = x W^T + b for the call's tokens x [N, C]; W [3 H D, C] holds the Q rows, then the K
  rows, then the V rows, each block head-major (row h D + d) - reading: the usual packed
  linear-layer layout; b [3 H D] or absent;
* Q and K are rotated by RoPE3D at the tokens' global positions (t0 + f, h, w); V is not;
* Q is returned; K (rotated) and V are written to the ring cache as a K/V append of the
  call's frames (the ring oracle's append).
"""
from __future__ import annotations

import numpy as np

from .rope3d import rope3d, token_positions


def qkv(x, w, b, heads: int, head_dim: int):
    """The projection alone: (q, k, v), each [N, H, D] float64, before any rotation."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = x @ w.T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)[None, :]
    hd = heads * head_dim
    q, k, v = y[:, :hd], y[:, hd:2 * hd], y[:, 2 * hd:3 * hd]
    return (q.reshape(-1, heads, head_dim), k.reshape(-1, heads, head_dim), v.reshape(-1, heads, head_dim))


def qkv_rope_append(x, w, b, ring, frames: int, t0: int, dims, theta):
    """Q rotated at the global positions (returned) and the K/V append of the call's frames
    to `ring` (K rotated by the ring's append)."""
    q, k, v = qkv(x, w, b, ring.heads, ring.head_dim)
    pos = token_positions(frames, ring.frame_h, ring.frame_w, t0)
    ring.append(k, v, frames, t0, dims, theta, rotate=True)
    return rope3d(q, pos, dims, theta)
