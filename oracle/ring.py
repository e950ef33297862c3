"""Ring-buffer KV cache indexed by global frame, float64 model.

Sources:
* "Accelerating Video Generation Inference with Sequential-Parallel 3D Positional
  Encoding Using a Global Time Index", section 2.A: the KV cache of causal
  generation keeps the keys and values of frames already produced.
* Wave Forcing / WaveRT page (airadar.tv papers, 2026-11-04), opening paragraph:
  block-causal generation refreshes the cached history once a block is denoised.
* Same Causal-RoPE SP page, section 2.B: positions follow the global time index, so
  a key rotated when its frame is written stays valid for every later chunk.

Model: `capacity` slots of one frame each.  Writing frame t puts its keys (rotated
at their global positions) and values in slot t mod capacity and records t in the
slot table, evicting whatever frame the slot held.  Slot table entry -1 = empty.
The cache's key set is every token of every non-empty slot.
"""
from __future__ import annotations

import numpy as np

from .rope3d import token_positions, rope3d


class RingCache:
    def __init__(self, capacity: int, frame_h: int, frame_w: int, heads: int, head_dim: int):
        self.capacity = capacity
        self.frame_h, self.frame_w = frame_h, frame_w
        self.tokens_per_frame = frame_h * frame_w
        self.heads, self.head_dim = heads, head_dim
        self.slot_frame = np.full(capacity, -1, dtype=np.int64)
        self.k = [None] * capacity  # per slot: [HW, H, D] float64, rotated
        self.v = [None] * capacity

    def slot_of(self, t: int) -> int:
        """Slot of global frame t."""
        return t % self.capacity

    def append(self, k: np.ndarray, v: np.ndarray, frames: int, t0: int, dims, theta, rotate: bool = True):
        """Write `frames` frames starting at global frame t0 (k, v: [frames*HW, H, D])."""
        hw = self.tokens_per_frame
        assert frames <= self.capacity
        if k is None:  # slot bookkeeping only (plan tests need no data)
            for f in range(frames):
                self.slot_frame[self.slot_of(t0 + f)] = t0 + f
            return
        assert k.shape == (frames * hw, self.heads, self.head_dim) and v.shape == k.shape
        k = np.asarray(k, dtype=np.float64)
        if rotate:
            k = rope3d(k, token_positions(frames, self.frame_h, self.frame_w, t0), dims, theta)
        for f in range(frames):
            t = t0 + f
            slot = self.slot_of(t)
            self.slot_frame[slot] = t
            self.k[slot] = k[f * hw:(f + 1) * hw].copy()
            self.v[slot] = np.asarray(v[f * hw:(f + 1) * hw], dtype=np.float64).copy()

    def key_layout(self, frame_stride: int):
        """(phys, t, s) of every cached token in slot order, without data."""
        hw = self.tokens_per_frame
        phys, tt, ss = [], [], []
        for slot in range(self.capacity):
            t = self.slot_frame[slot]
            if t < 0:
                continue
            s = np.arange(hw, dtype=np.int64)
            phys.append(slot * frame_stride + s)
            tt.append(np.full(hw, t, dtype=np.int64))
            ss.append(s)
        if not phys:
            e = np.zeros(0, dtype=np.int64)
            return e, e, e
        return np.concatenate(phys), np.concatenate(tt), np.concatenate(ss)

    def keys(self, frame_stride: int):
        """Cached tokens in slot order.

        Returns (phys, t, s, k, v): physical index slot*frame_stride + s, global
        frame t, within-frame index s, keys [Nk, H, D] and values [Nk, H, D].
        """
        phys, tt, ss = self.key_layout(frame_stride)
        full = [slot for slot in range(self.capacity) if self.slot_frame[slot] >= 0]
        if not full:
            z = np.zeros((0, self.heads, self.head_dim))
            return phys, tt, ss, z, z
        return (phys, tt, ss, np.concatenate([self.k[slot] for slot in full]),
                np.concatenate([self.v[slot] for slot in full]))
