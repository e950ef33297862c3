"""Seeded synthetic inputs.

Recipe (numpy PCG64):
* chunk tensors: Generator(PCG64(seed)) draws Q, then K, then V, each
  [tokens][heads][head_dim] float32 standard normal, multiplied by data_scale;
* history appends: Generator(PCG64(seed + 100)) draws K then V for each history
  append in order, same shape rule and scale;
* optional spatial low-frequency component (amplitude a): Generator(PCG64(seed + 200))
  draws phases phi, psi ~ U[0, 2*pi) of shape [heads][head_dim] separately for Q, K
  and V; the token at (h, w) of every frame gets
  a * cos(2*pi*h/frame_h + phi) * cos(2*pi*w/frame_w + psi) added (identical across
  frames, so that channels are correlated across frames);
* bf16 workloads round every value to bfloat16 (round to nearest even) once, at
  the end; the returned float32 arrays hold exactly the bf16 values.

Nothing here computes any part of the attention method itself.
"""
from __future__ import annotations

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, scale):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _lowfreq(rng, frames, fh, fw, heads, dim, amp):
    phi = rng.uniform(0.0, 2 * np.pi, size=(heads, dim))
    psi = rng.uniform(0.0, 2 * np.pi, size=(heads, dim))
    hh = np.arange(fh, dtype=np.float64)[:, None, None, None]
    ww = np.arange(fw, dtype=np.float64)[None, :, None, None]
    comp = amp * np.cos(2 * np.pi * hh / fh + phi) * np.cos(2 * np.pi * ww / fw + psi)  # [fh, fw, H, D]
    comp = comp.reshape(fh * fw, heads, dim).astype(np.float32)
    return np.tile(comp, (frames, 1, 1))


def make_inputs(w, with_history: bool = True) -> dict:
    """Inputs for workload `w`.

    Returns dict(q, k, v, history) where q/k/v are float32 [n_q][heads][head_dim] and
    history is a list of (t0, frames, k, v) appended before the chunk.
    """
    hw = w.tokens_per_frame
    shape = (w.n_q, w.heads, w.head_dim)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = _normal(rng, shape, w.data_scale)
    k = _normal(rng, shape, w.data_scale)
    v = _normal(rng, shape, w.data_scale)
    if w.lowfreq_amp:
        rng_lf = np.random.Generator(np.random.PCG64(w.seed + 200))
        for x in (q, k, v):
            x += _lowfreq(rng_lf, w.q_frames, w.frame_h, w.frame_w, w.heads, w.head_dim, w.lowfreq_amp)
    hist = []
    if with_history and w.history:
        rng_h = np.random.Generator(np.random.PCG64(w.seed + 100))
        for t0, f in w.history:
            hs = (f * hw, w.heads, w.head_dim)
            hk = _normal(rng_h, hs, w.data_scale)
            hv = _normal(rng_h, hs, w.data_scale)
            hist.append([t0, f, hk, hv])
    if w.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
        for h in hist:
            h[2], h[3] = bf16_round(h[2]), bf16_round(h[3])
    return dict(q=q, k=k, v=v, history=[tuple(h) for h in hist])
