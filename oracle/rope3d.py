"""Token positions and 3D rotary position encoding, float64.

Sources:
* "Accelerating Video Generation Inference with Sequential-Parallel 3D Positional
  Encoding Using a Global Time Index", section 2.B (Causal-RoPE SP, "Mecanismo" and
  "Formula"): a token's global time index is its local frame index plus the start
  frame s of the block it belongs to.
* "Timeripple: Accelerating vDiTs by Understanding the Spatio-Temporal Correlations in
  Latent Space", Metodologia 1 ("Codificacao Estruturada"): RoPE splits the channels
  into a group that encodes time and groups that encode the two spatial axes.

Readings where the pages are silent: the groups are laid out [t | h | w] in that
order; inside a group of width d_a, channel pair (2j, 2j+1) is rotated by the angle
p * theta**(-2j/d_a), p being the token's coordinate on that axis (the RoFormer
form of rotary encoding, applied per axis).
"""
from __future__ import annotations

import numpy as np


def token_positions(frames: int, height: int, width: int, t0: int) -> np.ndarray:
    """Global (t, h, w) of every token of a call, int64 [frames*height*width, 3].

    Tokens are ordered frame-major, then row, then column.  t = t0 + local frame
    (the global time index); h and w restart at 0 in every frame.
    """
    n = np.arange(frames * height * width, dtype=np.int64)
    per_frame = height * width
    f = n // per_frame
    s = n % per_frame
    return np.stack([t0 + f, s // width, s % width], axis=1)


def axis_frequencies(dim: int, theta: float) -> np.ndarray:
    """Angular frequency of each channel pair of an axis group of `dim` channels."""
    j = np.arange(dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / dim)


def rope3d(x: np.ndarray, pos: np.ndarray, dims, theta: float) -> np.ndarray:
    """Rotate x [N, H, D] (float64) by the 3D rotary encoding at positions pos [N, 3].

    dims = (d_t, d_h, d_w), each even, summing to D.  Returns a new array.
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.ndim == 3 and pos.shape == (x.shape[0], 3)
    assert sum(dims) == x.shape[2] and all(d % 2 == 0 for d in dims)
    out = x.copy()
    offset = 0
    for axis, d_a in enumerate(dims):
        if d_a == 0:
            continue
        angle = pos[:, axis].astype(np.float64)[:, None] * axis_frequencies(d_a, theta)[None, :]  # [N, d_a/2]
        c = np.cos(angle)[:, None, :]
        s = np.sin(angle)[:, None, :]
        x_even = x[:, :, offset:offset + d_a:2]
        x_odd = x[:, :, offset + 1:offset + d_a:2]
        out[:, :, offset:offset + d_a:2] = x_even * c - x_odd * s
        out[:, :, offset + 1:offset + d_a:2] = x_even * s + x_odd * c
        offset += d_a
    return out
