"""Pins of the fused QKV projection oracle (oracle/projection.py) against things outside it:
pure-Python dot products, weights that select input channels (reducing the result to the
pinned RoPE and ring oracles), the bias alone, and linearity in the input."""
import numpy as np

import oracle
from oracle import projection
from oracle.rope3d import rope3d, token_positions


def _ring(heads, d, frames=2, fh=2, fw=3):
    return oracle.RingCache(4, fh, fw, heads, d)


def test_projection_brute_force():
    """qkv[n, part, h, d] = sum_c x[n, c] w[part H D + h D + d, c] + b[...], by loops."""
    rng = np.random.default_rng(1)
    n, c, h, d = 5, 3, 2, 2
    x, w, b = rng.standard_normal((n, c)), rng.standard_normal((3 * h * d, c)), rng.standard_normal(3 * h * d)
    got = projection.qkv(x, w, b, h, d)
    for part in range(3):
        for t in range(n):
            for hh in range(h):
                for dd in range(d):
                    o = part * h * d + hh * d + dd
                    want = sum(x[t, cc] * w[o, cc] for cc in range(c)) + b[o]
                    assert abs(got[part][t, hh, dd] - want) < 1e-12


def test_selection_weights_reduce_to_rope_and_ring():
    """W that copies input channels: Q = x[:, sel_q] rotated, the cache holds x[:, sel_k]
    rotated and x[:, sel_v] as they are."""
    rng = np.random.default_rng(2)
    heads, d, c, frames, t0 = 2, 8, 64, 2, 5
    dims = (4, 2, 2)
    fh, fw = 2, 3
    x = rng.standard_normal((frames * fh * fw, c))
    sel = rng.permutation(c)[:3 * heads * d]
    w = np.zeros((3 * heads * d, c))
    w[np.arange(3 * heads * d), sel] = 1.0
    ring = _ring(heads, d, frames, fh, fw)
    q = projection.qkv_rope_append(x, w, None, ring, frames, t0, dims, 1e4)
    pos = token_positions(frames, fh, fw, t0)
    hd = heads * d
    part = [x[:, sel[i * hd:(i + 1) * hd]].reshape(-1, heads, d) for i in range(3)]
    np.testing.assert_allclose(q, rope3d(part[0], pos, dims, 1e4), atol=1e-13)
    k_rot = rope3d(part[1], pos, dims, 1e4)
    for f in range(frames):
        slot = (t0 + f) % 4
        assert ring.slot_frame[slot] == t0 + f
        np.testing.assert_allclose(ring.k[slot], k_rot[f * 6:(f + 1) * 6], atol=1e-13)
        np.testing.assert_allclose(ring.v[slot], part[2][f * 6:(f + 1) * 6], atol=0)


def test_bias_alone():
    heads, d = 1, 4
    b = np.arange(12, dtype=np.float64) + 1.0
    ring = _ring(heads, d)
    q = projection.qkv_rope_append(np.zeros((12, 3)), np.ones((12, 3)), b, ring, 2, 0, (2, 2, 0), 1e4)
    pos = token_positions(2, 2, 3, 0)
    np.testing.assert_allclose(q, rope3d(np.broadcast_to(b[:4], (12, 1, 4)), pos, (2, 2, 0), 1e4), atol=1e-13)
    np.testing.assert_allclose(ring.v[1], np.broadcast_to(b[8:12], (6, 1, 4)), atol=0)


def test_linear_in_the_input():
    rng = np.random.default_rng(3)
    heads, d, c = 2, 4, 6
    w = rng.standard_normal((3 * heads * d, c))
    x1, x2 = rng.standard_normal((6, c)), rng.standard_normal((6, c))
    outs = []
    for x in (x1, x2, 2.0 * x1 - 0.5 * x2):
        ring = _ring(heads, d, 1)
        q = projection.qkv_rope_append(x, w, None, ring, 1, 3, (2, 2, 0), 1e4)
        outs.append((q, ring.k[3], ring.v[3]))
    for a, b1, c1 in zip(*outs):
        np.testing.assert_allclose(c1, 2.0 * a - 0.5 * b1, atol=1e-12)
