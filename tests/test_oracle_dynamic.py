"""Pins of the dynamic-threshold plan oracle (oracle/dynamic.py) against things outside it:
the factorised form of the mean logit (linearity), the static plan it must reduce to, and a
hand-built case whose answer follows from the definition."""
import numpy as np
import pytest

import oracle
from oracle import dynamic
from oracle.masks import plan_from_mask, query_tiles
from workloads import MaskSpec, get_workload, make_inputs


def _state(name):
    w = get_workload(name)
    return oracle.build_state(w, make_inputs(w))


@pytest.mark.parametrize("name", ["small_chunk_pad", "small_radial"])
def test_proxy_equals_the_factorised_mean(name):
    """The mean of a tile pair's logit block equals, by linearity of the mean,
    scale * sum_h <mean of the tile's q_rot, mean of the tile's k_rot>: a different computation
    (pooled vectors, one dot product per head) of the same number."""
    st = _state(name)
    w = st.w
    scale = w.head_dim ** -0.5
    d = dynamic.dynamic_plan(st, tau=0.5)
    q_rot = oracle.rope3d(st.q, st.q_pos, w.rope_dims, w.theta)
    qbar = np.stack([q_rot[q0:q0 + ql].mean(axis=0) for q0, ql in d["qtiles"]])
    kbar = np.stack([st.k[idx].mean(axis=0) for idx in d["ktiles"]])
    want = scale * np.einsum("ihd,jhd->ij", qbar, kbar)
    size = scale * np.einsum("ihd,jhd->ij", np.abs(qbar), np.abs(kbar)) + 1e-300
    assert np.all(np.abs(d["proxies"] - want) <= 1e-12 * np.maximum(size, 1.0))


@pytest.mark.parametrize("name", ["small_chunk_pad", "small_radial", "tiny_d128"])
def test_tau_one_keeps_the_static_plan(name):
    st = _state(name)
    w = st.w
    d = dynamic.dynamic_plan(st, tau=1.0)
    q_s = np.arange(w.n_q) % w.tokens_per_frame
    static = plan_from_mask(w.mask, st.q_pos[:, 0], q_s, query_tiles(w.mask, w.q_frames, w.tokens_per_frame, w.q_t0),
                            st.k_phys, st.k_t, st.k_s)
    assert d["spans"] == static


def test_tau_zero_keeps_the_best_tiles_and_tau_is_monotone():
    st = _state("small_radial")
    d0 = dynamic.dynamic_plan(st, tau=0.0)
    p, cand = d0["proxies"], d0["cand"]
    for i in range(p.shape[0]):
        best = np.flatnonzero(cand[i] & (p[i] == p[i][cand[i]].max()))
        kept = np.concatenate([d0["ktiles"][j] for j in best])
        assert sum(kl for _, kl in d0["spans"][i]) == len(kept)
    prev = None
    for tau in (0.0, 0.1, 0.3, 0.6, 1.0):
        d = dynamic.dynamic_plan(st, tau=tau)
        cover = [set(k for s0, kl in sp for k in range(s0, s0 + kl)) for sp in d["spans"]]
        if prev is not None:
            assert all(a <= b for a, b in zip(prev, cover))
        prev = cover


def test_hand_built_case():
    """Three 15-token frames of keys (pitch 16), one query tile at position 0 (no rotation).
    Queries point along channel 0; frame 1's keys have 3 on channel 0, frame 0's 1, frame
    2's -2 (two heads, the second all zeros).  Proxies: scale * (1, 3, -2) over the tiles
    (frame = tile); tau = 0 keeps frame 1 only, tau = 0.5 keeps the proxies >= 3 - 2.5,
    i.e. frames 0 and 1, which are neighbours in physical order but not adjacent (padding)."""
    D, H = 4, 2
    q = np.zeros((15, H, D))
    q[:, 0, 0] = 1.0
    k = np.zeros((45, H, D))
    for f, val in enumerate((1.0, 3.0, -2.0)):
        k[15 * f:15 * (f + 1), 0, 0] = val
    k_phys = np.concatenate([16 * f + np.arange(15) for f in range(3)])
    k_t = np.repeat(np.arange(3), 15)
    k_s = np.tile(np.arange(15), 3)
    ktiles, _ = dynamic.key_tiles(k_phys, k_t, k_s, 128)
    assert [len(t) for t in ktiles] == [15, 15, 15]
    p = dynamic.proxies(q, np.zeros((15, 3), np.int64), k, [(0, 15)], ktiles, (2, 2, 0), 1e4, 0.5)
    np.testing.assert_allclose(p, [[0.5, 1.5, -1.0]], atol=1e-15)
    cand = np.ones((1, 3), bool)
    assert dynamic.dynamic_spans(p, cand, 0.0, ktiles, k_phys) == [[(16, 15)]]
    assert dynamic.dynamic_spans(p, cand, 0.5, ktiles, k_phys) == [[(0, 15), (16, 15)]]
    cand[0, 1] = False  # the best tile not a candidate: frame 0 is the best of the rest
    assert dynamic.dynamic_spans(p, cand, 0.0, ktiles, k_phys) == [[(0, 15)]]


def test_key_tiles_are_128_token_pieces_of_each_frame():
    """16 x 20 = 320-token frames: pieces of 128, 128 and 64 tokens per cached frame, in
    physical order, each within one frame."""
    st = _state("small_radial")
    ktiles, info = dynamic.key_tiles(st.k_phys, st.k_t, st.k_s, 128)
    frames = len(set(st.k_t.tolist()))
    assert [len(t) for t in ktiles] == [128, 128, 64] * frames
    assert [s for _, s in info] == [0, 128, 256] * frames
    for t in ktiles:
        assert len(set(st.k_t[t].tolist())) == 1
