"""Pins for the CPU oracle: each test checks it against something other than itself.

RoPE is pinned to the RoFormer rotary implementation in `transformers` (a library
routine) and to invariants of rotations; attention to torch's
scaled_dot_product_attention in float64 and to closed forms; the global time
index to the chunk-by-chunk == whole-sequence identity; masks and plans to
hand-derived fixtures under tests/golden/ and to brute-force counts.
"""
import os
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.masks import allowed_mask, query_tiles, plan_from_mask, radial_window
from workloads import MaskSpec, get_workload, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ positions
def test_positions_by_enumeration():
    frames, hgt, wid, t0 = 3, 4, 6, 5
    expect = []
    for f in range(frames):
        for h in range(hgt):
            for w in range(wid):
                expect.append([t0 + f, h, w])
    got = oracle.token_positions(frames, hgt, wid, t0)
    assert got.tolist() == expect
    # the tiny workload's tokens sit at global frames 5, 6, 7
    assert sorted(set(got[:, 0].tolist())) == [5, 6, 7]


# ------------------------------------------------------------------ RoPE
def _roformer_rotate(x, pos, dim):
    """Rotate x [N, dim] at integer positions pos [N] with transformers' RoFormer rotary code."""
    from transformers.models.roformer.modeling_roformer import (RoFormerSelfAttention,
                                                                 RoFormerSinusoidalPositionalEmbedding)
    emb = RoFormerSinusoidalPositionalEmbedding(int(pos.max()) + 1, dim)
    emb.weight.data = emb.create_weight()
    table = emb.weight.data.double()  # [P, dim]: sin half then cos half
    sinus = table[torch.as_tensor(pos)][None, None]  # [1, 1, N, dim]
    xt = torch.as_tensor(x, dtype=torch.float64)[None, None]
    rq, _ = RoFormerSelfAttention.apply_rotary_position_embeddings(sinus, xt, xt.clone())
    return rq[0, 0].numpy()


@pytest.mark.parametrize("dims", [(24, 20, 20), (44, 42, 42), (64, 0, 0)])
def test_rope_matches_roformer_per_axis(dims):
    rng = _rng(1)
    n, d = 40, sum(dims)
    x = rng.standard_normal((n, 1, d))
    pos = np.stack([rng.integers(0, 400, n), rng.integers(0, 30, n), rng.integers(0, 52, n)], axis=1)
    got = oracle.rope3d(x, pos, dims, 1e4)[:, 0]
    off = 0
    for axis, d_a in enumerate(dims):
        if d_a:
            ref = _roformer_rotate(x[:, 0, off:off + d_a], pos[:, axis], d_a)
            # the RoFormer table is stored in float32
            np.testing.assert_allclose(got[:, off:off + d_a], ref, atol=2e-5, rtol=0)
        off += d_a


def test_rope_complex_form():
    """Pair (2j, 2j+1) of axis group a, read as x0 + i*x1, is multiplied by exp(i*p*w_j)."""
    rng = _rng(2)
    dims, n = (44, 42, 42), 25
    x = rng.standard_normal((n, 3, 128))
    pos = np.stack([rng.integers(0, 50, n), rng.integers(0, 30, n), rng.integers(0, 52, n)], axis=1)
    got = oracle.rope3d(x, pos, dims, 1e4)
    off = 0
    for axis, d_a in enumerate(dims):
        z = x[:, :, off:off + d_a:2] + 1j * x[:, :, off + 1:off + d_a:2]
        freq = np.array([1e4 ** (-(2.0 * j) / d_a) for j in range(d_a // 2)])
        rot = z * np.exp(1j * pos[:, axis, None, None] * freq[None, None, :])
        np.testing.assert_allclose(got[:, :, off:off + d_a:2], rot.real, atol=1e-12)
        np.testing.assert_allclose(got[:, :, off + 1:off + d_a:2], rot.imag, atol=1e-12)
        off += d_a


def test_rope_invariants():
    rng = _rng(3)
    dims = (44, 42, 42)
    q = rng.standard_normal((64, 2, 128))
    k = rng.standard_normal((64, 2, 128))
    p = np.stack([rng.integers(0, 400, 64), rng.integers(0, 30, 64), rng.integers(0, 52, 64)], axis=1)
    pk = np.stack([rng.integers(0, 400, 64), rng.integers(0, 30, 64), rng.integers(0, 52, 64)], axis=1)
    rq = oracle.rope3d(q, p, dims, 1e4)
    # norm preserved per token and head
    np.testing.assert_allclose(np.linalg.norm(rq, axis=2), np.linalg.norm(q, axis=2), rtol=1e-12)
    # R(0) = identity
    np.testing.assert_array_equal(oracle.rope3d(q, np.zeros_like(p), dims, 1e4), q)
    # q.k depends only on the (t, h, w) offset
    for _ in range(4):
        delta = rng.integers(-50, 50, 3)
        a = (oracle.rope3d(q, p, dims, 1e4) * oracle.rope3d(k, pk, dims, 1e4)).sum(2)
        b = (oracle.rope3d(q, p + delta, dims, 1e4) * oracle.rope3d(k, pk + delta, dims, 1e4)).sum(2)
        np.testing.assert_allclose(a, b, atol=1e-10)
    # each axis drives only its own channel group
    off = 0
    for axis, d_a in enumerate(dims):
        p2 = p.copy()
        p2[:, axis] += 7
        r2 = oracle.rope3d(q, p2, dims, 1e4)
        changed = np.abs(r2 - rq).max(axis=(0, 1)) > 0
        inside = np.zeros(128, bool)
        inside[off:off + d_a] = True
        assert not changed[~inside].any()
        assert changed[inside].all()
        off += d_a


# ------------------------------------------------------------------ attention
def test_dense_attention_matches_torch_sdpa():
    rng = _rng(4)
    q, k, v = rng.standard_normal((37, 64)), rng.standard_normal((53, 64)), rng.standard_normal((53, 48))
    o, lse = oracle.masked_attention(q, k, v, np.ones((37, 53), bool), 64 ** -0.5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None])[0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    ref_lse = torch.logsumexp(torch.tensor(q) @ torch.tensor(k).T * 64 ** -0.5, dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_masked_attention_matches_torch_sdpa_bool_mask():
    rng = _rng(5)
    q, k, v = rng.standard_normal((30, 32)), rng.standard_normal((40, 32)), rng.standard_normal((40, 32))
    allowed = rng.random((30, 40)) < 0.4
    allowed[:, 0] = True
    o, _ = oracle.masked_attention(q, k, v, allowed, 0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None],
        attn_mask=torch.tensor(allowed)[None], scale=0.3)[0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_attention_closed_forms():
    rng = _rng(6)
    nq, nk, d = 20, 33, 16
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    allowed = rng.random((nq, nk)) < 0.5
    allowed[:, 3] = True
    # Q = 0: uniform weights over the visible keys
    o, lse = oracle.masked_attention(np.zeros((nq, d)), k, v, allowed, 0.25)
    for r in range(nq):
        np.testing.assert_allclose(o[r], v[allowed[r]].mean(0), atol=1e-12)
        np.testing.assert_allclose(lse[r], math.log(allowed[r].sum()), atol=1e-12)
    # V = 1: output 1
    o, _ = oracle.masked_attention(q, k, np.ones((nk, d)), allowed, 0.25)
    np.testing.assert_allclose(o, 1.0, atol=1e-12)
    # rows of P sum to one and vanish on hidden keys (V = identity gives O = P)
    p, _ = oracle.masked_attention(q, k, np.eye(nk), allowed, 0.25)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
    assert (p[~allowed] == 0).all() and (p >= 0).all()
    # one visible key: O = that key's value, LSE = its logit
    single = np.zeros((nq, nk), bool)
    single[np.arange(nq), np.arange(nq) % nk] = True
    o, lse = oracle.masked_attention(q, k, v, single, 0.25)
    np.testing.assert_allclose(o, v[np.arange(nq) % nk], atol=1e-12)
    np.testing.assert_allclose(lse, (q * k[np.arange(nq) % nk]).sum(1) * 0.25, atol=1e-12)
    # no visible key: O = 0, LSE = -inf
    o, lse = oracle.masked_attention(q, k, v, np.zeros((nq, nk), bool), 0.25)
    assert (o == 0).all() and np.isneginf(lse).all()


# ------------------------------------------------------------------ global time index
def test_chunk_by_chunk_equals_whole_sequence():
    """Calls of one frame each with global start frames equal one 3-frame call."""
    w = get_workload("tiny")
    inp = make_inputs(w)
    hw, dims = w.tokens_per_frame, w.rope_dims
    mask = w.mask  # 1-frame causal chunks
    scale = w.head_dim ** -0.5

    def call(ring, q, frames, t0):
        phys, kt, ks, kk, vv = ring.keys(oracle.frame_stride_for(hw))
        pos = oracle.token_positions(frames, w.frame_h, w.frame_w, t0)
        qr = oracle.rope3d(q, pos, dims, w.theta)
        out = np.zeros_like(qr)
        s_q = np.arange(frames * hw) % hw
        allowed = allowed_mask(mask, pos[:, 0, None], s_q[:, None], kt[None], ks[None])
        for h in range(w.heads):
            out[:, h], _ = oracle.masked_attention(qr[:, h], kk[:, h], vv[:, h], allowed, scale)
        return out

    whole_ring = oracle.RingCache(w.capacity, w.frame_h, w.frame_w, w.heads, w.head_dim)
    whole_ring.append(inp["k"], inp["v"], 3, w.q_t0, dims, w.theta)
    whole = call(whole_ring, inp["q"], 3, w.q_t0)
    ring = oracle.RingCache(w.capacity, w.frame_h, w.frame_w, w.heads, w.head_dim)
    parts = []
    for f in range(3):
        sl = slice(f * hw, (f + 1) * hw)
        ring.append(inp["k"][sl], inp["v"][sl], 1, w.q_t0 + f, dims, w.theta)
        parts.append(call(ring, inp["q"][sl], 1, w.q_t0 + f))
    np.testing.assert_allclose(np.concatenate(parts), whole, atol=1e-13)
    # dropping the start frame (local indices only) changes the result
    ring2 = oracle.RingCache(w.capacity, w.frame_h, w.frame_w, w.heads, w.head_dim)
    ring2.append(inp["k"][:hw], inp["v"][:hw], 1, 0, dims, w.theta)
    local = call(ring2, inp["q"][:hw], 1, 0)
    assert np.allclose(local, parts[0], atol=1e-13)  # a lone frame only sees itself: offsets unchanged
    sl = slice(hw, 2 * hw)
    ring2.append(inp["k"][sl], inp["v"][sl], 1, 0, dims, w.theta)  # wrong: frame 6 written as frame 0
    bad = call(ring2, inp["q"][sl], 1, 0)
    assert not np.allclose(bad, parts[1], atol=1e-6)


# ------------------------------------------------------------------ ring and masks
def _read_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_ring_slot_tables_golden():
    for line in _read_golden("ring_slots.txt"):
        cap, appends, table = (p.strip() for p in line.split(";"))
        ring = oracle.RingCache(int(cap), 1, 1, 1, 2)
        for a in appends.split():
            t0, f = (int(x) for x in a.split(":"))
            ring.append(None, None, f, t0, (2, 0, 0), 1e4)
        assert ring.slot_frame.tolist() == [int(x) for x in table.split()]


def test_tiny_plan_golden():
    w = get_workload("tiny")
    st = oracle.build_layout(w)
    plan = oracle.plan_for(st)
    nq, ns = plan[4], plan[5]
    qt = plan[12:12 + 2 * nq].reshape(nq, 2)
    rp = plan[12 + 2 * nq:12 + 3 * nq + 1]
    sp = plan[12 + 3 * nq + 1:].reshape(ns, 2)
    rows = _read_golden("tiny_plan.txt")
    assert len(rows) == nq
    for i, line in enumerate(rows):
        head, spans = line.split(":")
        assert [int(x) for x in head.split()] == qt[i].tolist()
        want = [tuple(int(x) for x in s.split()) for s in spans.split(",")]
        assert [tuple(x) for x in sp[rp[i]:rp[i + 1]].tolist()] == want
    assert plan[0] == 0x54494456 and plan[1] == 2 and plan[3] == 128
    assert plan[8:12].tolist() == [5, 3, 24, 0]  # the call: frames 5..7 of 4 x 6 tokens
    pairs = int(plan[6]) + (int(plan[7]) << 32)
    assert pairs == 24 * 24 + 24 * 48 + 24 * 72


def test_radial_window_golden():
    for line in _read_golden("radial_window.txt"):
        d, wd = (int(x) for x in line.split())
        assert radial_window(d, 13, 1) == wd


def test_chunk_causal_reductions():
    rng = _rng(7)
    tq, tk = rng.integers(0, 40, (50, 1)), rng.integers(0, 40, (1, 60))
    s = np.zeros((1, 1), np.int64)
    one = allowed_mask(MaskSpec("chunk_causal", chunk_frames=1), tq, s, tk, s)
    np.testing.assert_array_equal(one, tk <= tq)  # 1-frame chunks: plain frame causality
    big = allowed_mask(MaskSpec("chunk_causal", chunk_frames=64), tq, s, tk, s)
    assert big.all()  # one chunk covering everything: dense
    three = allowed_mask(MaskSpec("chunk_causal", chunk_frames=3), np.array([[6], [7], [8], [9]]), 0,
                         np.array([[5, 6, 8, 9]]), 0)
    assert three.tolist() == [[1, 1, 1, 0], [1, 1, 1, 0], [1, 1, 1, 0], [1, 1, 1, 1]]


def test_log_radial_tile_pair_count_brute_force():
    """Kept (query tile, key tile) pairs of the 21 x 1560-token log-radial clip, by loops."""
    frames, tiles_per_frame, w0, period = 21, 13, 13, 8
    kept = 0
    for i in range(frames):
        for j in range(frames):
            d = abs(i - j)
            wd = math.ceil(Fraction(w0, 2 ** d))
            for a in range(tiles_per_frame):
                for b in range(tiles_per_frame):
                    if d == 0 or d % period == 0 or abs(a - b) <= wd:
                        kept += 1
    assert kept == 30993
    # the oracle's element mask evaluated at tile granularity gives the same count
    tq = np.repeat(np.arange(frames), tiles_per_frame)[:, None]
    sq = (np.tile(np.arange(tiles_per_frame), frames) * 128)[:, None]
    m = allowed_mask(get_workload("log_radial").mask, tq, sq, tq.T, sq.T)
    assert int(m.sum()) == kept


@pytest.mark.parametrize("name", ["tiny", "small_chunk_pad", "small_radial", "small_dense_d64",
                                  "stream_wrap_straddle", "small_stream_radial"])
def test_plan_expands_to_element_mask(name):
    """Spans cover exactly the visible keys of every row of every query tile."""
    w = get_workload(name)
    st = oracle.build_layout(w)
    plan = oracle.plan_for(st)
    nq, ns = plan[4], plan[5]
    qt = plan[12:12 + 2 * nq].reshape(nq, 2)
    rp = plan[12 + 2 * nq:12 + 3 * nq + 1]
    sp = plan[12 + 3 * nq + 1:].reshape(ns, 2)
    assert qt[:, 1].sum() == w.n_q and (qt[:, 1] <= w.mask.tile).all()
    phys_to_key = {int(p): i for i, p in enumerate(st.k_phys)}
    s_q = np.arange(w.n_q) % w.tokens_per_frame
    for i in range(nq):
        q0, ql = qt[i]
        covered = np.zeros(len(st.k_phys), bool)
        for k0, kl in sp[rp[i]:rp[i + 1]]:
            for p in range(k0, k0 + kl):
                covered[phys_to_key[p]] = True
        for r in range(q0, q0 + ql, max(1, ql // 5)):
            row = allowed_mask(w.mask, st.q_pos[r, 0], s_q[r], st.k_t, st.k_s)
            np.testing.assert_array_equal(row, covered)


def test_query_tiles_units():
    m = MaskSpec("chunk_causal", chunk_frames=3)
    tiles = query_tiles(m, 3, 1560, 400)  # frames 400, 401 | 402 straddle a chunk boundary
    assert tiles[0] == (0, 128) and tiles[24] == (3072, 48)
    assert sum(l for _, l in tiles) == 4680
    assert (3120, 128) in tiles
    lr = query_tiles(MaskSpec("log_radial"), 2, 1560, 0)
    assert len(lr) == 26 and lr[12] == (1536, 24) and lr[13] == (1560, 128)


def test_padded_plan_golden():
    """Plans of 15-token frames (pitch 16): spans never merge across the padding."""
    from oracle.masks import frame_stride_for, serialize_plan
    for line in _read_golden("pad_plan.txt"):
        cap, cf, appends, query, tiles = (p.strip() for p in line.split(";"))
        mask = MaskSpec("chunk_causal", chunk_frames=int(cf))
        ring = oracle.RingCache(int(cap), 3, 5, 1, 2)
        for a in appends.split():
            t0, f = (int(x) for x in a.split(":"))
            ring.append(None, None, f, t0, (2, 0, 0), 1e4)
        phys, kt, ks = ring.key_layout(frame_stride_for(15))
        qt0, qf = (int(x) for x in query.split(":"))
        pos = oracle.token_positions(qf, 3, 5, qt0)
        q_s = np.arange(qf * 15) % 15
        qtiles = query_tiles(mask, qf, 15, qt0)
        spans = plan_from_mask(mask, pos[:, 0], q_s, qtiles, phys, kt, ks)
        want_tiles = [t.strip() for t in tiles.split("|")]
        assert len(qtiles) == len(want_tiles)
        for (q0, ql), sp, wt in zip(qtiles, spans, want_tiles):
            head, body = wt.split(":")
            assert [q0, ql] == [int(x) for x in head.split()]
            assert sp == [tuple(int(x) for x in s.split()) for s in body.split(",")]
        words = serialize_plan(mask, qtiles, spans, qt0, qf, 15)
        assert words[8:12].tolist() == [qt0, qf, 15, 0]
        pairs = sum(ql * sum(kl for _, kl in sp) for (_, ql), sp in zip(qtiles, spans))
        assert int(np.uint32(words[6])) + (int(np.uint32(words[7])) << 32) == pairs


def test_plan_pair_count_words_beyond_32_bits():
    """Header words 6, 7 hold the visible-pair count q_len * sum(k_len) in two 32-bit halves."""
    from oracle.masks import serialize_plan
    mask = MaskSpec("dense")
    words = serialize_plan(mask, [(0, 128)], [[(0, 40_000_000), (40_000_008, 5)]], 0, 1, 128)
    pairs = 128 * (40_000_000 + 5)
    assert pairs > 2 ** 32
    assert int(np.uint32(words[6])) == pairs % 2 ** 32 and int(np.uint32(words[7])) == pairs // 2 ** 32
    assert words[4] == 1 and words[5] == 2 and words[8:12].tolist() == [0, 1, 128, 0]
    assert words[12:14].tolist() == [0, 128] and words[14:16].tolist() == [0, 2]


def test_log_radial_own_frame_and_window_edge():
    """Own frame (d = 0) fully visible whatever the window; at distance d the key tiles with
    |tile gap| <= W(d) are kept and the next one is not (token-sized tiles, w0 = 1)."""
    m = MaskSpec("log_radial", tile=1, radial_w0=1, radial_decay_log2=1, long_range_period=0)
    sk = np.arange(40)[None, :]
    own = allowed_mask(m, np.array([[4]]), np.array([[20]]), np.full((1, 40), 4), sk)
    assert own.all()
    m3 = MaskSpec("log_radial", tile=1, radial_w0=3, radial_decay_log2=0, long_range_period=0)  # W(d) = 3
    near = allowed_mask(m3, np.array([[9]]), np.array([[20]]), np.full((1, 40), 10), sk)[0]
    assert np.flatnonzero(near).tolist() == [17, 18, 19, 20, 21, 22, 23]


def test_stream_radial_plan_golden():
    """Streaming log-radial: the window at global frame distance, cut at later chunks."""
    from oracle.masks import frame_stride_for
    mask = MaskSpec("log_radial_causal", chunk_frames=2, tile=2, radial_w0=4, radial_decay_log2=1,
                    long_range_period=0)
    for line in _read_golden("stream_radial_plan.txt"):
        cap, cf, appends, query, tiles = (p.strip() for p in line.split(";"))
        assert int(cf) == mask.chunk_frames
        ring = oracle.RingCache(int(cap), 2, 3, 1, 2)
        for a in appends.split():
            t0, f = (int(x) for x in a.split(":"))
            ring.append(None, None, f, t0, (2, 0, 0), 1e4)
        phys, kt, ks = ring.key_layout(frame_stride_for(6))
        qt0, qf = (int(x) for x in query.split(":"))
        pos = oracle.token_positions(qf, 2, 3, qt0)
        q_s = np.arange(qf * 6) % 6
        qtiles = query_tiles(mask, qf, 6, qt0)
        spans = plan_from_mask(mask, pos[:, 0], q_s, qtiles, phys, kt, ks)
        want = [t.strip() for t in tiles.split("|")]
        assert len(qtiles) == len(want)
        for (q0, ql), sp, wt in zip(qtiles, spans, want):
            head, body = wt.split(":")
            assert [q0, ql] == [int(x) for x in head.split()]
            assert sp == [tuple(int(x) for x in s.split()) for s in body.split(",")]


def test_stream_radial_reductions():
    """One chunk holding every frame gives the plain log-radial rule; a window covering every
    piece with no long-range term gives the chunk-causal rule."""
    rng = np.random.default_rng(5)
    tq, tk = rng.integers(0, 40, (200, 1)), rng.integers(0, 40, (1, 200))
    sq, sk = rng.integers(0, 1560, (200, 1)), rng.integers(0, 1560, (1, 200))
    lr = MaskSpec("log_radial", tile=128, radial_w0=13, radial_decay_log2=1, long_range_period=8)
    big = MaskSpec("log_radial_causal", chunk_frames=1000, tile=128, radial_w0=13, radial_decay_log2=1,
                   long_range_period=8)
    assert np.array_equal(allowed_mask(big, tq, sq, tk, sk), allowed_mask(lr, tq, sq, tk, sk))
    wide = MaskSpec("log_radial_causal", chunk_frames=3, tile=128, radial_w0=1 << 20, radial_decay_log2=0,
                    long_range_period=0)
    cc = MaskSpec("chunk_causal", chunk_frames=3)
    assert np.array_equal(allowed_mask(wide, tq, sq, tk, sk), allowed_mask(cc, tq, sq, tk, sk))
    assert query_tiles(big, 2, 1560, 7) == query_tiles(lr, 2, 1560, 7)
