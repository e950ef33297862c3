"""GPU parity of the fused QKV projection + RoPE + K/V append (vdit_qkv_rope_append).

Bar, per element: |gpu - oracle| <= 2^-8 |oracle| + 2 * hidden * 2^-24 * S, S the largest
sum_c |x_c w_c| + |b| of the (one or two rotated) channels feeding the element: one bf16
rounding of the result (2^-9, doubled as a margin) plus the fp32 accumulation bound.  Slot
tables bit-exact, pad tokens zero, untouched slots unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import projection
from video_diffusion_transformer_rope3d_amd import binding as B
from workloads.synth import bf16_round

pytestmark = pytest.mark.gpu

# heads, head_dim, hidden, frame_h, frame_w, frames, t0, capacity, history appends, bias, rope dims
CASES = {
    "small_wrap": (2, 128, 256, 4, 6, 3, 6, 5, [(2, 2), (4, 2)], True, (44, 42, 42)),
    "pad_d64": (4, 64, 128, 3, 5, 2, 3, 4, [(0, 3)], False, (24, 20, 20)),
    "norope": (2, 128, 192, 4, 6, 2, 0, 3, [], True, None),
    "wan13b_chunk": (12, 128, 1536, 30, 52, 3, 6, 21, [(0, 3), (3, 3)], True, (44, 42, 42)),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _inputs(h, d, c, n, bias, seed):
    rng = np.random.default_rng(seed)
    x = bf16_round(rng.standard_normal((n, c)).astype(np.float32))
    w = bf16_round((rng.standard_normal((3 * h * d, c)) / np.sqrt(c)).astype(np.float32))
    b = (0.1 * rng.standard_normal(3 * h * d)).astype(np.float32) if bias else None
    return x, w, b


def _tol(x, w, b, ref, c, rotated):
    s = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    if b is not None:
        s = s + np.abs(b)
    acc = 2.0 * c * 2.0 ** -24 * (2.0 if rotated else 1.0) * s.max()
    return 2.0 ** -8 * np.abs(ref) + acc


@pytest.mark.parametrize("name", list(CASES))
def test_qkv_rope_append_matches_oracle(name):
    print("qkv", name, flush=True)
    _check_case(CASES[name], seed=len(name))


def _random_case(i):
    """Seeded random geometry: heads x head_dim a multiple of 128 (the entry point's rule), hidden a
    multiple of 64, ragged token tiles, earlier appends that may wrap the ring, bias and RoPE on or off."""
    rng = np.random.default_rng(5000 + i)
    d = int(rng.choice([64, 128]))
    h = int(rng.choice([2, 4])) if d == 64 else int(rng.choice([1, 2, 3]))
    c = 64 * int(rng.integers(1, 9))
    fh, fw = int(rng.integers(2, 13)), int(rng.integers(2, 15))
    frames = int(rng.integers(1, 5))
    cap = frames + int(rng.integers(0, 5))
    start, n_hist = int(rng.integers(0, 25)), int(rng.integers(0, cap + 3))
    hist, t = [], start
    while t < start + n_hist:
        f = min(int(rng.integers(1, 4)), start + n_hist - t, cap)
        hist.append((t, f))
        t += f
    dims = None if rng.random() < 0.2 else ((24, 20, 20) if d == 64 else (44, 42, 42))
    return (h, d, c, fh, fw, frames, start + n_hist, cap, hist, bool(rng.random() < 0.5), dims)


@pytest.mark.parametrize("case", range(12))
def test_qkv_rope_append_random_geometry(case):
    geom = _random_case(case)
    print("qkv random", case, geom, flush=True)
    _check_case(geom, seed=300 + case)


def _check_case(geom, seed):
    h, d, c, fh, fw, frames, t0, cap, hist, bias, dims = geom
    hw = fh * fw
    n = frames * hw
    x, w, b = _inputs(h, d, c, n, bias, seed=seed)
    theta = 1e4
    rope = B.Rope(d, dims, theta, t0 + frames + 4, fh, fw) if dims else None
    cache = B.KVCache(cap, hw, h, d)
    ring = oracle.RingCache(cap, fh, fw, h, d)
    rng = np.random.default_rng(99)
    for ht, hf in hist:  # earlier frames through the plain append, both sides
        kk = bf16_round(rng.standard_normal((hf * hw, h, d)).astype(np.float32))
        vv = bf16_round(rng.standard_normal((hf * hw, h, d)).astype(np.float32))
        B.vdit_kv_append(cache, rope, B.grid(hf, fh, fw), ht,
                         torch.from_numpy(kk).cuda().to(torch.bfloat16), torch.from_numpy(vv).cuda().to(torch.bfloat16))
        ring.append(kk, vv, hf, ht, dims or (0, 0, d), theta, rotate=dims is not None)
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    wd = torch.from_numpy(w).cuda().to(torch.bfloat16)
    bd = torch.from_numpy(b).cuda() if b is not None else None
    before_k = cache.k.clone()
    q = B.vdit_qkv_rope_append(xd, wd, bd, rope, B.grid(frames, fh, fw), t0, cache)
    torch.cuda.synchronize()
    if dims:
        q_ref = projection.qkv_rope_append(x, w, b, ring, frames, t0, dims, theta)
    else:  # no rotation: the projection and a plain append
        q_ref, k_raw, v_raw = projection.qkv(x, w, b, h, d)
        ring.append(k_raw, v_raw, frames, t0, (0, 0, d), theta, rotate=False)
    q_got = q.float().cpu().numpy()
    hd = h * d
    tq = _tol(x, w[:hd], None if b is None else b[:hd], q_ref.reshape(n, hd), c, dims is not None).reshape(n, h, d)
    bad = np.abs(q_got - q_ref) > tq
    assert not bad.any(), f"Q off at {np.argwhere(bad)[:5].tolist()}"
    fs = cache.frame_stride
    kc = cache.k.view(h, cap * fs, d).float().cpu().numpy()
    vt = cache.v.view(h, d, cap * fs).float().cpu().numpy()
    tk = _tol(x, w[hd:2 * hd], None if b is None else b[hd:2 * hd], np.zeros((n, hd)), c, dims is not None).max()
    tv = _tol(x, w[2 * hd:], None if b is None else b[2 * hd:], np.zeros((n, hd)), c, False).max()
    assert np.array_equal(cache.slot_dev.cpu().numpy(), ring.slot_frame.astype(np.int32))
    assert np.array_equal(cache.slot_host, ring.slot_frame.astype(np.int32))
    written = {(t0 + f) % cap for f in range(frames)}
    for slot in range(cap):
        if ring.slot_frame[slot] < 0:
            continue
        rows = slice(slot * fs, slot * fs + hw)
        k_ref = ring.k[slot].transpose(1, 0, 2)  # [H, HW, D]
        v_ref = ring.v[slot].transpose(1, 2, 0)  # [H, D, HW]
        if slot in written:
            assert (np.abs(kc[:, rows] - k_ref) <= 2.0 ** -8 * np.abs(k_ref) + tk).all(), f"K slot {slot}"
            assert (np.abs(vt[:, :, rows] - v_ref) <= 2.0 ** -8 * np.abs(v_ref) + tv).all(), f"V slot {slot}"
            if fs > hw:
                assert (kc[:, slot * fs + hw:(slot + 1) * fs] == 0).all() and (vt[:, :, slot * fs + hw:(slot + 1) * fs] == 0).all()
        else:  # earlier appends are untouched
            assert torch.equal(cache.k.view(h, cap * fs, d)[:, rows].cpu(), before_k.view(h, cap * fs, d)[:, rows].cpu())


def test_fused_equals_projection_then_append():
    """The fused call and the unfused sequence (fp32 GEMM rounded to bf16, then vdit_rope3d_qk
    on Q and vdit_kv_append of K, V, which round once more) agree to an ulp or two: the same
    layouts, one rounding less."""
    h, d, c, fh, fw, frames, t0, cap = 2, 128, 256, 4, 6, 2, 4, 3
    n = frames * fh * fw
    x, w, b = _inputs(h, d, c, n, True, seed=7)
    rope = B.Rope(d, (44, 42, 42), 1e4, 12, fh, fw)
    xd, wd, bd = (torch.from_numpy(a).cuda() for a in (x, w, b))
    y = (xd @ wd.T + bd).to(torch.bfloat16)  # fp32 GEMM on bf16-valued data, rounded once
    q1 = y[:, :h * d].reshape(n, h, d).contiguous()
    k1 = y[:, h * d:2 * h * d].reshape(n, h, d).contiguous()
    v1 = y[:, 2 * h * d:].reshape(n, h, d).contiguous()
    c1 = B.KVCache(cap, fh * fw, h, d)
    B.vdit_rope3d_qk(rope, B.grid(frames, fh, fw), t0, h, q=q1)
    B.vdit_kv_append(c1, rope, B.grid(frames, fh, fw), t0, k1, v1)
    c2 = B.KVCache(cap, fh * fw, h, d)
    q2 = B.vdit_qkv_rope_append(xd.to(torch.bfloat16), wd.to(torch.bfloat16), bd, rope, B.grid(frames, fh, fw), t0, c2)
    torch.cuda.synchronize()
    fs, hw = c1.frame_stride, fh * fw
    slots = [(t0 + f) % cap for f in range(frames)]
    pairs = [(q1, q2)]
    for sl in slots:
        rows = slice(sl * fs, sl * fs + hw)
        pairs += [(c1.k_view()[:, rows], c2.k_view()[:, rows]), (c1.v_view()[:, :, rows], c2.v_view()[:, :, rows])]
    for i, (a, bb) in enumerate(pairs):
        a, bb = a.float(), bb.float()
        # the unfused path rounds before rotating: where the rotation cancels, its error is an
        # ulp of the magnitude before the rotation, hence the absolute term
        ulp = 2.0 ** -7 * bb.abs().max().item()
        diff = (a - bb).abs()
        assert (diff <= 2.0 ** -6 * bb.abs() + 2 * ulp).all(), f"pair {i}: {diff.max().item()}"
        assert diff.median().item() <= 2.0 ** -8 * bb.abs().median().item(), f"pair {i}: median"
