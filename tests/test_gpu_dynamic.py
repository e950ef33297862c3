"""GPU parity of the dynamic-threshold plan (vdit_plan_dynamic) and of attention on it.

The keep / drop decision is floating point deciding an integer, so both sides take it at
the kernel's precision: the cache holds the rotated keys in bf16, and the oracle's proxies
here pool those same bf16 values (the oracle's fp64 rotated keys rounded to bf16).

Bars:
* proxies: within 1e-4 of scale * sum_hd |mean q_rot| * mean |k_rot| of the tile pair (the
  size of the terms; fp32 pooling and dot products lose at most about 1e-5 of it);
* the plan's header and query tiles exactly; every key tile kept whole or not at all;
* decisions: exactly the threshold rule applied in float32 to the device's own proxies,
  and equal to the oracle's fp64 decisions except where the oracle's margin from the
  threshold is within 3 proxy tolerances;
* attention on the device plan within the usual max-abs 2e-2 / rel-L2 5e-3 of the
  oracle's masked attention over exactly the keys that plan keeps.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import dynamic
from oracle.masks import KIND_CODE
from workloads import get_workload, make_inputs
from workloads.synth import bf16_round
from video_diffusion_transformer_rope3d_amd import binding as B

from harness import compare, device_plan_words, random_workload, run_workload
from schedule_model import item_start, tile_steps_from_plan, tile_work_list

pytestmark = pytest.mark.gpu

CASES = [("small_chunk_pad", 0.0), ("small_chunk_pad", 0.4), ("small_radial", 0.3), ("small_radial", 1.0),
         ("small_dense_d64", 0.5), ("wan13b_chunk_h2", 0.6), ("tiny", 0.5), ("small_stream_radial", 0.4)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _device_dynamic(w, inp, tau):
    r = run_workload(w, inp)
    s = r["session"]
    g = B.grid(w.q_frames, w.frame_h, w.frame_w)
    tpf = -(-w.tokens_per_frame // w.mask.tile)
    nq = len(oracle.query_tiles(w.mask, w.q_frames, w.tokens_per_frame, w.q_t0))
    prox = torch.full((nq, w.capacity * tpf), float("nan"), dtype=torch.float32, device="cuda")
    plan = B.vdit_plan_dynamic(s.mask, tau, r["q"], s.rope, g, w.q_t0, s.cache, proxies=prox)
    torch.cuda.synchronize()
    return r, plan, prox.cpu().numpy(), tpf


def _oracle_tile_index(st, d, tpf):
    """Device key-tile number (slot * tiles per frame + piece) of each oracle key tile."""
    fs = st.frame_stride
    return np.array([(int(st.k_phys[idx].min()) // fs) * tpf + s0 // st.w.mask.tile for idx, (_, s0) in
                     zip(d["ktiles"], d["kinfo"])])


def _kept_f32(p, cand, tau):
    """The threshold rule in float32, in the kernel's order of operations."""
    p = p.astype(np.float32)
    big = np.where(cand, p, np.float32(-np.inf)).max(axis=1)
    small = np.where(cand, p, np.float32(np.inf)).min(axis=1)
    with np.errstate(invalid="ignore"):
        cut = (np.float32(1.0) - np.float32(tau)) * (big - small)
        return cand & ((p - small[:, None]) >= cut[:, None])


# seeded random geometries (every rule, ragged tiles, ring wrap) with seeded thresholds
RANDOM = [(i, float(np.random.default_rng(40 + i).uniform(0.0, 1.0))) for i in range(100, 108)]


@pytest.mark.parametrize("name,tau", CASES)
def test_dynamic_plan_matches_oracle(name, tau):
    print("dynamic plan", name, tau, flush=True)
    _check_dynamic_plan(get_workload(name), tau)


@pytest.mark.parametrize("case,tau", RANDOM)
def test_dynamic_plan_random_geometry(case, tau):
    w = random_workload(case)
    print("dynamic plan random", case, tau, w, flush=True)
    _check_dynamic_plan(w, tau)


def _check_dynamic_plan(w, tau):
    inp = make_inputs(w)
    r, plan, prox, tpf = _device_dynamic(w, inp, tau)
    st = oracle.build_state(w, inp)
    d = dynamic.dynamic_plan(st, tau)
    jmap = _oracle_tile_index(st, d, tpf)
    scale = w.head_dim ** -0.5
    qtiles, ktiles, cand = d["qtiles"], d["ktiles"], d["cand"]
    # oracle proxies over the cache's bf16 keys, and the size of their terms
    k16 = bf16_round(st.k.astype(np.float32)).astype(np.float64)
    p = dynamic.proxies(st.q, st.q_pos, k16, qtiles, ktiles, w.rope_dims, w.theta, scale)
    q_rot = oracle.rope3d(st.q, st.q_pos, w.rope_dims, w.theta)
    qabs = np.stack([np.abs(q_rot[q0:q0 + ql].mean(axis=0)) for q0, ql in qtiles])
    kabs = np.stack([np.abs(k16[idx]).mean(axis=0) for idx in ktiles])
    tol = 1e-4 * scale * np.einsum("ihd,jhd->ij", qabs, kabs) + 1e-30
    got = prox[:, jmap].astype(np.float64)
    assert np.isfinite(got).all()
    bad = np.abs(got - p) > tol
    assert not bad.any(), f"proxies off at {np.argwhere(bad)[:8].tolist()}: {got[bad][:4]} vs {p[bad][:4]}"
    # plan words: header and query tiles exactly
    words = device_plan_words(plan)
    hdr, qt, rp, sp = B.plan_fields(words)
    assert hdr[0] == B.VDIT_PLAN_MAGIC and hdr[2] == (KIND_CODE[w.mask.kind] | B.VDIT_MASK_FLAG_DYNAMIC)
    assert qt.tolist() == [list(x) for x in qtiles]
    want32 = _kept_f32(prox[:, jmap], cand, tau)
    want64 = dynamic.kept(p, cand, tau)
    big, small = dynamic.spread(p, cand)
    margin = (p - small[:, None]) - (1.0 - tau) * (big - small)[:, None]
    tiles_phys = [set(st.k_phys[idx].tolist()) for idx in ktiles]
    pairs = 0
    for i in range(len(qtiles)):
        cover = set()
        for s0, kl in sp[rp[i]:rp[i + 1]].tolist():
            cover.update(range(s0, s0 + kl))
        have = np.array([t <= cover for t in tiles_phys])
        partial = [j for j, t in enumerate(tiles_phys) if not have[j] and cover & t]
        assert not partial, f"tile {i}: key tiles partly covered {partial}"
        assert np.array_equal(have, want32[i]), f"tile {i}: not the float32 rule on the device proxies"
        diff = np.flatnonzero(have != want64[i])
        band = np.abs(margin[i]) <= 3 * tol[i].max()
        assert band[diff].all(), f"tile {i}: decisions differ from the oracle's outside the band at {diff.tolist()}"
        pairs += qtiles[i][1] * len(cover)
        # spans are maximal runs
        runs = sp[rp[i]:rp[i + 1]]
        assert all(runs[k][0] + runs[k][1] < runs[k + 1][0] for k in range(len(runs) - 1))
    assert int(np.uint32(hdr[6])) + (int(np.uint32(hdr[7])) << 32) == pairs


def test_tau_one_equals_the_static_device_plan():
    w = get_workload("small_radial")
    inp = make_inputs(w)
    r, plan, _, _ = _device_dynamic(w, inp, 1.0)
    a, b = device_plan_words(plan).copy(), device_plan_words(r["plan"]).copy()
    assert a[2] == b[2] | B.VDIT_MASK_FLAG_DYNAMIC
    a[2] = b[2]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,tau", [("small_radial", 0.3), ("small_chunk_pad", 0.4), ("small_dense_d64", 0.5),
                                      ("wan13b_chunk_h2", 0.3)])
def test_attention_on_a_dynamic_plan(name, tau):
    """Attention with the flagged mask on the device's dynamic plan equals the oracle's masked
    attention over exactly the keys the plan keeps."""
    print("attention on dynamic plan", name, tau, flush=True)
    w = get_workload(name)
    _check_attention_on_dynamic(w, tau, split_expected=name == "wan13b_chunk_h2")


@pytest.mark.parametrize("case,tau", RANDOM)
def test_attention_on_a_dynamic_plan_random_geometry(case, tau):
    w = random_workload(case)
    print("attention on dynamic plan random", case, tau, w, flush=True)
    _check_attention_on_dynamic(w, tau, split_expected=False)


def _check_attention_on_dynamic(w, tau, split_expected):
    inp = make_inputs(w)
    r, plan, _, _ = _device_dynamic(w, inp, tau)
    s = r["session"]
    lse = torch.empty((w.heads, w.n_q), dtype=torch.float32, device="cuda")
    o = s.attend(r["q"], w.q_frames, w.q_t0, plan, lse=lse, mask=B.dynamic_mask(s.mask))
    torch.cuda.synchronize()
    hdr, qt, rp, sp = B.plan_fields(device_plan_words(plan))
    st = oracle.build_state(w, inp)
    allowed = np.zeros((w.n_q, len(st.k_phys)), dtype=bool)
    for i, (q0, ql) in enumerate(qt.tolist()):
        keep = np.zeros(len(st.k_phys), dtype=bool)
        for s0, kl in sp[rp[i]:rp[i + 1]].tolist():
            keep |= (st.k_phys >= s0) & (st.k_phys < s0 + kl)
        allowed[q0:q0 + ql] = keep
    q_rot = oracle.rope3d(st.q, st.q_pos, w.rope_dims, w.theta)
    o_gpu = o.float().cpu().numpy()
    for h in range(w.heads):
        ref, ref_lse = oracle.masked_attention(q_rot[:, h], st.k[:, h], st.v[:, h], allowed, w.head_dim ** -0.5)
        compare(o_gpu[:, h], ref, what=f"{w.name} tau {tau} head {h}")
        np.testing.assert_allclose(lse.cpu().numpy()[h], ref_lse, atol=1e-2, rtol=0)
    # the work list the call ran: the host model's, up to the order of equal lengths
    want, _ = tile_work_list(tile_steps_from_plan(qt.tolist(), rp.tolist(), sp.tolist()), w.heads)
    ws = s.attn_workspace.buf.cpu().numpy()
    n_items = int(ws[:4].view(np.int32)[0])
    raw = ws[256:256 + 32 * n_items].view(np.int32).reshape(-1, 8)
    got = [tuple(x) for x in raw[:, :6].tolist()]
    assert sorted(got) == sorted(want)
    rpl, spl = rp.tolist(), sp.tolist()
    for it in raw.tolist():  # each item's first key step located in the plan's spans
        assert tuple(it[6:]) == item_start(rpl, spl, it[0], it[1])
    assert [min(it[2] - it[1], 1023) for it in got] == [min(it[2] - it[1], 1023) for it in want]
    if split_expected:  # long tiles: chunks and their merge are exercised
        assert any(it[5] > 1 for it in got)
