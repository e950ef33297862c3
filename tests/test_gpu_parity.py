"""GPU parity of libvdit against the fp64 oracle, through the C ABI.

Bars: positions, slot tables and plans bit-exact; attention outputs within max-abs 2e-2 and
relative L2 5e-3 (bf16 inputs, fp32 accumulation); full outputs for the reduced workloads,
sampled rows (tile edges, ragged tails, random rows) of sampled heads for the full-size ones,
which run in the same launch configuration as the benchmark.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import get_workload, make_inputs
from video_diffusion_transformer_rope3d_amd import AttentionSession
from video_diffusion_transformer_rope3d_amd import binding as B

from harness import compare, device_plan_words, run_workload, sample_rows, session_for, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "tiny_d128", "small_chunk_pad", "small_radial", "small_dense_d64", "wan13b_chunk_h2",
         "small_stream_radial", "wave_two_chunks"]
LARGE = ["wan13b_chunk", "stream_wrap_straddle", "log_radial", "dense_clip", "stream14b_chunk", "stream_radial_chunk",
         "wan13b_chunk_h14"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ integer parts
def test_positions_device_bit_exact():
    for (f, hgt, wid, t0) in [(3, 4, 6, 5), (3, 30, 52, 396), (21, 30, 52, 0), (2, 10, 13, 401)]:
        got = B.vdit_token_positions(B.grid(f, hgt, wid), t0, B.VDIT_WHERE_DEVICE).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.token_positions(f, hgt, wid, t0).astype(np.int32))


@pytest.mark.parametrize("name", SMALL + LARGE)
def test_device_plan_bit_exact(name):
    _print("device plan", name)
    w = get_workload(name)
    s = session_for(w)
    dt = torch_dtype(w)
    hw = w.tokens_per_frame
    for t0, f in w.appends():  # slot tables only matter: append zeros
        z = torch.zeros((f * hw, w.heads, w.head_dim), dtype=dt, device="cuda")
        s.append(z, z, t0)
    st = oracle.build_layout(w)
    np.testing.assert_array_equal(s.cache.slot_dev.cpu().numpy(), st.ring.slot_frame)
    np.testing.assert_array_equal(s.cache.slot_host, st.ring.slot_frame)
    want = oracle.plan_for(st)  # the full log-radial clip takes the oracle about 20 s
    dev = device_plan_words(s.plan(w.q_frames, w.q_t0, B.VDIT_WHERE_DEVICE))
    host = s.plan(w.q_frames, w.q_t0, B.VDIT_WHERE_HOST)
    np.testing.assert_array_equal(dev, host)
    np.testing.assert_array_equal(dev, want)


# Geometries past the device builder's LDS tables (more than 2048 query tiles, more than
# 16384 (tile, slot) pairs, frames of more than 65535 tokens) and one that fits them but
# needs two rounds of 1024 tiles.  Slot tables are written directly (frames with holes and
# out-of-order slots); no K/V data is needed for a plan.
PLAN_GEOMETRIES = [
    # name, mask kind, chunk frames, frame h, w, capacity, query frames, query t0
    ("pairs_over_table", "log_radial", 1, 16, 20, 128, 64, 40),
    ("tiles_over_table", "dense", 1, 64, 64, 66, 65, 3),
    ("frame_over_16_bits", "chunk_causal", 2, 256, 257, 3, 2, 4),
    ("two_rounds_in_table", "dense", 1, 96, 96, 15, 15, 0),
    ("two_rounds_chunks", "chunk_causal", 3, 96, 96, 15, 15, 2),
]


@pytest.mark.parametrize("geom", PLAN_GEOMETRIES, ids=[g[0] for g in PLAN_GEOMETRIES])
def test_device_plan_large_geometry_equals_host(geom):
    name, kind, cf, fh, fw, cap, qf, qt0 = geom
    _print("device plan geometry", name)
    s = AttentionSession(1, 64, fh, fw, cap, (24, 20, 20), 1e4, max_t=qt0 + qf + cap + 4, mask=kind,
                         chunk_frames=cf)
    rng = np.random.default_rng(len(name))
    table = np.arange(qt0 + qf - cap, qt0 + qf, dtype=np.int32)  # the newest cap frames
    table = np.where(table < 0, -1, table)
    rng.shuffle(table)
    table[rng.random(cap) < 0.2] = -1  # holes
    s.cache.slot_host[:] = table
    s.cache.slot_dev.copy_(torch.from_numpy(table))
    dev = device_plan_words(s.plan(qf, qt0, B.VDIT_WHERE_DEVICE))
    host = s.plan(qf, qt0, B.VDIT_WHERE_HOST)
    assert int(host[4]) > 0 and int(host[5]) > 0
    np.testing.assert_array_equal(dev, host)


def _assert_same_cache(a, b):
    """Both slot tables equal, and the bits of K and V^T of every occupied slot (pad tokens
    included); empty slots hold whatever the allocation held."""
    np.testing.assert_array_equal(b.cache.slot_host, a.cache.slot_host)
    assert torch.equal(b.cache.slot_dev, a.cache.slot_dev)
    fs = a.cache.kv_rows // a.cache.desc.capacity
    ka, kb = a.cache.k_view().view(torch.int16), b.cache.k_view().view(torch.int16)
    va, vb = a.cache.v_view().view(torch.int16), b.cache.v_view().view(torch.int16)
    for slot in np.flatnonzero(a.cache.slot_host >= 0).tolist():
        r = slice(slot * fs, (slot + 1) * fs)
        assert torch.equal(ka[:, r], kb[:, r]), f"K of slot {slot}"
        assert torch.equal(va[:, :, r], vb[:, :, r]), f"V of slot {slot}"


@pytest.mark.parametrize("name", SMALL + LARGE)
def test_append_plan_equals_separate_calls(name):
    """vdit_kv_append_plan: cache contents, both slot tables and plan words equal those of
    vdit_kv_append then vdit_plan_mask; the plan also equals the host plan."""
    _print("append + plan", name)
    w = get_workload(name)
    inp = make_inputs(w)
    dt = torch_dtype(w)
    a, b = session_for(w), session_for(w)
    for t0, f, hk, hv in inp["history"]:
        hk, hv = to_dev(hk, dt), to_dev(hv, dt)
        a.append(hk, hv, t0)
        b.append(hk, hv, t0)
    k, v = to_dev(inp["k"], dt), to_dev(inp["v"], dt)
    a.append(k, v, w.q_t0)
    pa = a.plan(w.q_frames, w.q_t0)
    pb = b.append_plan(k, v, w.q_t0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(device_plan_words(pb), device_plan_words(pa))
    np.testing.assert_array_equal(device_plan_words(pb), b.plan(w.q_frames, w.q_t0, B.VDIT_WHERE_HOST))
    _assert_same_cache(a, b)


@pytest.mark.parametrize("kind,fh,fw,cap,frames", [("dense", 64, 64, 21, 20), ("log_radial", 30, 52, 30, 30)],
                         ids=["tiles_past_table", "pairs_past_table"])
def test_append_plan_past_the_workgroup_tables(kind, fh, fw, cap, frames):
    """Plans past the append launch's plan tables (more than 512 query tiles, more than 6144
    (tile, slot) pairs): the plan workgroup computes the slot ranges inline."""
    _print("append + plan past the tables", kind)
    mk = lambda: AttentionSession(1, 64, fh, fw, cap, (24, 20, 20), 1e4, max_t=2 * cap + frames, mask=kind)
    a, b = mk(), mk()
    g = torch.Generator(device="cuda").manual_seed(5)
    hist = torch.randn((cap * fh * fw, 1, 64), device="cuda", generator=g).to(torch.bfloat16)
    a.append(hist, hist, 0)
    b.append(hist, hist, 0)
    k = torch.randn((frames * fh * fw, 1, 64), device="cuda", generator=g).to(torch.bfloat16)
    a.append(k, k, cap)
    pa = a.plan(frames, cap)
    pb = b.append_plan(k, k, cap)
    torch.cuda.synchronize()
    words = device_plan_words(pb)
    assert int(words[4]) > 512 or int(words[4]) * cap > 6144
    np.testing.assert_array_equal(words, device_plan_words(pa))
    np.testing.assert_array_equal(words, b.plan(frames, cap, B.VDIT_WHERE_HOST))
    _assert_same_cache(a, b)


def test_append_plan_capacity_over_lds_table():
    """Capacity 1100 (beyond the plan workgroup's 1024-slot table): the two-launch path."""
    cap, fh, fw = 1100, 1, 8
    a = AttentionSession(1, 64, fh, fw, cap, (24, 20, 20), 1e4, max_t=cap + 40, mask="chunk_causal", chunk_frames=3)
    b = AttentionSession(1, 64, fh, fw, cap, (24, 20, 20), 1e4, max_t=cap + 40, mask="chunk_causal", chunk_frames=3)
    g = torch.Generator(device="cuda").manual_seed(3)
    hist = torch.randn((cap * fh * fw, 1, 64), device="cuda", generator=g).to(torch.bfloat16)
    a.append(hist, hist, 20)
    b.append(hist, hist, 20)
    k = torch.randn((4 * fh * fw, 1, 64), device="cuda", generator=g).to(torch.bfloat16)
    a.append(k, k, cap + 20)
    pa = a.plan(4, cap + 20)
    pb = b.append_plan(k, k, cap + 20)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(device_plan_words(pb), device_plan_words(pa))
    np.testing.assert_array_equal(device_plan_words(pb), b.plan(4, cap + 20, B.VDIT_WHERE_HOST))
    _assert_same_cache(a, b)


def test_append_of_more_frames_than_threads_updates_every_slot():
    """One append of 300 frames (more than a workgroup's 256 threads) into a 300-slot ring:
    the device slot table equals the host mirror and the oracle's ring."""
    cap, fh, fw, t0 = 300, 2, 4, 17
    s = AttentionSession(1, 64, fh, fw, cap, (24, 20, 20), 1e4, max_t=t0 + cap + 4, mask="dense")
    z = torch.zeros((cap * fh * fw, 1, 64), dtype=torch.bfloat16, device="cuda")
    s.append(z, z, t0)
    ring = oracle.RingCache(cap, fh, fw, 1, 64)
    ring.append(np.zeros((cap * fh * fw, 1, 64)), np.zeros((cap * fh * fw, 1, 64)), cap, t0, (24, 20, 20), 1e4)
    np.testing.assert_array_equal(s.cache.slot_host, ring.slot_frame)
    np.testing.assert_array_equal(s.cache.slot_dev.cpu().numpy(), ring.slot_frame)


# ------------------------------------------------------------------ RoPE and the cache
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_inplace_vs_oracle(dtype):
    rng = np.random.default_rng(7)
    fr, hgt, wid, t0, heads = 3, 30, 52, 396, 3
    x = rng.standard_normal((fr * hgt * wid, heads, 128)).astype(np.float32)
    xd = to_dev(x, dtype)
    exact = xd.float().cpu().numpy().astype(np.float64)  # the values the kernel starts from
    rope = B.Rope(128, (44, 42, 42), 1e4, 400, 30, 52)
    B.vdit_rope3d_qk(rope, B.grid(fr, hgt, wid), t0, heads, q=xd)
    got = xd.float().cpu().numpy()
    ref = oracle.rope3d(exact, oracle.token_positions(fr, hgt, wid, t0), (44, 42, 42), 1e4)
    if dtype == torch.float32:
        assert np.abs(got - ref).max() < 2e-5
    else:  # one bf16 rounding: relative error <= 2^-8 per element
        assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6).all()
        compare(got, ref, what="rope bf16")


@pytest.mark.parametrize("qdt,kdt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.float32, torch.bfloat16)])
def test_rope_q_and_k_in_one_call(qdt, kdt):
    """Q and K rotated by one call: one launch when their dtypes match (K's rows in the grid's
    second row), two otherwise.  K is a strided view (every other token row of a wider buffer,
    heads 3 apart), Q a plain tensor; each must equal the oracle at its own layout."""
    rng = np.random.default_rng(11)
    fr, hgt, wid, t0, heads = 2, 7, 9, 13, 3  # 126 tokens: ragged against the 256-thread blocks
    n = fr * hgt * wid
    q = to_dev(rng.standard_normal((n, heads, 64)).astype(np.float32), qdt)
    wide = to_dev(rng.standard_normal((n, 2 * heads, 64)).astype(np.float32), kdt)
    k = wide[:, :heads]  # token stride 2 * heads * 64, head stride 64
    q0 = q.float().cpu().numpy().astype(np.float64)
    k0 = k.float().cpu().numpy().astype(np.float64)
    rest0 = wide[:, heads:].float().cpu().numpy()
    rope = B.Rope(64, (24, 20, 20), 1e4, 20, hgt, wid)
    B.vdit_rope3d_qk(rope, B.grid(fr, hgt, wid), t0, heads, q=q, k=k)
    pos = oracle.token_positions(fr, hgt, wid, t0)
    for got, start, dt in ((q, q0, qdt), (k, k0, kdt)):
        ref = oracle.rope3d(start, pos, (24, 20, 20), 1e4)
        g = got.float().cpu().numpy()
        if dt == torch.float32:
            assert np.abs(g - ref).max() < 2e-5
        else:
            assert (np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6).all()
    assert np.array_equal(wide[:, heads:].float().cpu().numpy(), rest0)  # the other heads untouched


@pytest.mark.parametrize("same", [False, True])
def test_rope_q_and_k_sharing_memory(same):
    """Q and K whose address ranges overlap take one launch after the other: the two head
    halves of one buffer (disjoint elements) are each rotated once, and Q and K given as the
    same tensor are rotated twice, in order, as two calls would."""
    rng = np.random.default_rng(12)
    fr, hgt, wid, t0, heads = 2, 5, 8, 4, 2
    n = fr * hgt * wid
    buf = to_dev(rng.standard_normal((n, 2 * heads, 64)).astype(np.float32), torch.bfloat16)
    start = buf.float().cpu().numpy().astype(np.float64)
    rope = B.Rope(64, (24, 20, 20), 1e4, 12, hgt, wid)
    pos = oracle.token_positions(fr, hgt, wid, t0)
    if same:
        x = buf[:, :heads]
        B.vdit_rope3d_qk(rope, B.grid(fr, hgt, wid), t0, heads, q=x, k=x)
        once = oracle.rope3d(start[:, :heads], pos, (24, 20, 20), 1e4)
        # the second rotation starts from the first one's bf16 result, as two calls would
        mid = torch.from_numpy(once).to(torch.bfloat16).float().numpy().astype(np.float64)
        ref = oracle.rope3d(mid, pos, (24, 20, 20), 1e4)
        got = buf[:, :heads].float().cpu().numpy()
        # each rounding errs by at most 2^-9 of its value and a rotation keeps a pair's norm,
        # so two roundings stay within 2^-8 of the pair's norm per element (2^-7 with margin)
        pair = np.repeat(np.linalg.norm(ref.reshape(n, heads, 32, 2), axis=3), 2, axis=2)
        assert (np.abs(got - ref) <= pair * 2.0 ** -7 + 1e-6).all()
        assert np.array_equal(buf[:, heads:].float().cpu().numpy(), start[:, heads:])
    else:
        B.vdit_rope3d_qk(rope, B.grid(fr, hgt, wid), t0, heads, q=buf[:, :heads], k=buf[:, heads:])
        ref = np.concatenate([oracle.rope3d(start[:, :heads], pos, (24, 20, 20), 1e4),
                              oracle.rope3d(start[:, heads:], pos, (24, 20, 20), 1e4)], axis=1)
        got = buf.float().cpu().numpy()
        assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6).all()


@pytest.mark.parametrize("name", ["tiny", "small_chunk_pad"])
def test_kv_append_cache_contents(name):
    w = get_workload(name)
    inp = make_inputs(w)
    r = run_workload(w, inp, with_lse=False)
    s = r["session"]
    st = oracle.build_state(w, inp)
    fs = oracle.frame_stride_for(w.tokens_per_frame)
    kc = s.cache.k_view().float().cpu().numpy()  # [H][rows][D]
    vt = s.cache.v_view().float().cpu().numpy()  # [H][D][rows]
    hw = w.tokens_per_frame
    for slot in range(w.capacity):
        if st.ring.slot_frame[slot] < 0:
            continue
        rows = slice(slot * fs, slot * fs + hw)
        k_ref = st.ring.k[slot].transpose(1, 0, 2)  # [H][HW][D]
        got = kc[:, rows, :]
        assert (np.abs(got - k_ref) <= np.abs(k_ref) * 2.0 ** -8 + 2e-6).all(), f"slot {slot} keys"
        v_ref = torch.from_numpy(st.ring.v[slot]).to(torch.bfloat16).float().numpy().transpose(1, 2, 0)
        np.testing.assert_array_equal(vt[:, :, rows], v_ref)  # values: one RNE rounding, bit-exact
        if fs > hw:
            assert (kc[:, slot * fs + hw:(slot + 1) * fs, :] == 0).all()
            assert (vt[:, :, slot * fs + hw:(slot + 1) * fs] == 0).all()


# ------------------------------------------------------------------ attention
def _oracle_rows(w, inp, heads, rows):
    st = oracle.build_state(w, inp)
    out = {}
    for h in heads:
        out[h] = oracle.attention_rows(st, h, rows)
    return out


@pytest.mark.parametrize("name", SMALL)
def test_attention_parity_full(name):
    _print("attention full", name)
    w = get_workload(name)
    inp = make_inputs(w)
    r = run_workload(w, inp)
    o = r["o"].float().cpu().numpy()
    lse = r["lse"].cpu().numpy()
    ref = _oracle_rows(w, inp, range(w.heads), np.arange(w.n_q))
    for h in range(w.heads):
        compare(o[:, h], ref[h][0], what=f"{name} head {h}")
        np.testing.assert_allclose(lse[h], ref[h][1], atol=1e-2, rtol=0)


@pytest.mark.parametrize("name", LARGE)
def test_attention_parity_sampled(name):
    _print("attention sampled", name)
    w = get_workload(name)
    inp = make_inputs(w)
    r = run_workload(w, inp)
    rows = sample_rows(w)
    heads = sorted({0, w.heads // 2, w.heads - 1})
    o = r["o"].float().cpu().numpy()
    lse = r["lse"].cpu().numpy()
    assert np.isfinite(o).all()
    ref = _oracle_rows(w, inp, heads, rows)
    for h in heads:
        compare(o[rows, h], ref[h][0], what=f"{name} head {h}")
        np.testing.assert_allclose(lse[h, rows], ref[h][1], atol=1e-2, rtol=0)


def test_attention_parity_headline_every_row():
    """The benchmark's workload (Wan-1.3B chunk: 12 heads, 4680 queries, 14040 cached keys), in the
    benchmark's launch configuration: every output element and every LSE against the oracle, not
    a sample (the oracle takes about a second per head)."""
    _print("attention every row", "wan13b_chunk")
    w = get_workload("wan13b_chunk")
    inp = make_inputs(w)
    r = run_workload(w, inp)
    o = r["o"].float().cpu().numpy()
    lse = r["lse"].cpu().numpy()
    ref = _oracle_rows(w, inp, range(w.heads), np.arange(w.n_q))
    for h in range(w.heads):
        compare(o[:, h], ref[h][0], what=f"wan13b_chunk every row, head {h}")
        np.testing.assert_allclose(lse[h], ref[h][1], atol=1e-2, rtol=0)


@pytest.mark.parametrize("name", ["small_radial", "small_chunk_pad", "stream_wrap_straddle", "small_stream_radial"])
def test_zero_queries_average_visible_values(name):
    """Q = 0: every visible key gets the same weight, so O = mean of the visible V rows."""
    w = get_workload(name)
    inp = make_inputs(w)
    r = run_workload(w, inp, q_override=np.zeros_like(inp["q"]))
    st = oracle.build_state(w, inp)
    o = r["o"].float().cpu().numpy()
    q_s = np.arange(w.n_q) % w.tokens_per_frame
    rows = sample_rows(w, n_random=32)
    for row in rows:
        vis = oracle.allowed_mask(w.mask, st.q_pos[row, 0], q_s[row], st.k_t, st.k_s)
        want = st.v[vis].mean(axis=0)  # [H, D]
        np.testing.assert_allclose(o[row], want, atol=2e-3, rtol=1e-2, err_msg=f"row {row}")


def test_fused_rope_and_standalone_rope_both_match_the_oracle():
    """Q rotated while the attention kernel loads it, or rotated beforehand by vdit_rope3d_qk and
    passed with rope = NULL: both match the oracle.  The kernel folds the softmax scale into Q
    before rounding it to bf16, so the fused path rounds Q once and the standalone path twice (its
    rotated bf16 Q, then the scaled one): the two agree to the usual bar, not bit for bit."""
    w = get_workload("small_chunk_pad")
    inp = make_inputs(w)
    fused = run_workload(w, inp)
    qd = to_dev(inp["q"], torch.bfloat16)
    B.vdit_rope3d_qk(fused["session"].rope, B.grid(w.q_frames, w.frame_h, w.frame_w), w.q_t0, w.heads, q=qd)
    s = fused["session"]
    o2 = s.attend(qd, w.q_frames, w.q_t0, fused["plan"], rotate=False)
    torch.cuda.synchronize()
    st = oracle.build_state(w, inp)
    a, b = fused["o"].float().cpu().numpy(), o2.float().cpu().numpy()
    for h in range(w.heads):
        ref, _ = oracle.attention_rows(st, h)
        compare(a[:, h], ref, what=f"fused rope, head {h}")
        compare(b[:, h], ref, what=f"standalone rope, head {h}")
        compare(b[:, h], a[:, h], what=f"standalone vs fused, head {h}")


def test_two_streams_with_their_own_workspaces():
    """Two chunks in flight at once on two streams, each with its own session (ring, plan and
    caller-owned workspace, which the library only borrows): append, device plan and attention of
    each match the oracle.  Nothing is synchronised between the two streams' calls."""
    names = ["small_chunk_pad", "small_dense_d64"]  # unit-kernel plans: both use a workspace
    cur = torch.cuda.current_stream()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for name, st in zip(names, streams):
        w = get_workload(name)
        inp = make_inputs(w)
        dt = torch_dtype(w)
        s = session_for(w, stream=st)
        hist = [(t0, to_dev(hk, dt), to_dev(hv, dt)) for t0, f, hk, hv in inp["history"]]
        k, v, q = to_dev(inp["k"], dt), to_dev(inp["v"], dt), to_dev(inp["q"], dt)
        runs.append((w, inp, s, st, hist, k, v, q))
    for w, inp, s, st, hist, k, v, q in runs:
        st.wait_stream(cur)  # the inputs and the session's tables were made on the current stream
    outs = []
    for w, inp, s, st, hist, k, v, q in runs:  # both streams' work is enqueued before either is awaited
        for t0, hk, hv in hist:
            s.append(hk, hv, t0)
        plan = s.append_plan(k, v, w.q_t0)
        outs.append(s.attend(q, w.q_frames, w.q_t0, plan))
    torch.cuda.synchronize()
    for (w, inp, s, st, hist, k, v, q), o in zip(runs, outs):
        assert s.attn_workspace.buf is not None
        st_o = oracle.build_state(w, inp)
        got = o.float().cpu().numpy()
        for h in range(w.heads):
            ref, _ = oracle.attention_rows(st_o, h)
            compare(got[:, h], ref, what=f"{w.name} on its own stream, head {h}")


def test_chunk_by_chunk_equals_whole_call():
    """Three 1-frame calls with global start frames give the 3-frame call's output."""
    w = get_workload("tiny")
    inp = make_inputs(w)
    whole = run_workload(w, inp)["o"]
    s = session_for(w)
    hw = w.tokens_per_frame
    parts = []
    for f in range(3):
        sl = slice(f * hw, (f + 1) * hw)
        s.append(to_dev(inp["k"][sl], torch.float32), to_dev(inp["v"][sl], torch.float32), w.q_t0 + f)
        plan = s.plan(1, w.q_t0 + f)
        parts.append(s.attend(to_dev(inp["q"][sl], torch.float32), 1, w.q_t0 + f, plan))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts), whole)


def test_deterministic():
    w = get_workload("small_radial")
    inp = make_inputs(w)
    a = run_workload(w, inp)
    b = run_workload(w, inp)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])
    assert (device_plan_words(a["plan"]) == device_plan_words(b["plan"])).all()


def test_workspace_reuse_across_shapes_and_streams():
    """One caller workspace serves calls of different shapes: a call whose units are all split
    (2 heads: every unit is merged from partials by counters) leaves its counters at zero, so a
    later call with more (head, query tile) counters, and one with fewer, both give the
    oracle's output; the same workspace on a second stream gives the same output."""
    _print("workspace reuse")
    ws = B.Workspace()
    first = get_workload("small_chunk_pad")
    inp0 = make_inputs(first)
    r0 = run_workload(first, inp0, workspace=ws)
    w = get_workload("wan13b_chunk_h2")
    inp = make_inputs(w)
    r = run_workload(w, inp, workspace=ws)
    rows = sample_rows(w)
    o = r["o"].float().cpu().numpy()
    ref = _oracle_rows(w, inp, range(w.heads), rows)
    for h in range(w.heads):
        compare(o[rows, h], ref[h][0], what=f"after reuse, head {h}")
    again = run_workload(first, inp0, workspace=ws)["o"]
    assert torch.equal(again, r0["o"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the session has no stream of its own: it uses the current one
        o2 = r["session"].attend(r["q"], w.q_frames, w.q_t0, r["plan"])
    torch.cuda.synchronize()
    assert torch.equal(o2, r["o"])


def test_split_stream_path_is_taken():
    """The 14-head Wan-1.3B geometry takes one round of whole units and a split stream on this
    device (the schedule model, with the device's own grid); test_attention_parity_sampled checks
    its outputs, including the last head, whose units are the split ones."""
    from schedule_model import schedule
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    G = max(8, cus // 8 * 8)
    sch = schedule([220] * 19, 14, G)
    if G == 256:
        assert not sch.whole and sch.rounds == 1 and 0 < sch.sk_base < sch.total
    split_heads = {h for (h, k) in sch.nseg}
    assert split_heads and 13 in split_heads or G != 256


@pytest.mark.parametrize("name,corrupt,dyn", [("small_chunk_pad", "magic", False), ("small_chunk_pad", "tiles", False),
                                              ("small_chunk_pad", "span", False), ("small_chunk_pad", "kind", False),
                                              ("small_radial", "magic", False), ("small_radial", "span", False),
                                              ("small_radial", "tile", False), ("small_chunk_pad", "magic", True),
                                              ("small_chunk_pad", "span", True), ("small_chunk_pad", "kind", True),
                                              ("small_chunk_pad", "t0", False), ("small_chunk_pad", "frames", False),
                                              ("small_radial", "t0", False), ("small_chunk_pad", "t0", True)])
def test_rejected_plan_gives_nan_outputs(name, corrupt, dyn):
    """A plan that does not belong to the call (wrong magic, another rule or tile size, another tile
    count, another query start frame or frame count, a span past the cache) is not computed.  The check is in the kernel, which exits normally, so the call returns
    OK; the outputs it did not compute are NaN.  A bad header, or a bad span under the unit
    kernel (every workgroup validates the whole plan), poisons every output; under the tile
    kernel a bad span poisons its own query tile, here tile 0 of every head.  With the dynamic
    flag (the tile kernel behind its schedule kernel, which checks the spans) the same holds."""
    _print("rejected plan", name, corrupt, "dynamic" if dyn else "")
    w = get_workload(name)
    inp = make_inputs(w)
    r = run_workload(w, inp)
    s = r["session"]
    bad = r["plan"].clone()
    if dyn:  # the static plan's words as a dynamic plan of the same rule would carry them
        bad[2] |= B.VDIT_MASK_FLAG_DYNAMIC
    nq = int(bad[4].item())
    if corrupt == "magic":
        bad[0] = 0
    elif corrupt == "tiles":
        bad[4] = nq + 1
    elif corrupt == "kind":  # a plan of another rule: the static plan under the dynamic mask, else another rule
        bad[2] = int(r["plan"][2].item()) if dyn else int(r["plan"][2].item()) ^ 1
    elif corrupt == "tile":
        bad[3] = int(bad[3].item()) // 2
    elif corrupt == "t0":  # a plan built for the call one frame later
        bad[8] = int(bad[8].item()) + 1
    elif corrupt == "frames":  # for a call of one frame more (same tiles and spans otherwise)
        bad[9] = int(bad[9].item()) + 1
    else:  # the first span of tile 0 starts at the end of the cache (8-aligned, outside it)
        bad[12 + 3 * nq + 1] = s.cache.kv_rows
    lse = torch.zeros((w.heads, w.n_q), dtype=torch.float32, device="cuda")
    o = s.attend(r["q"], w.q_frames, w.q_t0, bad, lse=lse, mask=B.dynamic_mask(s.mask) if dyn else None)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    if corrupt == "span" and (w.mask.kind == "log_radial" or dyn):
        q0, ql = (int(x) for x in r["plan"][12:14].tolist())
        assert np.isnan(o[q0:q0 + ql]).all() and np.isnan(lse[:, q0:q0 + ql]).all()
        assert np.isfinite(o[q0 + ql:]).all()
    else:
        assert np.isnan(o).all() and np.isnan(lse).all()


@pytest.mark.parametrize("dyn", [False, True])
def test_query_tile_without_keys(dyn):
    """A plan row with no spans (possible in a hand-made plan) gives O = 0 and LSE = -inf
    for that query tile; every other tile is unchanged (with the dynamic flag: as the same
    kernels compute them on the full plan)."""
    _print("query tile without keys", "dynamic" if dyn else "")
    w = get_workload("small_chunk_pad")
    inp = make_inputs(w)
    r = run_workload(w, inp)
    p = device_plan_words(r["plan"]).copy()
    nq, ns = int(p[4]), int(p[5])
    qt = p[12:12 + 2 * nq].reshape(nq, 2)
    rp = p[12 + 2 * nq:12 + 3 * nq + 1].copy()
    sp = p[12 + 3 * nq + 1:].reshape(ns, 2)
    drop = 1
    keep = np.r_[0:rp[drop], rp[drop + 1]:ns]
    rp2 = rp.copy()
    rp2[drop + 1:] -= rp[drop + 1] - rp[drop]
    hdr = p[:12].copy()
    hdr[5] = len(keep)
    if dyn:  # the words a dynamic plan of the same rule would carry
        hdr[2] |= B.VDIT_MASK_FLAG_DYNAMIC
    words = np.concatenate([hdr, qt.ravel(), rp2, sp[keep].ravel()]).astype(np.int32)
    plan2 = torch.from_numpy(words).to("cuda")
    mask = B.dynamic_mask(r["session"].mask) if dyn else None
    lse = torch.empty((w.heads, w.n_q), dtype=torch.float32, device="cuda")
    o = r["session"].attend(r["q"], w.q_frames, w.q_t0, plan2, lse=lse, mask=mask)
    if dyn:
        ref_plan = r["plan"].clone()
        ref_plan[2] |= B.VDIT_MASK_FLAG_DYNAMIC
        ref_lse = torch.empty_like(lse)
        ref_o = r["session"].attend(r["q"], w.q_frames, w.q_t0, ref_plan, lse=ref_lse, mask=mask)
    else:
        ref_o, ref_lse = r["o"], r["lse"]
    torch.cuda.synchronize()
    rows = slice(int(qt[drop, 0]), int(qt[drop, 0] + qt[drop, 1]))
    assert (o[rows].float() == 0).all()
    assert torch.isneginf(lse[:, rows]).all()
    other = torch.ones(w.n_q, dtype=torch.bool, device="cuda")
    other[rows] = False
    assert torch.equal(o[other], ref_o[other])
    assert torch.equal(lse[:, other], ref_lse[:, other])
