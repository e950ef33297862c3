"""GPU-side helpers for the tests: run a workload through libvdit and compare with the oracle."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from workloads.configs import MaskSpec, Workload
from video_diffusion_transformer_rope3d_amd import AttentionSession
from video_diffusion_transformer_rope3d_amd import binding as B

# tolerance on attention outputs (bf16 inputs, fp32 accumulation)
MAX_ABS = 2e-2
REL_L2 = 5e-3


def torch_dtype(w):
    return torch.float32 if w.dtype == "fp32" else torch.bfloat16


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def session_for(w, stream=None):
    m = w.mask
    return AttentionSession(w.heads, w.head_dim, w.frame_h, w.frame_w, w.capacity, w.rope_dims, w.theta,
                            max_t=w.rope_max_t + 4, mask=m.kind, chunk_frames=m.chunk_frames, tile=m.tile,
                            radial_w0=m.radial_w0, radial_decay_log2=m.radial_decay_log2,
                            long_range_period=m.long_range_period, stream=stream)


def run_workload(w, inputs, with_lse=True, rotate_q=True, q_override=None, workspace=None):
    """History appends, chunk append, device plan, attention.  Returns a dict of results.
    `workspace`: a binding Workspace for the attention call (the session's own when None)."""
    dt = torch_dtype(w)
    s = session_for(w)
    if workspace is not None:
        s.attn_workspace = workspace
    for t0, f, hk, hv in inputs["history"]:
        s.append(to_dev(hk, dt), to_dev(hv, dt), t0)
    s.append(to_dev(inputs["k"], dt), to_dev(inputs["v"], dt), w.q_t0)
    plan = s.plan(w.q_frames, w.q_t0)
    q = to_dev(inputs["q"] if q_override is None else q_override, dt)
    lse = torch.empty((w.heads, w.n_q), dtype=torch.float32, device="cuda") if with_lse else None
    o = s.attend(q, w.q_frames, w.q_t0, plan, lse=lse, rotate=rotate_q)
    torch.cuda.synchronize()
    return dict(session=s, plan=plan, q=q, o=o, lse=lse)


def device_plan_words(plan_dev):
    p = plan_dev.cpu().numpy()
    nq, ns = int(p[4]), int(p[5])
    return p[:B.PLAN_HEADER_WORDS + 3 * nq + 1 + 2 * ns]


def sample_rows(w, n_random=96, seed=0):
    """Rows covering the first/last rows of several query tiles, the ragged tail and random rows."""
    rng = np.random.default_rng(seed)
    n = w.n_q
    rows = set(range(min(n, 8)))
    rows.update(range(max(0, n - 80), n))
    for t in range(0, n, 128 * 7):
        rows.update(r for r in (t, t + 1, t + 63, t + 64, t + 127) if r < n)
    rows.update(rng.integers(0, n, n_random).tolist())
    return np.array(sorted(rows))


# Every comparison's achieved margins, by test: (test id, what, max-abs, rel-L2, max-abs bar,
# rel-L2 bar).  tests/conftest.py prints the worst ones at the end of the run.
MARGINS = []


def compare(o_gpu, o_ref, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    """Element-wise comparison against the bar; returns (max-abs, rel-L2) and records them."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite GPU output"
    err = float(np.abs(o_gpu - o_ref).max()) if o_gpu.size else 0.0
    rel = float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    MARGINS.append((test, what, err, rel, max_abs, rel_l2))
    assert err <= max_abs and rel <= rel_l2, f"{what}: max-abs {err:.3e} (<= {max_abs}), rel-L2 {rel:.3e} (<= {rel_l2})"
    return err, rel


def random_workload(i: int) -> Workload:
    """Seeded random geometry for the parity tests: heads, head_dim, frame shape (ragged tiles), mask
    rule, chunk length, ring capacity, history (wrapping the ring or not), dtype and data scale."""
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([64, 128]))
    dims = (24, 20, 20) if d == 64 else (44, 42, 42)
    kind = str(rng.choice(["dense", "chunk_causal", "log_radial", "log_radial_causal"]))
    cf = int(rng.integers(1, 4))
    causal = kind in ("chunk_causal", "log_radial_causal")
    q_frames = cf * int(rng.integers(1, 3)) if causal else int(rng.integers(1, 5))
    capacity = q_frames + int(rng.integers(0, 7))
    n_hist = int(rng.integers(0, capacity - q_frames + 5))  # past capacity - q_frames: the ring wraps
    start = int(rng.integers(0, 30))
    history, t = [], start
    while t < start + n_hist:
        f = min(int(rng.integers(1, 4)), start + n_hist - t, capacity)
        history.append((t, f))
        t += f
    mask = MaskSpec(kind, chunk_frames=cf, tile=128, radial_w0=int(rng.integers(1, 6)), radial_decay_log2=1,
                    long_range_period=int(rng.choice([0, 2, 4])))
    return Workload(
        name=f"random_{i}", description="seeded random geometry", heads=int(rng.choice([1, 2, 3, 5])), head_dim=d,
        frame_h=int(rng.integers(2, 25)), frame_w=int(rng.integers(2, 33)), q_frames=q_frames, q_t0=start + n_hist,
        rope_dims=dims, theta=1e4, mask=mask, capacity=capacity, history=tuple(history),
        dtype="fp32" if rng.random() < 0.2 else "bf16", data_scale=float(rng.choice([1.0, 0.3])), seed=9000 + i)
