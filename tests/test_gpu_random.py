"""GPU parity on seeded random geometries: the whole path (history appends into a ring that may
wrap, the chunk's append, the device plan, attention) against the fp64 oracle, every output row
and every LSE, at the same bar as the named workloads.

Each case draws its own heads, head_dim, frame shape (ragged query and key tiles), mask rule
(dense, chunk-causal, log-radial, log-radial within causal chunks), chunk length, ring capacity,
history length (wrapping the ring or not) and dtype.  The calls are small, so on a device with
many CUs the unit kernel takes its stream schedule (units split over workgroups and merged), and
the log-radial rules take the tile kernel.
"""
import numpy as np
import pytest
import torch

from workloads import make_inputs
from workloads.configs import MaskSpec, Workload
from video_diffusion_transformer_rope3d_amd import binding as B

import oracle
from harness import compare, run_workload

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def random_workload(i: int) -> Workload:
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


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_geometry_matches_oracle(case):
    w = random_workload(case)
    print(f"random case {case}: heads {w.heads} d {w.head_dim} frame {w.frame_h}x{w.frame_w} q_frames {w.q_frames} "
          f"t0 {w.q_t0} capacity {w.capacity} history {w.history} mask {w.mask.kind}/{w.mask.chunk_frames} "
          f"w0 {w.mask.radial_w0} period {w.mask.long_range_period} {w.dtype}", flush=True)
    inp = make_inputs(w)
    r = run_workload(w, inp)
    o = r["o"].float().cpu().numpy()
    lse = r["lse"].cpu().numpy()
    st = oracle.build_state(w, inp)
    ref = [oracle.attention_rows(st, h, np.arange(w.n_q)) for h in range(w.heads)]
    for h in range(w.heads):
        compare(o[:, h], ref[h][0], what=f"random case {case} head {h}")
        np.testing.assert_allclose(lse[h], ref[h][1], atol=1e-2, rtol=0)
