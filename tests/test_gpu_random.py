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
from video_diffusion_transformer_rope3d_amd import binding as B

import oracle
from harness import compare, random_workload, run_workload

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


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
