"""The unit kernel's work schedule, replayed on the host (tests/schedule_model.py): every key
iteration of every unit is computed exactly once, split units are counted with the segments
that actually hold them, and the three paths (rounds only, rounds plus one more round of whole
units, rounds plus a split stream) are all reached by the geometries the GPU tests run."""
import numpy as np
import pytest

import oracle
from workloads import get_workload, make_inputs
import schedule_model as sched
from schedule_model import cover_counts, schedule, units_from_plan


def _units(name):
    w = get_workload(name)
    qt = oracle.query_tiles(w.mask, w.q_frames, w.tokens_per_frame, w.q_t0)
    st = oracle.build_state(w, make_inputs(w))
    q_s = np.arange(w.n_q) % w.tokens_per_frame
    spans = oracle.plan_from_mask(w.mask, st.q_pos[:, 0], q_s, qt, st.k_phys, st.k_t, st.k_s)
    row_ptr = np.cumsum([0] + [len(sp) for sp in spans])
    flat = [s for sp in spans for s in sp]
    return units_from_plan(qt, row_ptr, flat), w.heads


@pytest.mark.parametrize("G", [8, 64, 128, 240, 256, 304, 512])
@pytest.mark.parametrize("iters,heads", [([220] * 18 + [220], 12), ([220] * 18 + [220], 14), ([220] * 18 + [220], 2),
                                         ([512] * 128, 12), ([7, 0, 3, 220, 220, 1], 5), ([220] * 18 + [220], 40)])
def test_every_iteration_is_computed_once(G, iters, heads):
    sch = schedule(iters, heads, G)
    cnt, segs = cover_counts(sch, iters, heads)
    for h in range(heads):
        for k, n in enumerate(iters):
            for i in range(n):
                assert cnt.get((h, k, i), 0) == 1, (G, h, k, i)
    assert sum(cnt.values()) == sch.total
    for (h, k), n in sch.nseg.items():
        assert segs[(h, k)] == n  # the last arriving segment is the one that merges


def test_the_three_paths_on_256_workgroups():
    """On a 256-CU device: the Wan-1.3B chunk runs whole units (one round and one more), 14 heads
    of the same geometry take one round and a split stream (the path that merges partials),
    and 2 heads run as a pure stream."""
    unit_iters = [220] * 19
    wan = schedule(unit_iters, 12, 256)
    assert wan.whole and wan.rounds == 1 and wan.sk_base == wan.total
    h14 = schedule(unit_iters, 14, 256)
    assert not h14.whole and h14.rounds == 1 and 0 < h14.sk_base < h14.total and h14.nseg
    h2 = schedule(unit_iters, 2, 256)
    assert not h2.whole and h2.rounds == 0 and h2.sk_base == 0


@pytest.mark.parametrize("name,heads", [("wan13b_chunk", 12), ("wan13b_chunk_h14", 14), ("wan13b_chunk_h2", 2)])
def test_plan_units_of_the_gpu_workloads(name, heads):
    """The units the model builds from the oracle's plan of the workloads: 18 pairs and the
    72-row last tile, 220 iterations each (14040 keys in 64-key iterations)."""
    units, h = _units(name)
    assert h == heads
    assert [u[2] for u in units] == [220] * 19
    assert [u[1] for u in units] == [True] * 18 + [False]


@pytest.mark.parametrize("heads", [1, 2, 12, 40])
def test_tile_work_list_covers_each_tile_once_within_the_bounds(heads):
    """Chunks of a tile cover its key steps once, in order, with lengths at most L that differ by at
    most one; split chunks of all heads stay below the partial-slot cap and the list below
    n_qtiles + 1024 / heads items (the bounds the workspace size rests on); the list is longest
    first."""
    rng = np.random.default_rng(heads)
    for trial in range(200):
        nq = int(rng.integers(1, 400))
        kind = trial % 4
        if kind == 0:
            steps = rng.integers(0, 600, nq)
        elif kind == 1:  # a few very long tiles among short ones
            steps = np.where(rng.random(nq) < 0.05, rng.integers(300, 5000, nq), rng.integers(0, 20, nq))
        elif kind == 2:
            steps = rng.integers(0, 9, nq)
        else:
            steps = np.full(nq, int(rng.integers(1, 2000)))
        steps = [int(x) for x in steps]
        items, L = sched.tile_work_list(steps, heads)
        assert len(items) <= nq + sched.SPLIT_CAP // heads
        split = [it for it in items if it[3] >= 0]
        assert len(split) * heads < sched.SPLIT_CAP
        assert sorted({it[3] for it in split}) == list(range(len(split)))
        for t in range(nq):
            mine = sorted((it for it in items if it[0] == t), key=lambda it: it[4])
            assert [it[4] for it in mine] == list(range(len(mine)))
            assert mine[0][1] == 0 and mine[-1][2] == steps[t]
            assert all(a[2] == b[1] for a, b in zip(mine, mine[1:]))
            lens = [it[2] - it[1] for it in mine]
            assert max(lens) - min(lens) <= 1 and (len(mine) == 1 or max(lens) <= L)
        lens = [min(it[2] - it[1], 1023) for it in items]
        assert lens == sorted(lens, reverse=True)
