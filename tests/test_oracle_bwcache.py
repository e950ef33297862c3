"""Pins of the block-reuse indicator and policy oracle (oracle/bwcache.py): closed forms of the
relative L1 distance, brute force on a tiny input, an invariant, and hand-derived schedules."""
import math
import os

import numpy as np

from oracle import bwcache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_rel_l1_closed_forms():
    rng = np.random.default_rng(1)
    prev = rng.standard_normal((4, 7, 5))
    np.testing.assert_allclose(bwcache.rel_l1(prev, prev), 0.0, atol=0)
    np.testing.assert_allclose(bwcache.rel_l1(2 * prev, prev), 1.0, rtol=1e-15)
    np.testing.assert_allclose(bwcache.rel_l1(-prev, prev), 2.0, rtol=1e-15)
    np.testing.assert_allclose(bwcache.rel_l1(np.zeros_like(prev), prev), 1.0, rtol=1e-15)
    z = np.zeros((2, 3))
    r = bwcache.rel_l1(np.array([[0.0, 0, 0], [1, 0, 0]]), z)
    assert r[0] == 0.0 and math.isinf(r[1])


def test_rel_l1_brute_force_and_mean():
    rng = np.random.default_rng(2)
    cur, prev = rng.standard_normal((3, 4, 6)), rng.standard_normal((3, 4, 6))
    want = []
    for b in range(3):
        num = den = 0.0
        for i in range(4):
            for j in range(6):
                num += abs(cur[b, i, j] - prev[b, i, j])
                den += abs(prev[b, i, j])
        want.append(num / den)
    np.testing.assert_allclose(bwcache.rel_l1(cur, prev), want, rtol=1e-13)
    assert abs(bwcache.indicator(cur, prev) - sum(want) / 3) < 1e-13


def test_rel_l1_scale_invariant():
    rng = np.random.default_rng(3)
    cur, prev = rng.standard_normal((2, 50)), rng.standard_normal((2, 50))
    np.testing.assert_allclose(bwcache.rel_l1(3.5 * cur, 3.5 * prev), bwcache.rel_l1(cur, prev), rtol=1e-14)


def test_policy_golden_schedules():
    for line in open(os.path.join(GOLDEN, "bwcache_policy.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        nb, delta, r, total, ind, flags = (p.strip() for p in line.split(";"))
        pol = bwcache.ReusePolicy(int(nb), float(delta), int(r), int(total))
        ind = [float(x) for x in ind.split()]
        want = flags.split()
        assert len(ind) == len(want) == int(total)
        got = ["".join("1" if f else "0" for f in pol.decide(step, m)) for step, m in enumerate(ind)]
        assert got == want, (line, got)
