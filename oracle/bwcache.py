"""Block-wise feature reuse indicator and policy, float64.  Test infrastructure only (see
oracle/__init__.py).

Source: "BWCache: Accelerating Video Diffusion Transformers through Block-Wise Caching",
section 2 (methodology): the dynamic similarity indicator, periodic recomputation and the
protection of the final timesteps.

Definitions (readings where the page is silent are marked):
* relative L1 of block b between consecutive timesteps:
  r_b = sum |F_t[b] - F_{t-1}[b]| / sum |F_{t-1}[b]| over all elements of the block's
  features (reading: 0 when both sums are 0, +inf when only the denominator is);
* indicator: the mean of r_b over all blocks;
* decision at a step: recompute every block at the first step (nothing cached) and inside the
  protected tail; otherwise reuse the cached features of every block when the indicator is
  below delta, except that a block already reused R - 1 times in a row is recomputed
  (periodic recomputation inside the reuse interval R; reading: at most R - 1 consecutive
  reuses, R >= 1, R = 1 never reuses);
* protected tail: when the first reuse happens at step k, the last floor(k / 2) steps are
  always recomputed (reading: k counted from 0, so "step k" is the (k+1)-th step);
* delta is given by the caller (the page adapts it to the scene without a formula).
"""
from __future__ import annotations

import numpy as np


def rel_l1(cur, prev):
    """Per-block relative L1 distance: cur, prev [blocks, ...] -> [blocks] float64."""
    cur = np.asarray(cur, dtype=np.float64).reshape(len(cur), -1)
    prev = np.asarray(prev, dtype=np.float64).reshape(len(prev), -1)
    num = np.abs(cur - prev).sum(axis=1)
    den = np.abs(prev).sum(axis=1)
    out = np.empty(len(cur))
    for b in range(len(cur)):
        if den[b] > 0:
            out[b] = num[b] / den[b]
        else:
            out[b] = 0.0 if num[b] == 0 else np.inf
    return out


def indicator(cur, prev) -> float:
    """Mean over blocks of the relative L1 distance."""
    return float(rel_l1(cur, prev).mean())


class ReusePolicy:
    """The per-step reuse decision with its state (reuse runs per block, first reuse step)."""

    def __init__(self, n_blocks: int, delta: float, reuse_interval: int, total_steps: int):
        self.delta, self.R, self.total = delta, reuse_interval, total_steps
        self.run = [0] * n_blocks  # consecutive reuses of each block so far
        self.first_reuse = -1

    def protected(self, step: int) -> bool:
        return self.first_reuse >= 0 and step >= self.total - self.first_reuse // 2

    def decide(self, step: int, mean_rel_l1: float):
        """Reuse flags of every block at `step` given the latest indicator."""
        can = step > 0 and mean_rel_l1 < self.delta and not self.protected(step)
        if can and self.first_reuse < 0 and step >= self.total - step // 2:
            can = False  # activating here would put this very step inside its protected tail
        flags = [can and self.run[b] + 1 < self.R for b in range(len(self.run))]
        if any(flags) and self.first_reuse < 0:
            self.first_reuse = step
        for b, f in enumerate(flags):
            self.run[b] = self.run[b] + 1 if f else 0
        return flags
