"""Mutation check of the oracle's pins (CPU only).

Each entry plants one plausible mistake in a copy of oracle/: a dropped term, a wrong
sign, index or operand order, an off-by-one.  The pins of tests/test_oracle_pins.py and
tests/test_oracle_dynamic.py (closed forms, library routines, hand-derived fixtures,
brute force) must fail on every
mutant; a mutant that passes them shows a part of the oracle that nothing external pins.
The mutants run in parallel subprocesses, each in a scratch tree holding the mutated
oracle, the seeded workloads and the pin tests.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ("test_oracle_pins.py", "test_oracle_dynamic.py", "test_oracle_bwcache.py", "test_oracle_projection.py")

# (file under oracle/, original text, mutated text, what the mistake is)
MUTATIONS = [
    # token positions and RoPE
    ("rope3d.py", "return np.stack([t0 + f, s // width, s % width], axis=1)",
     "return np.stack([f, s // width, s % width], axis=1)", "local frame index instead of the global one"),
    ("rope3d.py", "return np.stack([t0 + f, s // width, s % width], axis=1)",
     "return np.stack([t0 + f, s % width, s // width], axis=1)", "h and w swapped"),
    ("rope3d.py", "return np.power(float(theta), -2.0 * j / dim)",
     "return np.power(float(theta), -1.0 * j / dim)", "wrong frequency exponent"),
    ("rope3d.py", "out[:, :, offset:offset + d_a:2] = x_even * c - x_odd * s",
     "out[:, :, offset:offset + d_a:2] = x_even * c + x_odd * s", "sign of the rotation"),
    ("rope3d.py", "out[:, :, offset + 1:offset + d_a:2] = x_even * s + x_odd * c",
     "out[:, :, offset + 1:offset + d_a:2] = x_odd * s + x_even * c", "operands of the odd channel swapped"),
    ("rope3d.py", "offset += d_a", "offset += d_a // 2", "wrong group offset"),
    ("rope3d.py", "for axis, d_a in enumerate(dims):",
     "for axis, d_a in zip((2, 1, 0), dims):", "axis groups in the wrong order"),
    # attention
    ("attention.py", "s = (q @ k.T) * scale", "s = (q @ k.T)", "softmax scale dropped"),
    ("attention.py", "s = np.where(allowed, s, -np.inf)", "s = np.where(allowed, s, 0.0)",
     "masked logits kept at 0"),
    ("attention.py", "o = (p @ v) / np.where(empty, 1.0, l)[:, None]", "o = (p @ v)",
     "no normalisation by the row sum"),
    ("attention.py", "lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))",
     "lse = np.where(empty, -np.inf, np.log(np.where(empty, 1.0, l)))", "row max missing from the LSE"),
    # ring cache
    ("ring.py", "return t % self.capacity", "return (t + 1) % self.capacity", "frame written to the wrong slot"),
    ("ring.py", "self.slot_frame[self.slot_of(t0 + f)] = t0 + f",
     "self.slot_frame[self.slot_of(t0 + f)] = f", "slot table records the local frame"),
    ("ring.py", "k = rope3d(k, token_positions(frames, self.frame_h, self.frame_w, t0), dims, theta)",
     "k = rope3d(k, token_positions(frames, self.frame_h, self.frame_w, 0), dims, theta)",
     "keys rotated at local positions"),
    ("ring.py", "phys.append(slot * frame_stride + s)", "phys.append(slot * hw + s)",
     "physical index ignores the padded frame stride"),
    # visibility rules
    ("masks.py", "return (tokens_per_frame + 7) // 8 * 8", "return tokens_per_frame", "frame stride not padded"),
    ("masks.py", "return math.ceil(Fraction(w0) / Fraction(2) ** (decay_log2 * d))",
     "return math.floor(Fraction(w0) / Fraction(2) ** (decay_log2 * d))", "window rounded down"),
    ("masks.py", "return math.ceil(Fraction(w0) / Fraction(2) ** (decay_log2 * d))",
     "return math.ceil(Fraction(w0) / Fraction(2) ** (decay_log2 * (d + 1)))", "window decays one step early"),
    ("masks.py", "(tk // mask.chunk_frames) <= (tq // mask.chunk_frames)",
     "(tk // mask.chunk_frames) < (tq // mask.chunk_frames)", "a chunk does not see itself"),
    ("masks.py", "(tk // mask.chunk_frames) <= (tq // mask.chunk_frames)", "tk <= tq",
     "frame-causal instead of chunk-causal"),
    ("masks.py", "keep = (d_b == 0) | (np.broadcast_to(tile_gap, shape) <= window)",
     "keep = np.broadcast_to(tile_gap, shape) <= window", "own frame limited to the window"),
    ("masks.py", "keep = (d_b == 0) | (np.broadcast_to(tile_gap, shape) <= window)",
     "keep = (d_b == 0) | (np.broadcast_to(tile_gap, shape) < window)", "window edge excluded"),
    ("masks.py", "keep |= (d_b % mask.long_range_period) == 0", "pass", "long-range frames dropped"),
    # fused QKV projection
    ("projection.py", "    y = x @ w.T\n", "    y = (x @ w.T)[:, ::-1]\n",
     "output features reversed"),
    ("projection.py", "        y = y + np.asarray(b, dtype=np.float64)[None, :]", "        pass", "bias dropped"),
    ("projection.py", "q, k, v = y[:, :hd], y[:, hd:2 * hd], y[:, 2 * hd:3 * hd]",
     "k, q, v = y[:, :hd], y[:, hd:2 * hd], y[:, 2 * hd:3 * hd]", "Q and K rows swapped"),
    ("projection.py", "return (q.reshape(-1, heads, head_dim), k.reshape(-1, heads, head_dim), v.reshape(-1, heads, head_dim))",
     "return (q.reshape(-1, head_dim, heads).transpose(0, 2, 1), k.reshape(-1, heads, head_dim), v.reshape(-1, heads, head_dim))",
     "Q rows channel-major instead of head-major"),
    ("projection.py", "    pos = token_positions(frames, ring.frame_h, ring.frame_w, t0)",
     "    pos = token_positions(frames, ring.frame_h, ring.frame_w, 0)", "Q rotated at local positions"),
    # block-reuse indicator and policy
    ("bwcache.py", "num = np.abs(cur - prev).sum(axis=1)", "num = np.abs(cur).sum(axis=1) - np.abs(prev).sum(axis=1)",
     "difference of norms instead of the norm of the difference"),
    ("bwcache.py", "den = np.abs(prev).sum(axis=1)", "den = np.abs(cur).sum(axis=1)", "normalised by the current features"),
    ("bwcache.py", "and self.run[b] + 1 < self.R", "and self.run[b] < self.R", "one reuse too many per interval"),
    ("bwcache.py", "step >= self.total - self.first_reuse // 2", "step >= self.total - self.first_reuse",
     "protected tail of k steps instead of k / 2"),
    ("bwcache.py", "can = step > 0 and mean_rel_l1 < self.delta", "can = mean_rel_l1 < self.delta",
     "reuse at the first step"),
    ("bwcache.py", "can = False  # activating here", "pass  # activating here",
     "activation inside its own protected tail"),
    ("masks.py", "        return radial & causal", "        return radial",
     "streaming log-radial sees later chunks"),
    ("masks.py", "        return radial & causal", "        return radial & causal & (np.asarray(tk) <= np.asarray(tq))",
     "streaming log-radial cut at the frame instead of the chunk"),
    ("masks.py", 'elif mask.kind in ("log_radial", "log_radial_causal"):', 'elif mask.kind == "log_radial":',
     "streaming log-radial query tiles not per frame"),
    ("masks.py", "tile_gap = np.abs(sq // mask.tile - sk // mask.tile)",
     "tile_gap = np.abs(sq - sk) // mask.tile", "tile distance taken on token indices"),
    # plan
    ("masks.py", "tiles.append((start + off, min(mask.tile, length - off)))",
     "tiles.append((start + off, mask.tile))", "ragged last tile not shortened"),
    ("masks.py", "cut = np.flatnonzero(np.diff(vis) != 1) + 1", "cut = np.flatnonzero(np.diff(vis) > 8) + 1",
     "runs merged across small gaps"),
    ("masks.py", "pairs & 0xFFFFFFFF, pairs >> 32, q_t0", "pairs & 0xFFFF, pairs >> 32, q_t0", "pair count truncated"),
    ("masks.py", "q_t0, q_frames, tokens_per_frame, 0]", "q_frames, q_t0, tokens_per_frame, 0]",
     "call words of the header swapped"),
    ("masks.py", "        acc += len(sp)\n        words.append(acc)", "        words.append(acc)\n        acc += len(sp)",
     "row pointers shifted by one tile"),
    # dynamic-threshold plan
    ("dynamic.py", "p[i, j] = logits[:, idx].mean()", "p[i, j] = logits[:, idx].sum() / len(idx)",
     "logit block summed over the query rows, not averaged"),
    ("dynamic.py", "logits += q_rot[q0:q0 + ql, h, :] @ k_rot[:, h, :].T",
     "logits += q_rot[q0:q0 + ql, h, :] @ k_rot[:, 0, :].T", "every head scored against head 0's keys"),
    ("dynamic.py", "(p - small[:, None]) >= (1.0 - tau) * (big - small)[:, None]",
     "(p - small[:, None]) >= tau * (big - small)[:, None]", "threshold fraction inverted"),
    ("dynamic.py", "c[i, j] = vis.all()", "c[i, j] = True", "candidates ignore the static rule"),
    ("dynamic.py", "while end < n and k_t[order[end]] == t and k_s[order[end]] // tile == piece:",
     "while end < n and k_t[order[end]] == t:", "key tiles are whole frames"),
]


def _run_mutant(i, mutation):
    fname, old, new, what = mutation
    with tempfile.TemporaryDirectory(prefix="oracle_mutant_") as tmp:
        for d in ("oracle", "workloads"):
            shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                            ignore=shutil.ignore_patterns("__pycache__"))
        os.makedirs(os.path.join(tmp, "tests"))
        for f in ("conftest.py",) + PIN_FILES:
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tmp, "tests", f))
        shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))
        path = os.path.join(tmp, "oracle", fname)
        with open(path) as f:
            src = f.read()
        if src.count(old) < 1:
            return i, "stale", f"{what}: text not found in oracle/{fname}"
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                           [os.path.join(tmp, "tests", f) for f in PIN_FILES],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=900)
        last = (r.stdout.strip().splitlines() or [""])[-1]
        if r.returncode == 0:
            return i, "survived", what
        # killed means a pin failed, not that the mutant broke the test collection
        return i, ("killed" if " failed" in last else "broken"), f"{what}: {last}"


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin():
    workers = max(1, min(8, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda a: _run_mutant(*a), enumerate(MUTATIONS)))
    stale = [r for r in results if r[1] == "stale"]
    broken = [r for r in results if r[1] == "broken"]
    survived = [r for r in results if r[1] == "survived"]
    assert not stale, f"mutations no longer apply: {stale}"
    assert not broken, f"mutants that stop the pin tests from running: {broken}"
    assert not survived, f"mutants the pins do not catch: {[r[2] for r in survived]}"
