"""Visibility rules and the block plan, integer / boolean.

Sources:
* Wave Forcing / WaveRT page (airadar.tv papers, 2026-11-04), opening paragraph:
  block-causal attention, a block sees itself and the blocks before it.
* "Accelerating Video Generation Inference ... Using a Global Time Index",
  analogy section 2.B and Wave Forcing "Utilisation": blocks of 3 latent frames
  starting at frames 0, 3, 6, ...; so chunk ids are global frame // chunk_frames.
* "DynamicRad: Content-Adaptive Sparse Attention for Long Video Diffusion",
  section 2 ("Estrutura de Janela Radial Logaritmica"): the window width shrinks
  exponentially with temporal distance by a decay factor gamma, and a long-range
  factor lambda keeps distant frames chosen by a periodic rule; "Estrategia de
  Duplo Modo" 1: static-ratio mode keeps a fixed set fixed by the decay state.

Readings: the window is counted in key tiles of `tile` tokens inside a frame,
W(d) = ceil(w0 * gamma**d) with gamma = 2**-decay_log2 at frame distance d; a key
tile is kept when its tile index differs from the query tile's by at most W(d);
d = 0 and (if the period lambda > 0) every d that is a multiple of lambda keep the
whole frame; the rule is symmetric in time (a full clip, no causality).

Streaming log-radial ("log_radial_causal"): the same window at the global frame distance,
restricted to block-causal visibility (a key frame's chunk is not after the query's),
for chunk-wise generation against the ring cache (the Wave Forcing page's block-causal
chunks with the DynamicRad window; the global time index of the Causal-RoPE SP page makes
frame distances between a chunk and cached frames well defined).
"""
from __future__ import annotations

import math
from dataclasses import replace
from fractions import Fraction

import numpy as np

PLAN_MAGIC = 0x54494456  # bytes 'V','D','I','T' little-endian
PLAN_VERSION = 2
KIND_CODE = {"dense": 0, "chunk_causal": 1, "log_radial": 2, "log_radial_causal": 3}


def frame_stride_for(tokens_per_frame: int) -> int:
    """Physical slot pitch of the cache in tokens: tokens_per_frame rounded up to 8."""
    return (tokens_per_frame + 7) // 8 * 8


def radial_window(d: int, w0: int, decay_log2: int) -> int:
    """W(d) = ceil(w0 * (1/2**decay_log2)**d), computed in exact rationals."""
    return math.ceil(Fraction(w0) / Fraction(2) ** (decay_log2 * d))


def allowed_mask(mask, tq, sq, tk, sk) -> np.ndarray:
    """Element mask: may a query at (global frame tq, within-frame index sq) see a key
    at (tk, sk)?  Arguments broadcast (numpy int arrays)."""
    tq, sq, tk, sk = (np.asarray(a, dtype=np.int64) for a in (tq, sq, tk, sk))
    shape = np.broadcast_shapes(tq.shape, sq.shape, tk.shape, sk.shape)
    if mask.kind == "dense":
        return np.ones(shape, dtype=bool)
    if mask.kind == "chunk_causal":
        return np.broadcast_to((tk // mask.chunk_frames) <= (tq // mask.chunk_frames), shape).copy()
    if mask.kind == "log_radial_causal":
        radial = allowed_mask(replace(mask, kind="log_radial"), tq, sq, tk, sk)
        causal = allowed_mask(replace(mask, kind="chunk_causal"), tq, sq, tk, sk)
        return radial & causal
    if mask.kind == "log_radial":
        d = np.abs(tq - tk)
        d_b = np.broadcast_to(d, shape)
        table = np.array([radial_window(dv, mask.radial_w0, mask.radial_decay_log2)
                          for dv in range(int(d.max(initial=0)) + 1)], dtype=np.int64)
        window = table[d_b]
        tile_gap = np.abs(sq // mask.tile - sk // mask.tile)
        keep = (d_b == 0) | (np.broadcast_to(tile_gap, shape) <= window)
        if mask.long_range_period > 0:
            keep |= (d_b % mask.long_range_period) == 0
        return keep
    raise ValueError(mask.kind)


def query_tiles(mask, frames: int, tokens_per_frame: int, t0: int):
    """Query tiles of a call: consecutive `tile`-token pieces of each mask unit.

    Units: the whole call (dense); maximal runs of call frames in the same chunk
    (chunk_causal); each frame (log_radial).  Every row of a tile then has the same
    visible key set.  Returns a list of (q_start, q_len).
    """
    n = frames * tokens_per_frame
    if mask.kind == "dense":
        units = [(0, n)] if n > 0 else []
    elif mask.kind == "chunk_causal":
        units = []
        f = 0
        while f < frames:
            cid = (t0 + f) // mask.chunk_frames
            g = f
            while g < frames and (t0 + g) // mask.chunk_frames == cid:
                g += 1
            units.append((f * tokens_per_frame, (g - f) * tokens_per_frame))
            f = g
    elif mask.kind in ("log_radial", "log_radial_causal"):
        units = [(f * tokens_per_frame, tokens_per_frame) for f in range(frames)]
    else:
        raise ValueError(mask.kind)
    tiles = []
    for start, length in units:
        for off in range(0, length, mask.tile):
            tiles.append((start + off, min(mask.tile, length - off)))
    return tiles


def plan_from_mask(mask, q_t, q_s, qtiles, k_phys, k_t, k_s):
    """Per query tile, the maximal ascending runs of visible physical key indices.

    q_t, q_s: global frame and within-frame index of every query token; k_*: the same
    for every cached key plus its physical index.  Evaluates the element mask for
    every row of the tile, checks the rows agree, and returns
    list over tiles of list of (k_start, k_len).
    """
    order = np.argsort(k_phys, kind="stable")
    k_phys, k_t, k_s = k_phys[order], k_t[order], k_s[order]
    spans_per_tile = []
    for q0, ql in qtiles:
        rows = allowed_mask(mask, q_t[q0:q0 + ql, None], q_s[q0:q0 + ql, None], k_t[None, :], k_s[None, :])
        if not (rows == rows[0:1]).all():
            raise AssertionError("rows of a query tile disagree on visibility")
        vis = k_phys[rows[0]]
        # a run breaks wherever the next visible physical index is not the successor
        cut = np.flatnonzero(np.diff(vis) != 1) + 1
        first = np.concatenate([[0], cut]).astype(np.int64)
        last = np.concatenate([cut, [len(vis)]]).astype(np.int64)
        spans_per_tile.append([(int(vis[a]), int(b - a)) for a, b in zip(first, last) if b > a])
    return spans_per_tile


def serialize_plan(mask, qtiles, spans_per_tile, q_t0: int, q_frames: int, tokens_per_frame: int) -> np.ndarray:
    """Plan as int32 words: header[12], qtile{start,len}[n], row_ptr[n+1], span{start,len}[m].

    header = magic, version, kind code, tile, n_qtiles, n_spans, flops_lo, flops_hi, q_t0,
    q_frames, tokens_per_frame, 0 with flops = sum over tiles and spans of q_len * k_len (the
    number of visible query-key pairs), split into low and high 32-bit words; the next three
    words name the query call the plan was built for.
    """
    nq = len(qtiles)
    ns = sum(len(s) for s in spans_per_tile)
    pairs = sum(ql * sum(kl for _, kl in sp) for (_, ql), sp in zip(qtiles, spans_per_tile))
    words = [PLAN_MAGIC, PLAN_VERSION, KIND_CODE[mask.kind], mask.tile, nq, ns,
             pairs & 0xFFFFFFFF, pairs >> 32, q_t0, q_frames, tokens_per_frame, 0]
    for q0, ql in qtiles:
        words += [q0, ql]
    acc = 0
    words.append(0)
    for sp in spans_per_tile:
        acc += len(sp)
        words.append(acc)
    for sp in spans_per_tile:
        for k0, kl in sp:
            words += [k0, kl]
    return np.array(words, dtype=np.uint32).view(np.int32)
