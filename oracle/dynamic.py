"""Dynamic-threshold block plan, float64.  Test infrastructure only (see oracle/__init__.py).

Source: "DynamicRad: Content-Adaptive Sparse Attention for Long Video Diffusion",
section 2, dual-mode strategy, mode 2 (dynamic threshold): pre-softmax attention logits
serve as importance proxies, an adaptive threshold filters the candidates, and the
candidates are the same structured set the static mode chooses from.

Readings where the page is silent:
* granularity: the plan's query tiles against key tiles, the consecutive `tile`-token
  pieces of each cached frame (the last piece of a frame is ragged);
* proxy: the mean of the pre-softmax logits scale * <q_rot, k_rot> over all query-key
  pairs of a (query tile, key tile), summed over heads so that one plan serves every head.
  `proxies` computes exactly that: the logit block of each tile pair, then its mean (the
  pins check it against the factorised form scale * sum_h <mean q_rot, mean k_rot>, which
  linearity makes equal, and against a hand-built case);
* candidates: the key tiles the static rule of the call lets the query tile see;
* adaptive threshold: per query tile, with M and m the largest and smallest candidate
  proxies, a candidate with proxy p is kept when p - m >= (1 - tau) * (M - m), tau in
  [0, 1] (the same as p >= M - tau * (M - m), written so that tau = 1 keeps every
  candidate and tau = 0 exactly the best ones whatever the rounding);
* the kept key tiles become maximal runs of physical key indices, as in the static plan.
"""
from __future__ import annotations

import numpy as np

from .masks import allowed_mask, query_tiles
from .rope3d import rope3d


def key_tiles(k_phys, k_t, k_s, tile: int):
    """Key tiles of the cache in physical order: list of index arrays into the key list
    (keys sorted by physical index), and each tile's (frame t, first within-frame index)."""
    order = np.argsort(k_phys, kind="stable")
    tiles, info = [], []
    start = 0
    n = len(order)
    while start < n:
        i0 = order[start]
        t, piece = k_t[i0], k_s[i0] // tile
        end = start
        while end < n and k_t[order[end]] == t and k_s[order[end]] // tile == piece:
            end += 1
        tiles.append(order[start:end])
        info.append((int(t), int(k_s[i0])))
        start = end
    return tiles, info


def proxies(q, q_pos, k_rot, qtiles, ktiles, dims, theta, scale):
    """P[i, j] = mean over the query rows of tile i and the keys of tile j of the logit
    scale * sum_h <q_rot, k_rot>: the logits of each query tile against every key are formed
    head by head, then each key tile's block of them is averaged."""
    q_rot = rope3d(np.asarray(q, dtype=np.float64), q_pos, dims, theta)  # [Nq, H, D]
    k_rot = np.asarray(k_rot, dtype=np.float64)
    heads = q_rot.shape[1]
    p = np.zeros((len(qtiles), len(ktiles)))
    for i, (q0, ql) in enumerate(qtiles):
        logits = np.zeros((ql, k_rot.shape[0]))
        for h in range(heads):
            logits += q_rot[q0:q0 + ql, h, :] @ k_rot[:, h, :].T
        logits *= scale
        for j, idx in enumerate(ktiles):
            p[i, j] = logits[:, idx].mean()
    return p


def candidates(mask, q_t, q_s, qtiles, ktiles, k_t, k_s):
    """C[i, j]: key tile j visible to query tile i under the static rule (whole tiles)."""
    c = np.zeros((len(qtiles), len(ktiles)), dtype=bool)
    for i, (q0, ql) in enumerate(qtiles):
        for j, idx in enumerate(ktiles):
            vis = allowed_mask(mask, q_t[q0], q_s[q0], k_t[idx], k_s[idx])
            assert vis.all() or not vis.any(), "a key tile is partly visible"
            c[i, j] = vis.all()
    return c


def spread(p, cand):
    """Per query tile: largest and smallest candidate proxy (-inf / inf without candidates)."""
    return np.where(cand, p, -np.inf).max(axis=1), np.where(cand, p, np.inf).min(axis=1)


def kept(p, cand, tau: float):
    """K[i, j]: candidate j of query tile i passes the adaptive threshold."""
    big, small = spread(p, cand)
    with np.errstate(invalid="ignore"):
        return cand & ((p - small[:, None]) >= (1.0 - tau) * (big - small)[:, None])


def dynamic_spans(p, cand, tau, ktiles, k_phys):
    """Kept key tiles of every query tile as maximal runs of physical indices."""
    keep_all = kept(p, cand, tau)
    spans = []
    for i in range(p.shape[0]):
        keep = keep_all[i]
        vis = np.sort(np.concatenate([k_phys[ktiles[j]] for j in np.flatnonzero(keep)] or [np.zeros(0, np.int64)]))
        cut = np.flatnonzero(np.diff(vis) != 1) + 1
        first = np.concatenate([[0], cut]).astype(np.int64)
        last = np.concatenate([cut, [len(vis)]]).astype(np.int64)
        spans.append([(int(vis[a]), int(b - a)) for a, b in zip(first, last) if b > a])
    return spans


def dynamic_plan(st, tau: float, scale=None):
    """Everything the device builder must reproduce for a workload state `st`
    (from pipeline.build_state): query tiles, key tiles, proxies, candidates, spans."""
    w = st.w
    scale = w.head_dim ** -0.5 if scale is None else scale
    qtiles = query_tiles(w.mask, w.q_frames, w.tokens_per_frame, w.q_t0)
    ktiles, kinfo = key_tiles(st.k_phys, st.k_t, st.k_s, w.mask.tile)
    p = proxies(st.q, st.q_pos, st.k, qtiles, ktiles, w.rope_dims, w.theta, scale)
    q_s = np.arange(w.n_q) % w.tokens_per_frame
    cand = candidates(w.mask, st.q_pos[:, 0], q_s, qtiles, ktiles, st.k_t, st.k_s)
    spans = dynamic_spans(p, cand, tau, ktiles, st.k_phys)
    return dict(qtiles=qtiles, ktiles=ktiles, kinfo=kinfo, proxies=p, cand=cand, spans=spans)
