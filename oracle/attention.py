"""Masked softmax attention, float64.

The method reaches this exact result faster (tile skipping and online softmax do not
change it; "DynamicRad ..." page section 1 and "Accelerating Video Generation
Inference ..." page section 1 describe the full O(N^2) spatiotemporal attention it
replaces).  Definition: S = (Q K^T) * scale; masked entries are -inf; each row of
P = softmax(S) is exp(S - row max) / sum; O = P V; LSE = row max + ln(row sum).
A row with no visible key has O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray, scale: float):
    """q [Nq, D], k [Nk, D], v [Nk, Dv], allowed [Nq, Nk] bool -> (O [Nq, Dv], LSE [Nq])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    s = np.where(allowed, s, -np.inf)
    empty = ~allowed.any(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1, initial=-np.inf))
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (p @ v) / np.where(empty, 1.0, l)[:, None]
    o[empty] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return o, lse
