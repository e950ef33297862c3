"""The seeded random geometries of the GPU parity tests cover what those tests claim to cover (CPU only:
the generators are plain host code)."""
import numpy as np

from harness import random_workload
from test_gpu_proj import _random_case


def test_attention_random_geometries_cover_the_rules_dtypes_and_ring_states():
    ws = [random_workload(i) for i in range(24)]
    assert {w.mask.kind for w in ws} == {"dense", "chunk_causal", "log_radial", "log_radial_causal"}
    assert {w.head_dim for w in ws} == {64, 128}
    assert {w.dtype for w in ws} == {"bf16", "fp32"}
    assert {w.heads for w in ws} >= {1, 2, 3, 5}
    # ragged query and key tiles, and frames of several tiles
    assert any(w.tokens_per_frame % 128 for w in ws) and any(w.tokens_per_frame > 256 for w in ws)
    # a ring that wraps (more frames appended than it holds), one that does not, and a call without history
    frames = [sum(f for _, f in w.history) + w.q_frames for w in ws]
    assert any(n > w.capacity for n, w in zip(frames, ws)) and any(n <= w.capacity for n, w in zip(frames, ws))
    assert any(not w.history for w in ws)
    # appends are contiguous in time, each within the ring, and end where the chunk starts
    for w in ws:
        t = w.history[0][0] if w.history else w.q_t0
        for t0, f in w.history:
            assert t0 == t and 1 <= f <= w.capacity
            t += f
        assert t == w.q_t0 and w.q_frames <= w.capacity


def test_projection_random_geometries_cover_bias_rope_and_shapes():
    cs = [_random_case(i) for i in range(12)]
    assert {c[1] for c in cs} == {64, 128}
    assert {c[9] for c in cs} == {True, False}  # bias
    assert any(c[10] is None for c in cs) and any(c[10] is not None for c in cs)  # RoPE off / on
    assert all((c[0] * c[1]) % 128 == 0 and c[2] % 64 == 0 for c in cs)  # the entry point's shape rules
    assert any((c[3] * c[4] * c[5]) % 128 for c in cs)  # a ragged token tile
    assert any(sum(f for _, f in c[8]) + c[5] > c[7] for c in cs)  # the ring wraps
    for c in cs:
        assert all(1 <= f <= c[7] for _, f in c[8])
