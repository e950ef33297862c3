"""Workload shapes for spatiotemporal RoPE3D + block-sparse KV-cache attention.

Each workload is one attention call of a denoising chunk (or a full clip)
against a ring-buffer KV cache of earlier latent frames.  The five headline
workloads follow the problem statement of the streaming video-diffusion pages:

* Wan2.1-style latent grid 30 x 52 = 1560 tokens per latent frame
  (480 x 832 pixels, page "Accelerating Video Generation Inference with
  Sequential-Parallel 3D Positional Encoding Using a Global Time Index",
  section 4; Wave Forcing / WaveRT page, "Utilisation": --height 480 --width 832);
* 3-frame chunks starting at multiples of 3 (same pages: start frames 0, 3, 6;
  latent frame count divisible by 3);
* global start frame t0 per call (page 1, section 2.B, the global time index);
* a log-radial window (DynamicRad page, section 2, "Estrutura de Janela Radial
  Logaritmica", static-ratio mode).

The remaining entries are reduced-size variants used by the parity tests to
cover ragged tiles, padded frame strides, ring wrap-around and calls that
straddle a chunk boundary.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MaskSpec:
    """Attention visibility rule.

    kind: "dense" | "chunk_causal" | "log_radial" | "log_radial_causal".
    chunk_frames: frames per causal chunk (chunk_causal, log_radial_causal).
    tile: query/key tile length in tokens used by the block plan.
    radial_w0, radial_decay_log2, long_range_period: log-radial window
      W(d) = ceil(w0 * 2**(-decay_log2 * d)) tiles at frame distance d; frames at a
      distance that is a multiple of long_range_period (if > 0) are kept whole.
    """

    kind: str
    chunk_frames: int = 1
    tile: int = 128
    radial_w0: int = 13
    radial_decay_log2: int = 1
    long_range_period: int = 8


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    heads: int
    head_dim: int
    frame_h: int
    frame_w: int
    q_frames: int
    q_t0: int
    rope_dims: tuple  # (d_t, d_h, d_w) channel widths, order t | h | w
    theta: float
    mask: MaskSpec
    capacity: int  # ring capacity in frames
    history: tuple = ()  # (t0, frames) appends made before the chunk, in order
    dtype: str = "bf16"  # input / output dtype: "bf16" or "fp32"
    data_scale: float = 1.0
    lowfreq_amp: float = 0.0
    seed: int = 0
    max_t: int = field(default=0)  # rope table length on the t axis (0 -> derived)

    @property
    def tokens_per_frame(self) -> int:
        return self.frame_h * self.frame_w

    @property
    def n_q(self) -> int:
        return self.q_frames * self.tokens_per_frame

    @property
    def rope_max_t(self) -> int:
        last = max([self.q_t0 + self.q_frames] + [t + f for t, f in self.history])
        return max(self.max_t, last)

    def appends(self):
        """All appends in order: history first, then the chunk's own K/V."""
        return list(self.history) + [(self.q_t0, self.q_frames)]


def _chunks(t_first, t_last_excl, step=3):
    return tuple((t, min(step, t_last_excl - t)) for t in range(t_first, t_last_excl, step))


_W = {}


def _add(w: Workload):
    _W[w.name] = w
    return w


# --- headline workloads -----------------------------------------------------
_add(Workload(
    name="tiny", seed=1,
    description="Tiny fp32: 2 heads, head_dim 64, 3 latent frames of 4x6 tokens (72 tokens), "
                "RoPE3D split 24/20/20, theta 1e4, t0=5, block-causal with 1-frame chunks, ring of 3 frames.",
    heads=2, head_dim=64, frame_h=4, frame_w=6, q_frames=3, q_t0=5, rope_dims=(24, 20, 20),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=1), capacity=3, dtype="fp32"))

_add(Workload(
    name="wan13b_chunk", seed=2,
    description="Wan-1.3B-shaped chunk denoise, bf16: 12 heads, head_dim 128, 30x52 tokens per frame; "
                "query chunk of 3 frames (4680 tokens) at t0=6 against a ring of 21 frames holding "
                "frames 0..8 (14040 keys); chunk-causal with 3-frame chunks; RoPE 44/42/42; data x 1/sqrt(128).",
    heads=12, head_dim=128, frame_h=30, frame_w=52, q_frames=3, q_t0=6, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=3), capacity=21,
    history=((0, 3), (3, 3)), data_scale=128 ** -0.5))

_add(Workload(
    name="dense_clip", seed=3,
    description="Dense bidirectional full clip, bf16: 21 latent frames x 1560 = 32760 tokens, 12 heads, "
                "head_dim 128, RoPE3D with t0=0, no mask.",
    heads=12, head_dim=128, frame_h=30, frame_w=52, q_frames=21, q_t0=0, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("dense"), capacity=21))

_add(Workload(
    name="log_radial", seed=4,
    description="Log-radial static-ratio sparse, bf16: 21 x 1560 tokens, 12 heads, head_dim 128, 128x128 tiles; "
                "window ceil(13 * 0.5^|i-j|) tiles, same frame whole, every 8th frame distance whole; "
                "inputs carry a spatial low-frequency component of amplitude 0.5.",
    heads=12, head_dim=128, frame_h=30, frame_w=52, q_frames=21, q_t0=0, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("log_radial", tile=128, radial_w0=13, radial_decay_log2=1, long_range_period=8),
    capacity=21, lowfreq_amp=0.5))

_add(Workload(
    name="stream14b_chunk", seed=5,
    description="14B-shaped long-stream chunk, bf16: 40 heads, head_dim 128; query chunk of 3 x 1560 tokens at "
                "t0=396 against a ring of the last 21 frames (378..398, 32760 keys); chunk-causal.",
    heads=40, head_dim=128, frame_h=30, frame_w=52, q_frames=3, q_t0=396, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=3), capacity=21,
    history=_chunks(378, 396)))

HEADLINE = ("tiny", "wan13b_chunk", "dense_clip", "log_radial", "stream14b_chunk")

# --- reduced variants for parity / edge-case tests -----------------------------
_add(Workload(
    name="tiny_d128", seed=11,
    description="Tiny at head_dim 128 with the 44/42/42 split.",
    heads=2, head_dim=128, frame_h=4, frame_w=6, q_frames=3, q_t0=5, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=1), capacity=3, dtype="fp32"))

_add(Workload(
    name="small_chunk_pad", seed=12,
    description="Chunk-causal, 10x13 = 130 tokens per frame (frame stride padded to 136), ring of 7 frames "
                "that has wrapped (frames 2..8), 2 heads, head_dim 128.",
    heads=2, head_dim=128, frame_h=10, frame_w=13, q_frames=3, q_t0=6, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=3), capacity=7,
    history=((0, 3), (3, 3)), data_scale=128 ** -0.5))

_add(Workload(
    name="small_radial", seed=13,
    description="Log-radial on 9 frames of 16x20 = 320 tokens (3 tiles per frame, last one 64 rows), "
                "w0=3, decay 1/2, long-range period 4, 3 heads, head_dim 128, spatial component 0.5.",
    heads=3, head_dim=128, frame_h=16, frame_w=20, q_frames=9, q_t0=0, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("log_radial", tile=128, radial_w0=3, radial_decay_log2=1, long_range_period=4),
    capacity=9, lowfreq_amp=0.5))

_add(Workload(
    name="small_dense_d64", seed=14,
    description="Dense, 5 frames of 8x10 tokens, 3 heads, head_dim 64, bf16, t0=2.",
    heads=3, head_dim=64, frame_h=8, frame_w=10, q_frames=5, q_t0=2, rope_dims=(24, 20, 20),
    theta=1e4, mask=MaskSpec("dense"), capacity=5))

_add(Workload(
    name="stream_wrap_straddle", seed=15,
    description="Ring of 21 frames of 30x52 that has wrapped (frames 382..402); the call covers frames "
                "400..402, which straddle a 3-frame chunk boundary, 4 heads, head_dim 128.",
    heads=4, head_dim=128, frame_h=30, frame_w=52, q_frames=3, q_t0=400, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=3), capacity=21,
    history=_chunks(379, 400)))

_add(Workload(
    name="wan13b_chunk_h2", seed=16,
    description="Wan-1.3B-shaped chunk with 2 heads (same token geometry as the full chunk).",
    heads=2, head_dim=128, frame_h=30, frame_w=52, q_frames=3, q_t0=6, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=3), capacity=21,
    history=((0, 3), (3, 3)), data_scale=128 ** -0.5))

_add(Workload(
    name="stream_radial_chunk", seed=17,
    description="Streaming log-radial, bf16: 12 heads, head_dim 128, 30x52 tokens per frame; query chunk of 3 "
                "frames at t0=396 against a ring of the last 21 frames (378..398); log-radial window w0=13, decay "
                "1/2, every 8th frame distance whole, restricted to block-causal 3-frame chunks; spatial "
                "component 0.5.",
    heads=12, head_dim=128, frame_h=30, frame_w=52, q_frames=3, q_t0=396, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("log_radial_causal", chunk_frames=3, tile=128, radial_w0=13, radial_decay_log2=1,
                             long_range_period=8),
    capacity=21, history=_chunks(378, 396), lowfreq_amp=0.5))

_add(Workload(
    name="small_stream_radial", seed=18,
    description="Streaming log-radial on a wrapped ring of 7 frames of 16x20 tokens (3 tiles per frame); the call "
                "covers frames 13..15, which straddle 3-frame chunks 4 and 5, so frames 13 and 14 must not see "
                "frame 15; w0=3, decay 1/2, period 4, 2 heads, head_dim 128, spatial component 0.5.",
    heads=2, head_dim=128, frame_h=16, frame_w=20, q_frames=3, q_t0=13, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("log_radial_causal", chunk_frames=3, tile=128, radial_w0=3, radial_decay_log2=1,
                             long_range_period=4),
    capacity=7, history=_chunks(4, 13), lowfreq_amp=0.5))

_add(Workload(
    name="wave_two_chunks", seed=19,
    description="Two whole 3-frame chunks in one call (frames 12..17, chunks 4 and 5 at different noise levels, "
                "as in staggered wave denoising): 30x52 tokens per frame, a ring of 9 frames that has wrapped; "
                "the history wrote chunk 4's frames once already, the call's own append refreshes them with new "
                "data and adds chunk 5; chunk-causal with 3-frame chunks, so chunk 4 does not see chunk 5; "
                "2 heads, head_dim 128, data x 1/sqrt(128).",
    heads=2, head_dim=128, frame_h=30, frame_w=52, q_frames=6, q_t0=12, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=3), capacity=9,
    history=_chunks(3, 15), data_scale=128 ** -0.5))

_add(Workload(
    name="wan13b_chunk_h14", seed=20,
    description="Wan-1.3B-shaped chunk with 14 heads: 266 units of one or two query tiles, one round of whole "
                "units on 256 workgroups, the rest split over all of them.",
    heads=14, head_dim=128, frame_h=30, frame_w=52, q_frames=3, q_t0=6, rope_dims=(44, 42, 42),
    theta=1e4, mask=MaskSpec("chunk_causal", chunk_frames=3), capacity=21,
    history=((0, 3), (3, 3)), data_scale=128 ** -0.5))

WORKLOADS = dict(_W)


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
