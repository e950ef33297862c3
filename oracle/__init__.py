"""CPU fp64 oracle for RoPE3D + block-sparse KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The product library never calls
it and shares no code with it.

Every function is the plain definition of what the method computes, in float64
numpy, written for a reader to check against the pages by eye:

* rope3d    - token positions with the global time index, and the 3D rotary
              rotation (Causal-RoPE SP page, section 2.B; Timeripple page,
              "Metodologia 1", RoPE channel groups t / x / y);
* ring      - the ring-buffer KV cache indexed by global frame (Causal-RoPE SP
              page, section 2.A, KV cache for causal inference; Wave Forcing page,
              cache refresh after a block is denoised);
* masks     - the chunk-causal and log-radial visibility rules and the block plan
              built from the element mask (Wave Forcing page, block-causal
              attention; DynamicRad page, section 2, log-radial window and
              static-ratio mode);
* attention - masked softmax attention (the exact result the method reaches);
* dynamic   - the dynamic-threshold block plan (DynamicRad page, section 2, dual-mode
              strategy, mode 2): pooled pre-softmax logits of (query tile, key tile)
              pairs as importance proxies and an adaptive threshold;
* projection- the fused QKV projection with RoPE at the global time index and the K/V
              append (Causal-RoPE SP page, section 2.C, fused QKV + RoPE);
* bwcache   - the block-wise feature reuse indicator (mean relative L1 distance of block
              features between timesteps) and the reuse policy (BWCache page, section 2).

Pins (see tests/test_oracle_*.py): RoPE against the RoFormer rotary implementation in
`transformers` and against invariants (norm, relative offset, per-axis
independence); dense attention against torch's scaled_dot_product_attention in
float64; closed forms (Q = 0, V = 1, one visible key); chunk-by-chunk calls with
global start frames equal one whole-sequence call; hand-derived block plans and
ring slot tables under tests/golden/; brute-force tile-pair counts.

Parity unpinned: the order of the channel groups (t, h, w) and the rule that
splits head_dim into group widths are readings of the pages, which name the
groups but neither their order nor their widths.
"""
from .rope3d import token_positions, axis_frequencies, rope3d  # noqa: F401
from .ring import RingCache  # noqa: F401
from .masks import (allowed_mask, radial_window, query_tiles, plan_from_mask,  # noqa: F401
                    serialize_plan, frame_stride_for)
from .attention import masked_attention  # noqa: F401
from .pipeline import build_state, build_layout, attention_rows, plan_for  # noqa: F401
