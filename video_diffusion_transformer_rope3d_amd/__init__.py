"""MI355X-native RoPE3D + block-sparse KV-cache attention for video diffusion transformers.

The computation lives in libvdit.so (HIP kernels for gfx950 behind the C ABI of
include/vdit.h); `binding` mirrors that ABI with the same names and `session` wraps the
usual append / plan / attend sequence of a denoising chunk.
"""
from . import binding  # noqa: F401
from .binding import (VditError, lib, vdit_abi_version, vdit_block_attn_fwd, vdit_kv_append,  # noqa: F401
                      vdit_kv_cache_bytes, vdit_kv_cache_reset, vdit_last_error, vdit_plan_bound,
                      vdit_plan_mask, vdit_plan_qtiles, vdit_rope3d_qk, vdit_rope_table_build,
                      vdit_status_string, vdit_token_positions)
from .session import AttentionSession  # noqa: F401
