"""A streaming attention session: one rope table, one ring KV cache, one visibility rule.

Convenience over the C ABI for the usual call sequence of a denoising chunk:

    s = AttentionSession(heads=12, head_dim=128, frame_h=30, frame_w=52, capacity=21,
                         rope_dims=(44, 42, 42), theta=1e4, max_t=512,
                         mask="chunk_causal", chunk_frames=3)
    s.append(k, v, t0)                  # rotate K at global frames, write ring slots
    plan = s.plan(q_frames=3, q_t0=t0)  # block list on the device
    o = s.attend(q, q_frames=3, q_t0=t0, plan=plan)

Device memory comes from torch (the ring, tables, outputs and the session's workspace, zeroed
when allocated); every computation is a libvdit kernel.
"""
from __future__ import annotations

from . import binding as B


class AttentionSession:
    def __init__(self, heads, head_dim, frame_h, frame_w, capacity, rope_dims, theta, max_t,
                 mask="chunk_causal", chunk_frames=1, tile=128, radial_w0=13, radial_decay_log2=1,
                 long_range_period=8, device="cuda", stream=None):
        self.heads, self.head_dim = heads, head_dim
        self.frame_h, self.frame_w = frame_h, frame_w
        self.stream = stream
        self.rope = B.Rope(head_dim, rope_dims, theta, max_t, frame_h, frame_w, device=device)
        self.cache = B.KVCache(capacity, frame_h * frame_w, heads, head_dim, device=device, stream=stream)
        self.mask = B.mask_cfg(mask, chunk_frames, tile, radial_w0, radial_decay_log2, long_range_period)
        # workspaces of the session's calls, which run in order on its stream: attention (whose
        # counters must stay zero between calls) and the dynamic plan have one each
        self.attn_workspace = B.Workspace(device)
        self.dyn_workspace = B.Workspace(device)

    def grid(self, frames):
        return B.grid(frames, self.frame_h, self.frame_w)

    def append(self, k, v, t0, rotate=True):
        frames = k.shape[0] // (self.frame_h * self.frame_w)
        B.vdit_kv_append(self.cache, self.rope if rotate else None, self.grid(frames), t0, k, v, self.stream)

    def append_plan(self, k, v, t0, rotate=True, out=None):
        """append(k, v, t0) and the device plan of the same frames as the query call, in one
        launch."""
        frames = k.shape[0] // (self.frame_h * self.frame_w)
        return B.vdit_kv_append_plan(self.cache, self.rope if rotate else None, self.grid(frames), t0, k, v,
                                     self.mask, out, self.stream)

    def plan(self, q_frames, q_t0, where=B.VDIT_WHERE_DEVICE, out=None):
        return B.vdit_plan_mask(self.mask, self.grid(q_frames), q_t0, self.cache, where, out, self.stream)

    def plan_bound(self, q_frames, q_t0):
        return B.vdit_plan_bound(self.mask, self.grid(q_frames), q_t0, self.cache)

    def attend(self, q, q_frames, q_t0, plan, o=None, lse=None, rotate=True, softmax_scale=0.0, mask=None):
        """`mask`: the session's rule by default; B.dynamic_mask(session.mask) for a plan from
        plan_dynamic."""
        return B.vdit_block_attn_fwd(q, self.rope if rotate else None, self.grid(q_frames), q_t0, self.cache,
                                     self.mask if mask is None else mask, plan, softmax_scale, o, lse, self.stream,
                                     self.attn_workspace)

    def plan_dynamic(self, q, q_frames, q_t0, tau, out=None, proxies=None, rotate=True, softmax_scale=0.0):
        """Dynamic-threshold plan of the session's rule on the device."""
        return B.vdit_plan_dynamic(self.mask, tau, q, self.rope if rotate else None, self.grid(q_frames), q_t0,
                                   self.cache, softmax_scale, out, proxies, self.stream, self.dyn_workspace)
