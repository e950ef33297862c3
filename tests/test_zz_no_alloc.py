"""The allocation-free attention entry point, vdit_block_attn_fwd_static (the library's static
scratch array in place of a caller's workspace), against vdit_block_attn_fwd with a workspace:
two calls in a row, the second with a smaller input, through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

from workloads import get_workload, make_inputs
from video_diffusion_transformer_rope3d_amd import binding as B

from harness import compare, run_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def test_static_scratch_matches_the_workspace_entry_point_on_two_calls():
    # the Wan-1.3B chunk geometry with 2 heads, then a smaller padded-frame chunk
    for name in ("wan13b_chunk_h2", "small_chunk_pad"):
        print("no-alloc entry point", name, flush=True)
        w = get_workload(name)
        r = run_workload(w, make_inputs(w))  # appends, device plan, attention with a workspace
        s = r["session"]
        lse = torch.full((w.heads, w.n_q), float("nan"), dtype=torch.float32, device="cuda")
        o = torch.full_like(r["q"], float("nan"))
        L = B.lib()
        st = L.vdit_block_attn_fwd_static(B.tensor(r["q"]), ctypes.byref(s.rope.cfg), s.grid(w.q_frames), w.q_t0,
                                          ctypes.byref(s.cache.desc), ctypes.byref(s.mask), r["plan"].data_ptr(),
                                          ctypes.c_float(0.0), B.tensor(o), lse.data_ptr(), B._stream(None))
        assert st == B.VDIT_OK, B.vdit_last_error()
        torch.cuda.synchronize()
        a, b = o.float().cpu().numpy(), r["o"].float().cpu().numpy()
        for h in range(w.heads):
            compare(a[:, h], b[:, h], what=f"{name} head {h}: static scratch vs workspace")
        np.testing.assert_allclose(lse.cpu().numpy(), r["lse"].cpu().numpy(), atol=1e-5, rtol=0)


def test_static_scratch_refuses_calls_beyond_its_size():
    """A call whose workspace would exceed the 72 MiB array is refused before anything runs: 400
    heads x 4096 query tiles of arrival counters (the pointers are never dereferenced)."""
    fake = 0x10000
    slots = np.zeros(1, np.int32)
    heads, hd, hw = 400, 64, 512 * 1024
    desc = B.VditKVCache(fake, fake, fake, slots.ctypes.data, 1, hw, heads, hd)
    t = B.VditTensor(fake, B.VDIT_DTYPE_BF16, 0, heads * hd, hd)
    m = B.mask_cfg("dense")
    g = B.grid(1, 512, 1024)
    n = ctypes.c_size_t(0)
    L = B.lib()
    assert L.vdit_block_attn_workspace_bytes(ctypes.byref(m), g, 0, ctypes.byref(desc), ctypes.byref(n)) == 0
    assert n.value > 72 << 20
    st = L.vdit_block_attn_fwd_static(t, None, g, 0, ctypes.byref(desc), ctypes.byref(m), fake, ctypes.c_float(0.0),
                                      t, None, B._stream(None))
    assert st == B.VDIT_ERR_UNSUPPORTED
    assert "static scratch" in B.vdit_last_error()
