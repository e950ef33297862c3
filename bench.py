"""Benchmark of one denoising-chunk attention step on one MI355X.

A step is the whole hot path for one chunk: the chunk's K/V append into the ring cache
(K rotated at global frames), the block plan built on the device, and the block-sparse
attention forward with RoPE applied to Q while it is loaded.  Inputs are resident in HBM
before the timed region.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line.  value = attention FLOP on computed blocks / step time (TFLOP/s);
the attention kernel alone is timed with HIP events on its launch stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention ms/chunk and TFLOP/s on computed blocks; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
ATTN_SRC = os.path.join(ROOT, "video_diffusion_transformer_rope3d_amd", "csrc", "vdit_attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan13b_chunk")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="query rows of the oracle sample (0 = auto)")
    return ap.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_per_launch():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_sha(ATTN_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, inputs, rows_wanted):
    """The fp64 oracle on a bounded sample of the same workload, on this host's cores."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    st = oracle.build_state(w, inputs)
    n_keys = len(st.k_phys)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(w.n_q, size=min(rows_wanted, w.n_q), replace=False))
    t = time.perf_counter()
    oracle.attention_rows(st, 0, rows)
    dt = time.perf_counter() - t
    # visible pairs of the sampled rows (every row of this workload sees all cached keys
    # when the rule is chunk-causal over the whole ring; count exactly from the mask)
    q_s = np.arange(w.n_q) % w.tokens_per_frame
    vis = oracle.allowed_mask(w.mask, st.q_pos[rows, 0][:, None], q_s[rows][:, None], st.k_t[None], st.k_s[None])
    flop = 4.0 * w.head_dim * float(vis.sum())
    return dict(value=flop / dt / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"head 0, {len(rows)} of {w.n_q} query rows against {n_keys} cached keys: RoPE of the "
                       f"rows, element mask, fp64 masked softmax attention ({dt:.1f} s); ring build excluded")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from workloads import get_workload, make_inputs
    from video_diffusion_transformer_rope3d_amd import AttentionSession
    from video_diffusion_transformer_rope3d_amd import binding as B

    w = get_workload(args.workload)
    inputs = make_inputs(w)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dt)

    m = w.mask
    s = AttentionSession(w.heads, w.head_dim, w.frame_h, w.frame_w, w.capacity, w.rope_dims, w.theta,
                         max_t=w.rope_max_t + 4, mask=m.kind, chunk_frames=m.chunk_frames, tile=m.tile,
                         radial_w0=m.radial_w0, radial_decay_log2=m.radial_decay_log2,
                         long_range_period=m.long_range_period)
    for t0, f, hk, hv in inputs["history"]:
        s.append(dev(hk), dev(hv), t0)
    q, k, v = dev(inputs["q"]), dev(inputs["k"]), dev(inputs["v"])
    o = torch.empty_like(q)
    plan = torch.empty(s.plan_bound(w.q_frames, w.q_t0), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        s.append(k, v, w.q_t0)
        s.plan(w.q_frames, w.q_t0, out=plan)
        if ev is not None:
            ev[0].record(stream)
        s.attend(q, w.q_frames, w.q_t0, plan, o=o)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    header = plan[:8].cpu().numpy()
    pairs = int(np.uint32(header[6])) + (int(np.uint32(header[7])) << 32)
    flop = 4.0 * w.head_dim * w.heads * pairs

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(events[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in events]
    attn_avg = sum(attn_ms) / len(attn_ms)
    attn_tflops = flop / (attn_avg * 1e-3) / 1e12

    traffic = traffic_per_launch()
    result = {
        "metric": METRIC,
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": w.heads, "head_dim": w.head_dim,
                   "q_tokens": w.n_q, "kv_tokens": int(pairs // max(w.n_q, 1)) if m.kind != "log_radial" else None,
                   "frame": f"{w.frame_h}x{w.frame_w}", "q_t0": w.q_t0, "mask": m.kind,
                   "computed_block_flop": flop},
        "attn_ms_per_chunk": round(attn_avg, 4),
        "attn_tflops": round(attn_tflops, 2),
        "attn_frac_of_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rows = args.cpu_rows or 1024
        result["cpu_baseline"] = cpu_baseline(w, inputs, rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
