"""Benchmark of one denoising-chunk attention step on one MI355X.

A step is the whole hot path for one chunk: the chunk's K/V append into the ring cache
(K rotated at global frames), the block plan built on the device (by one extra workgroup of
the append launch; --separate-plan: its own launch), and the block-sparse attention forward
with RoPE applied to Q while it is loaded.  Inputs are resident in HBM before the timed
region.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--dynamic-tau TAU] [--no-cpu-baseline]
                    [--library-reference]

--dynamic-tau builds the content-adaptive plan (pooled tile logits, adaptive threshold)
in place of the static one; the step then carries the append and that plan's four launches.

Before the W warmup steps, the step runs for 200 ms of wall time (clock_ramp_ms), so that the
timed steps see the GPU at its sustained clocks.

Prints one JSON line.  value = attention FLOP on computed blocks / step time (TFLOP/s), the
step time taken over K steps back to back with HIP events only at the two ends; K more
steps carry events around each launch, which time the attention kernel alone on its launch
stream (mean and median, warm caches) and the append (+ plan) launch; --cold-steps more
steps are each preceded by a read of 512 MiB of scratch that evicts the MALL and the L2s
(cold: K/V, Q and plan from HBM; --cold-write: a write of the scratch instead, whose dirty
lines the step then also writes back).
--library-reference adds the stock library call on the same shapes (torch's SDPA where every
query sees every cached key; F.linear with --qkv) as context, timed the same way.
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
# the attention kernel of the chunk-causal and dense workloads (one workgroup per CU, query
# tiles paired into units); log-radial plans run attn_tile_kernel
ATTN_KERNEL = "attn_unit_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan13b_chunk")
    ap.add_argument("--dynamic-tau", type=float, default=None, metavar="TAU",
                    help="build the dynamic-threshold plan (tau in [0, 1]) instead of the static one")
    ap.add_argument("--separate-plan", action="store_true",
                    help="static plan from its own launch after the append (default: built in the append launch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only (by default a run on the Wan-1.3B chunk also times the "
                         "dense clip, the log-radial clip, the 14B stream and the streaming log-radial chunk)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (whole heads are added until reached)")
    ap.add_argument("--qkv", action="store_true",
                    help="time the fused QKV projection + RoPE + K/V append of the Wan-1.3B chunk")
    ap.add_argument("--rope", action="store_true",
                    help="time the standalone RoPE3D rotation of the Wan-1.3B chunk's Q and K (in place)")
    ap.add_argument("--rel-l1", action="store_true",
                    help="time the block-reuse indicator (relative L1 of 30 blocks of 4680 x 1536 bf16 features)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="attention calls timed after a 512 MiB scratch sweep each (cold MALL and L2); 0: skip")
    ap.add_argument("--cold-write", action="store_true",
                    help="cold steps: the sweep writes the scratch instead of reading it")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run one device-to-device copy of MIB MiB before timing (HBM counter calibration)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="offline: turn two rocprofv3 counter_collection CSVs into profiles/attn_fwd_traffic.json")
    ap.add_argument("--library-reference", action="store_true",
                    help="also time the stock library call for the same shapes: torch's SDPA (all keys visible "
                         "to every query only) or, with --qkv, the plain bf16 GEMM of F.linear")
    ap.add_argument("--traffic-copy-mib", type=int, default=256)
    ap.add_argument("--traffic-kernel", default=ATTN_KERNEL, help="kernel name the --traffic counters are taken for")
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE, help="where --traffic writes its summary")
    ap.add_argument("--traffic-command", default="")
    return ap.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_per_launch(workload):
    """HBM bytes per attention launch from a committed rocprofv3 counter summary
    (profiles/attn_*traffic.json), if one was taken on the current kernel source and on this
    workload."""
    import glob
    sha = source_sha(ATTN_SRC)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "attn_*traffic.json"))):
        try:
            with open(path) as f:
                t = json.load(f)
        except (OSError, ValueError):
            continue
        if t.get("kernel_source_sha256") == sha and t.get("workload", "wan13b_chunk") == workload:
            return t.get("hbm_bytes_per_launch")
    return None


def cpu_baseline(w, inputs, seconds):
    """The fp64 oracle on a bounded sample of the same workload, on this host's cores:
    whole heads (all query rows against all cached keys) until `seconds` have elapsed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    st = oracle.build_state(w, inputs)
    q_s = np.arange(w.n_q) % w.tokens_per_frame
    vis = oracle.allowed_mask(w.mask, st.q_pos[:, 0][:, None], q_s[:, None], st.k_t[None], st.k_s[None])
    flop_per_head = 4.0 * w.head_dim * float(vis.sum())
    spent, heads = 0.0, 0
    while spent < seconds and heads < 4 * w.heads:  # whole heads, cycling, until the budget is used
        t = time.perf_counter()
        oracle.attention_rows(st, heads % w.heads)
        spent += time.perf_counter() - t
        heads += 1
    return dict(value=flop_per_head * heads / spent / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                cpu_model=cpu_model(), affinity_cores=len(os.sched_getaffinity(0)),
                sample=f"{heads} head passes ({w.heads} heads per chunk), each all {w.n_q} query rows against "
                       f"{len(st.k_phys)} cached keys: RoPE of Q, element mask, fp64 masked softmax attention "
                       f"({spent:.1f} s); the ring build (K rotation of all heads) is excluded; cores = the BLAS "
                       f"threads the oracle ran on, affinity_cores = the CPUs this process may use")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


RAMP_SECONDS = 0.2


def clock_ramp(fn, seconds=RAMP_SECONDS):
    """Runs fn() in batches until `seconds` of wall time have passed: the GPU settles at its
    sustained clocks only after tens of milliseconds of load, and the counted warmup steps of a
    short call alone (a few milliseconds) would leave the timed steps on a rising clock."""
    import torch
    end = time.perf_counter() + seconds
    while time.perf_counter() < end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_back_to_back(fn, steps, stream):
    """ms per call of `steps` calls issued back to back, HIP events only at the two ends."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_library(fn, steps, warmup):
    """ms per call of a library call, timed as this library's calls are (back to back)."""
    import torch
    for _ in range(warmup):
        fn()
    return time_back_to_back(fn, steps, torch.cuda.current_stream())


def library_attention(heads, n_q, n_k, head_dim, flop, steps, warmup):
    """torch's scaled_dot_product_attention (ROCm flash backend) on random bf16 Q, K, V of
    the workload's shapes with no mask: the same FLOP as the chunk when every query sees
    every cached key."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    g = torch.Generator(device="cuda").manual_seed(1)
    q = torch.randn((1, heads, n_q, head_dim), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((1, heads, n_k, head_dim), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((1, heads, n_k, head_dim), device="cuda", generator=g).to(torch.bfloat16)
    with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
        ms = time_library(lambda: F.scaled_dot_product_attention(q, k, v), steps, warmup)
    return {"call": "torch.nn.functional.scaled_dot_product_attention (flash backend), bf16, no mask",
            "ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2)}


def write_traffic(fetch_csv, write_csv, copy_mib, command, kernel=ATTN_KERNEL, workload="wan13b_chunk",
                  out_file=TRAFFIC_FILE):
    """Per-launch HBM bytes of an attention kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for the device-to-device copy of copy_mib MiB made by --calibrate-copy."""
    import csv

    def per_kernel(path, counter, needle):
        vals = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter and needle in r.get("Kernel_Name", ""):
                    vals.append(float(r["Counter_Value"]))
        if not vals:
            raise SystemExit(f"no {counter} sample of a kernel matching {needle!r} in {path}")
        return vals

    attn_fetch = per_kernel(fetch_csv, "FETCH_SIZE", kernel)
    attn_write = per_kernel(write_csv, "WRITE_SIZE", kernel)
    # the calibration copy is the largest copy dispatch of the run
    copy_fetch = max(per_kernel(fetch_csv, "FETCH_SIZE", "copyBuffer"))
    copy_write = max(per_kernel(write_csv, "WRITE_SIZE", "copyBuffer"))
    copy_bytes = copy_mib * 2 ** 20
    f_fetch = copy_bytes / (copy_fetch * 1024)
    f_write = copy_bytes / (copy_write * 1024)
    fetch_kib = sum(attn_fetch) / len(attn_fetch)
    write_kib = sum(attn_write) / len(attn_write)
    hbm = fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write
    out = {"kernel": kernel, "workload": workload, "kernel_source_sha256": source_sha(ATTN_SRC),
           "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
           "dispatches": [len(attn_fetch), len(attn_write)],
           "copy_calibration": {"bytes": copy_bytes, "fetch_kib": copy_fetch, "write_kib": copy_write,
                                "fetch_factor": f_fetch, "write_factor": f_write},
           "hbm_bytes_per_launch": hbm, "command": command}
    os.makedirs(os.path.dirname(out_file), exist_ok=True)
    with open(out_file, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def bench_rel_l1(args):
    """The block-wise reuse indicator on Wan-1.3B-shaped block features (30 blocks, one 3-frame
    chunk of 4680 tokens x 1536 channels each, bf16): HBM-bound, 2 feature sets read once."""
    import numpy as np
    import torch

    from video_diffusion_transformer_rope3d_amd import binding as B

    nb, tokens, hidden = 30, 4680, 1536
    elems = tokens * hidden
    g = torch.Generator(device="cuda").manual_seed(0)
    prev = torch.randn((nb, elems), device="cuda", generator=g).to(torch.bfloat16)
    cur = (prev.float() + 0.05 * torch.randn((nb, elems), device="cuda", generator=g)).to(torch.bfloat16)
    out = torch.empty(nb + 1, dtype=torch.float32, device="cuda")
    ws = B.Workspace()
    ws.get(B.vdit_block_rel_l1_workspace_bytes(nb, elems))  # allocated before the timed calls
    stream = torch.cuda.current_stream()
    clock_ramp(lambda: B.vdit_block_rel_l1(cur, prev, out=out, workspace=ws))
    for _ in range(args.warmup):
        B.vdit_block_rel_l1(cur, prev, out=out, workspace=ws)
    ms = time_back_to_back(lambda: B.vdit_block_rel_l1(cur, prev, out=out, workspace=ws), args.steps, stream)
    nbytes = 2 * nb * elems * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import bwcache
        c0, p0 = cur[:1].float().cpu().numpy(), prev[:1].float().cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            bwcache.rel_l1(c0, p0)
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        cpu = {"value": round(elems * 2 * 2 / sec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"one block ({tokens} x {hidden} elements, bf16 values in fp64), {reps} passes"}
    result = {
        "metric": "block reuse indicator: feature bytes read per second", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "clock_ramp_ms": RAMP_SECONDS * 1e3,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "wan13b_block_features", "blocks": nb, "tokens": tokens, "hidden": hidden},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "traffic": None},
        "mean_rel_l1": float(out[-1].item()),
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def bench_rope(args):
    """The standalone RoPE3D rotation (vdit_rope3d_qk) of one Wan-1.3B-shaped chunk: Q and K
    [4680 x 12 x 128] bf16 rotated in place at global positions (6 + f, h, w), split 44/42/42.
    HBM-bound: each element read and written once.  On the hot path the same rotation is fused
    into the attention's Q load and the K/V append; this times it on its own."""
    import torch

    from video_diffusion_transformer_rope3d_amd import binding as B

    heads, d, fh, fw, frames, t0 = 12, 128, 30, 52, 3, 6
    n = frames * fh * fw
    gen = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn((n, heads, d), device="cuda", generator=gen).to(torch.bfloat16)
    k = torch.randn((n, heads, d), device="cuda", generator=gen).to(torch.bfloat16)
    rope = B.Rope(d, (44, 42, 42), 1e4, t0 + frames + 4, fh, fw)
    grid = B.grid(frames, fh, fw)
    stream = torch.cuda.current_stream()
    call = lambda: B.vdit_rope3d_qk(rope, grid, t0, heads, q=q, k=k)  # noqa: E731 (repeated rotations: timing only)
    clock_ramp(call)
    for _ in range(args.warmup):
        call()
    ms = time_back_to_back(call, args.steps, stream)
    nbytes = 2 * 2 * n * heads * d * 2  # Q and K, read and written
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        rows = 520  # a bounded sample: the first third of a frame
        xs = q[:rows].float().cpu().numpy().astype(np.float64)
        pos = oracle.token_positions(frames, fh, fw, t0)[:rows]
        t_start = time.perf_counter()
        reps = 0
        while time.perf_counter() - t_start < min(args.cpu_seconds, 10.0):
            oracle.rope3d(xs, pos, (44, 42, 42), 1e4)
            reps += 1
        sec = (time.perf_counter() - t_start) / reps
        cpu = {"value": round(rows * heads * d * 2 * 2 / sec / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{rows} tokens of Q (bf16 values in fp64, read and written), {reps} passes"}
    result = {
        "metric": "standalone RoPE3D rotation: bytes read and written per second", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "clock_ramp_ms": RAMP_SECONDS * 1e3, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "wan13b_chunk_rope", "tokens": n, "heads": heads, "head_dim": d, "t0": t0},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def bench_qkv(args):
    """The fused QKV projection of one Wan-1.3B-shaped chunk: x [4680 x 1536] bf16 times
    W_qkv [4608 x 1536] bf16 (random, 1/sqrt(1536) scale) plus bias, Q rotated out, K and V
    rotated / copied into a 21-frame ring (frames 6..8)."""
    import numpy as np
    import torch

    from video_diffusion_transformer_rope3d_amd import binding as B

    heads, d, hidden, fh, fw, frames, t0, cap = 12, 128, 1536, 30, 52, 3, 6, 21
    n = frames * fh * fw
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((n, hidden), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((3 * heads * d, hidden), device="cuda", generator=g) / hidden ** 0.5).to(torch.bfloat16)
    b = 0.1 * torch.randn(3 * heads * d, device="cuda", generator=g)
    rope = B.Rope(d, (44, 42, 42), 1e4, t0 + frames + 4, fh, fw)
    cache = B.KVCache(cap, fh * fw, heads, d)
    q = torch.empty((n, heads, d), dtype=torch.bfloat16, device="cuda")
    grid = B.grid(frames, fh, fw)
    stream = torch.cuda.current_stream()
    clock_ramp(lambda: B.vdit_qkv_rope_append(x, w, b, rope, grid, t0, cache, q_out=q))
    for _ in range(args.warmup):
        B.vdit_qkv_rope_append(x, w, b, rope, grid, t0, cache, q_out=q)
    ms = time_back_to_back(lambda: B.vdit_qkv_rope_append(x, w, b, rope, grid, t0, cache, q_out=q), args.steps,
                           stream)
    flop = 2.0 * n * 3 * heads * d * hidden
    tf = flop / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import projection
        import oracle
        rows = 64  # a bounded sample: 64 tokens through the oracle
        xs, ws, bs = x[:rows].float().cpu().numpy(), w.float().cpu().numpy(), b.cpu().numpy()
        t_start = time.perf_counter()
        reps = 0
        while time.perf_counter() - t_start < min(args.cpu_seconds, 10.0):
            ring = oracle.RingCache(cap, 1, rows, heads, d)
            projection.qkv_rope_append(xs, ws, bs, ring, 1, t0, (44, 42, 42), 1e4)
            reps += 1
        sec = (time.perf_counter() - t_start) / reps
        cpu = {"value": round(2.0 * rows * 3 * heads * d * hidden / sec / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
               "kind": "oracle", "sample": f"{rows} tokens of the chunk (one 1 x {rows} frame), {reps} passes"}
    result = {
        "metric": "fused QKV projection + RoPE + KV append TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "clock_ramp_ms": RAMP_SECONDS * 1e3,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "wan13b_chunk_qkv", "tokens": n, "hidden": hidden, "heads": heads, "head_dim": d},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    if args.library_reference:
        import torch.nn.functional as F
        lms = time_library(lambda: F.linear(x, w), args.steps, args.warmup)
        result["library_reference"] = {"call": "torch.nn.functional.linear (bf16 GEMM alone: no bias, RoPE or "
                                               "cache write)", "ms": round(lms, 4),
                                       "tflops": round(flop / (lms * 1e-3) / 1e12, 2)}
    print(json.dumps(result), flush=True)


def measure(args, name, steps, warmup, cold_steps, tau=None, separate_plan=False, library_reference=False,
            cpu=False):
    """One workload's step timed as described in the module docstring: returns the result fields
    (value, per-launch times, roofline, ...) of its JSON line."""
    import numpy as np
    import torch

    from workloads import get_workload, make_inputs
    from video_diffusion_transformer_rope3d_amd import AttentionSession
    from video_diffusion_transformer_rope3d_amd import binding as B

    w = get_workload(name)
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
    if tau is None:
        plan = torch.empty(s.plan_bound(w.q_frames, w.q_t0), dtype=torch.int32, device="cuda")
        mask = s.mask
    else:
        plan = torch.empty(B.vdit_plan_dynamic_bound(s.mask, s.grid(w.q_frames), w.q_t0, s.cache),
                           dtype=torch.int32, device="cuda")
        mask = B.dynamic_mask(s.mask)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if tau is not None:
            s.append(k, v, w.q_t0)
            s.plan_dynamic(q, w.q_frames, w.q_t0, tau, out=plan)
        elif separate_plan:
            s.append(k, v, w.q_t0)
            s.plan(w.q_frames, w.q_t0, out=plan)
        else:
            s.append_plan(k, v, w.q_t0, out=plan)
        if ev is not None:
            ev[1].record(stream)
        s.attend(q, w.q_frames, w.q_t0, plan, o=o, mask=mask)
        if ev is not None:
            ev[2].record(stream)

    if args.calibrate_copy:
        n = args.calibrate_copy * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    clock_ramp(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    words = plan.cpu().numpy()
    hw = B.PLAN_HEADER_WORDS
    header = words[:hw]
    pairs = int(np.uint32(header[6])) + (int(np.uint32(header[7])) << 32)
    flop = 4.0 * w.head_dim * w.heads * pairs
    # work the kernels execute: a query tile's rows in whole 32-row waves (a wave past the
    # tile's end does no math), every span in whole 64-key tiles
    nq = int(header[4])
    q_lens = words[hw:hw + 2 * nq].reshape(-1, 2)[:, 1]
    row_ptr = words[hw + 2 * nq:hw + 3 * nq + 1]
    spans = words[hw + 3 * nq + 1:hw + 3 * nq + 1 + 2 * int(header[5])].reshape(-1, 2)
    executed_pairs = sum(int((q_lens[i] + 31) // 32 * 32) * int(((spans[row_ptr[i]:row_ptr[i + 1], 1] + 63) // 64).sum())
                         * 64 for i in range(nq))
    executed_flop = 4.0 * w.head_dim * w.heads * executed_pairs

    # value: K steps back to back with events only at the two ends (an event between two
    # launches costs a few microseconds of its own, which would be charged to the step)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    # per-launch times: K more steps with events around the append (+ plan) and the attention
    events = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    attn_times = [b.elapsed_time(c) for _, b, c in events]
    attn_avg = sum(attn_times) / steps
    prep_avg = sum(a.elapsed_time(b) for a, b, _ in events) / steps
    attn_tflops = flop / (attn_avg * 1e-3) / 1e12

    # cold: before each step, a sweep over 512 MiB of scratch evicts the 256 MB MALL and the
    # L2s, so the step reads the cached K/V, Q and the plan from HBM (the sweep is outside the
    # timed events).  By default the sweep reads (the caches then hold clean lines); with
    # --cold-write it writes, and the step also pays for writing the scratch's dirty lines back.
    cold = []
    if cold_steps > 0:
        scratch = torch.ones(512 * 2 ** 20 // 4, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        cev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(cold_steps)]
        for i in range(cold_steps):
            if args.cold_write:
                scratch.fill_(i)
            else:
                scratch.sum(dtype=torch.int64)
            step(cev[i])
        torch.cuda.synchronize()
        cold = [b.elapsed_time(c) for _, b, c in cev]
        del scratch

    traffic = traffic_per_launch(w.name)
    result = {
        "metric": METRIC,
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "clock_ramp_ms": RAMP_SECONDS * 1e3,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": w.heads, "head_dim": w.head_dim,
                   "q_tokens": w.n_q, "kv_tokens": int(pairs // max(w.n_q, 1)) if m.kind != "log_radial" and tau is None else None,
                   "mean_keys_per_query": round(pairs / max(w.n_q, 1), 1),
                   "frame": f"{w.frame_h}x{w.frame_w}", "q_t0": w.q_t0, "mask": m.kind,
                   "computed_block_flop": flop,
                   "plan": (f"dynamic tau={tau}" if tau is not None else
                            "static, separate launch" if separate_plan else "static, built in the append launch")},
        "append_plan_ms_per_chunk": round(prep_avg, 4),
        "attn_ms_per_chunk": round(attn_avg, 4),
        "attn_ms_per_chunk_median": round(float(np.median(attn_times)), 4),
        "attn_ms_per_chunk_cold": round(float(np.median(cold)), 4) if cold else None,
        "attn_tflops": round(attn_tflops, 2),
        "attn_frac_of_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "mfma_valid_fraction": round(flop / executed_flop, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": None,
    }
    if library_reference:
        n_k = int((s.cache.slot_host >= 0).sum()) * w.tokens_per_frame  # keys of the valid slots
        if n_k and pairs == w.n_q * n_k:
            result["library_reference"] = library_attention(w.heads, w.n_q, n_k, w.head_dim, flop, steps, warmup)
        else:
            result["library_reference"] = None  # masked: no stock call computes the same blocks
    if cpu:
        result["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    return result


# the other workloads one default run also times (the headline is the Wan-1.3B-shaped chunk)
OTHER_CONFIGS = ("dense_clip", "log_radial", "stream14b_chunk", "stream_radial_chunk")




def main():
    args = parse()
    if args.qkv:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_qkv(args)
        return
    if args.rope:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_rope(args)
        return
    if args.rel_l1:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_rel_l1(args)
        return
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], args.traffic_copy_mib, args.traffic_command,
                      args.traffic_kernel, args.workload, args.traffic_out)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch

    result = measure(args, args.workload, args.steps, args.warmup, args.cold_steps, tau=args.dynamic_tau,
                     separate_plan=args.separate_plan, library_reference=args.library_reference,
                     cpu=not args.no_cpu_baseline)
    if not args.no_configs and args.dynamic_tau is None and args.workload == "wan13b_chunk":
        # every headline workload in the same run, fewer steps each: ms per chunk of the attention
        # launch (warm, median of cold), its TFLOP/s and fraction of the bf16 peak, the work the
        # kernel executes per computed-block FLOP, and the append + plan launch
        result["configs"] = {}
        for name in OTHER_CONFIGS:
            r = measure(args, name, min(args.steps, 10), min(args.warmup, 3), min(args.cold_steps, 3))
            torch.cuda.empty_cache()
            result["configs"][name] = {
                "attn_ms_per_chunk": r["attn_ms_per_chunk"], "attn_ms_per_chunk_cold": r["attn_ms_per_chunk_cold"],
                "attn_tflops": r["attn_tflops"], "attn_frac_of_bf16_peak": r["attn_frac_of_bf16_peak"],
                "mfma_valid_fraction": r["mfma_valid_fraction"], "append_plan_ms_per_chunk":
                r["append_plan_ms_per_chunk"], "step_tflops": r["value"], "steps": r["steps"],
                "kernel": "attn_tile_kernel" if r["config"]["mask"] in ("log_radial", "log_radial_causal")
                else ATTN_KERNEL, "config": r["config"]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
