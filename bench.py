#!/usr/bin/env python3
"""Benchmark of the HSTU causal pointwise attention forward on one MI355X.

One step = one hstu_attn_fwd call (work-list build + attention kernel) over the
long-history workload: 4 sequences x 8192 tokens, 8 heads, dqk = dv = 128,
relative position + time bias, divisor n, bf16 inputs with fp32 accumulation.
Inputs are synthetic (seeded recipes in ``workloads``) and resident in HBM
before the timed region.

Prints ONE JSON line with the causal-effective TFLOP/s (the metric), tokens/s,
a roofline object for the attention kernel (bf16 MFMA bound) and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --copy-calib      # plain copy of known size, for counter scaling
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

METRIC = "HSTU attention causal-effective TFLOP/s + tokens/s/layer, jagged bf16, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_c3_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "hstu_pointwise_attention_causal_amd", "csrc", "attn_fwd.hip")
COPY_BYTES = 1 << 30


def _kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(steps_note=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the attention kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != _kernel_hash():
        return None
    return t.get("bytes_per_launch")


def copy_calib():
    import torch
    dev = torch.device("cuda:0")
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read": COPY_BYTES, "copy_calib_bytes_written": COPY_BYTES}))


def cpu_baseline(wl, target_s: float):
    """The fp64 oracle as it stands, on (sequence, head) units of the same
    workload until about target_s seconds of CPU work; scaled to TFLOP/s."""
    import numpy as np
    from oracle import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    off = wl.seq_offsets
    flops = 0.0
    units = 0
    t0 = time.perf_counter()
    for b in range(wl.num_seqs):
        for h in range(wl.num_heads):
            s = slice(int(off[b]), int(off[b + 1]))
            n = int(off[b + 1] - off[b])
            orc.attn_fwd(wl.q[s][:, h:h + 1], wl.k[s][:, h:h + 1], wl.v[s][:, h:h + 1],
                         np.array([0, n]), alpha=wl.alpha, divisor=wl.divisor,
                         pos_table=wl.pos_table[h:h + 1], time_table=wl.time_table[h:h + 1],
                         timestamps=wl.timestamps[s])
            flops += n * (n + 1) / 2 * 2.0 * (wl.dqk + wl.dv)
            units += 1
            if time.perf_counter() - t0 >= target_s:
                break
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} of {wl.num_seqs * wl.num_heads} (sequence, head) units of the "
                      f"workload, fp64 NumPy oracle, {dt:.1f} s wall; BLAS threads {threads}, "
                      f"elementwise steps single-threaded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calib()
        return

    import torch
    import hstu_pointwise_attention_causal_amd as hstu
    from workloads import make_workload

    hstu.load()
    dev = torch.device("cuda:0")
    wl = make_workload(args.workload)
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)  # noqa: E731
    q, k, v = t(wl.q, torch.bfloat16), t(wl.k, torch.bfloat16), t(wl.v, torch.bfloat16)
    off = torch.from_numpy(wl.seq_offsets).to(dev)
    ts = torch.from_numpy(wl.timestamps).to(dev) if wl.timestamps is not None else None
    pt = t(wl.pos_table, torch.float32) if wl.pos_table is not None else None
    tt = t(wl.time_table, torch.float32) if wl.time_table is not None else None
    out = torch.empty_like(v)
    ws = torch.empty(hstu.attn_workspace_size(wl.num_heads, wl.dqk, wl.dv, torch.bfloat16,
                                              wl.num_seqs, wl.total_tokens), dtype=torch.uint8,
                     device=dev)

    def step():
        hstu.attn_fwd(q, k, v, off, timestamps=ts, pos_table=pt, time_table=tt,
                      alpha=wl.alpha, divisor=wl.divisor, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)   # the stream every kernel is launched on
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_events = ev0.elapsed_time(ev1) / args.steps
    ms_step = max(ms_events, wall * 1e3 / args.steps)

    flops = wl.attn_fwd_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_events * 1e-3) / 1e12
    tokens_s = wl.total_tokens / (ms_step * 1e-3)

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {wl.note}",
            "global_batch": wl.num_seqs,
            "seq_len": wl.max_seq_len,
            "total_tokens": wl.total_tokens,
            "heads": wl.num_heads,
            "dqk": wl.dqk,
            "dv": wl.dv,
            "parallelism": "none (1 GPU)",
        },
        "tokens_per_s": round(tokens_s, 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": _traffic(),
            "kernel": "attn_fwd_bf16_kernel<128,128> (+ work-list builder inside the timed call)",
            "algorithmic_flops_per_launch": flops,
            "avg_launch_ms": round(ms_events, 5),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
