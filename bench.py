#!/usr/bin/env python3
"""Benchmark of the HSTU hot path on one MI355X.

Headline (the JSON line's ``value``): causal-effective TFLOP/s of the attention
forward on the long-history workload -- 4 sequences x 8192 tokens, 8 heads,
dqk = dv = 128, relative position + time bias, divisor n, bf16 inputs with
fp32 accumulation. One step = one hstu_attn_fwd call (work-list build, block
metadata, attention kernel). Inputs are synthetic (seeded recipes in
``workloads``) and resident in HBM before the timed region.

Also on the line:
  roofline      the attention kernel's own average launch time, taken with HIP
                events that the library records around each launch on the
                launch stream (hstu_timing_enable), against the bf16 MFMA peak;
                HBM traffic (bytes per launch, and over this run's launch
                time as hbm_gbs) and the MFMA-busy fraction (mfma_util) from
                the committed rocprofv3 counter summary when it was taken on
                the current kernel source, else null;
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload;
  secondary     tokens/s per layer of the 4-layer stack (8 x 1024 tokens) and
                of one layer over the 64-sequence jagged batch, and the
                attention forward + backward of the 32-sequence jagged batch, one
                layer forward + backward, candidate scoring against cached
                histories, the final RMSNorm + tied retrieval head, and
                Stochastic Length (keyed selection + row gathers).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --copy-calib      # plain copy of known size, for counter scaling
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HSTU attention causal-effective TFLOP/s + tokens/s/layer, jagged bf16, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_fwd_c3_counters.json")
KERNEL_SRCS = [os.path.join(ROOT, "hstu_pointwise_attention_causal_amd", "csrc", f)
               for f in ("attn_fwd.hip", "attn_common.h", "common.h")]
LAUNCH_H = os.path.join(ROOT, "hstu_pointwise_attention_causal_amd", "csrc", "launch.h")
COPY_BYTES = 1 << 30


def _code_only(text: str) -> str:
    """C++ source without comments, trailing blanks or empty lines (the
    kernel files hold no string literal with a comment marker)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_hash() -> str:
    """Hash of the code the attention forward kernel is compiled from: its own
    file and headers, and of the launch header only the argument struct it
    reads (the header also declares every other kernel's launcher). Comments
    are left out, so editing one keeps a counter measurement valid."""
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p) as f:
            h.update(_code_only(f.read()).encode())
    with open(LAUNCH_H) as f:
        text = f.read()
    start = text.index("struct AttnArgs {")
    h.update(_code_only(text[start:text.index("};", start)]).encode())
    return h.hexdigest()[:16]


def _counters():
    """The committed rocprofv3 counter summary of the attention forward on
    this workload (MFMA busy fraction, HBM bytes per launch, ...), or None
    when the kernel source changed since it was taken."""
    try:
        with open(COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t


# Kernels the counter summary reports, by a substring of their symbol name.
COUNTER_KERNELS = {
    "attn_fwd": ("attn_fwd_bf16_kernel", "attn_fwd_pp_kernel"),
    "attn_bwd_kv": "attn_bwd_kv_kernel",
    "attn_bwd_q": "attn_bwd_q_kernel",
    "attn_cand": "attn_cand_kernel",
    "head_gemm": "gemm_kernel",
    "copy": "copyBuffer",
}
SIMDS, CUS, XCDS = 1024, 256, 8      # MI355X: 256 compute units of 4 SIMDs in 8 XCDs


def summarize_counters(csv_paths, kernels):
    """Per-dispatch averages of the counters in rocprofv3 --pmc CSV files
    (p_counter_collection.csv), for each named kernel, and the figures derived
    from them. Counters summed over the whole device per dispatch; the later
    half of each kernel's dispatches is used (after warm-up)."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))   # kernel -> counter -> [per dispatch]
    meta = {}
    for path in csv_paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"]
                for kname, subs in kernels.items():
                    if any(sub in name for sub in ((subs,) if isinstance(subs, str) else subs)):
                        # one entry per (kernel, grid size): a workload's launches of that kernel
                        key = f"{kname} grid {int(row['Grid_Size']) // int(row['Workgroup_Size'])}"
                        vals[key][row["Counter_Name"]].append((int(row["Dispatch_Id"]), float(row["Counter_Value"]),
                                                              int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
                        meta[key] = dict(vgpr=int(row["VGPR_Count"]), agpr=int(row["Accum_VGPR_Count"]),
                                         lds=int(row["LDS_Block_Size"]), wg=int(row["Workgroup_Size"]))
    out = {}
    for key, cs in vals.items():
        avg, ns = {}, []
        for cname, lst in cs.items():
            lst.sort()
            later = lst[len(lst) // 2:]
            avg[cname] = sum(v for _, v, _ in later) / len(later)
            ns += [d for _, _, d in later]
        r = {"dispatches": max(len(v) for v in cs.values()), "counters": {k: round(v, 1) for k, v in avg.items()},
             **meta.get(key, {})}
        g = avg.get("GRBM_GUI_ACTIVE")
        if g:
            # GRBM_GUI_ACTIVE is the sum over the XCDs: one XCD's busy cycles is that over XCDS
            g /= XCDS
            r["gui_active_cycles_per_xcd"] = round(g, 1)
            if ns:
                r["avg_clock_ghz"] = round(g / (sum(ns) / len(ns)), 3)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                r["mfma_busy_frac"] = round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * SIMDS), 4)
            if "SQ_LDS_IDX_ACTIVE" in avg:
                r["lds_active_frac"] = round(avg["SQ_LDS_IDX_ACTIVE"] / (g * CUS), 4)
        if avg.get("SQ_INSTS_MFMA"):
            m = avg["SQ_INSTS_MFMA"]
            for c, label in (("SQ_INSTS_VALU", "valu_per_mfma"), ("SQ_INSTS_SALU", "salu_per_mfma"),
                             ("SQ_INSTS_LDS", "lds_per_mfma")):
                if c in avg:
                    r[label] = round((avg[c] - (m if c == "SQ_INSTS_VALU" else 0)) / m, 3)
        if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
            r["coexec_frac_of_mfma_busy"] = round(avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg and ns:
            # 512 flops per MOP (the rocprofv3 derived-metric definition)
            r["mfma_bf16_tflops_from_counters"] = round(avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 /
                                                        (sum(ns) / len(ns) * 1e-9) / 1e12, 1)
        if ns:
            r["avg_dispatch_ns_under_profiler"] = round(sum(ns) / len(ns), 1)
        out[key] = r
    return out


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
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} of {wl.num_seqs * wl.num_heads} (sequence, head) units of the "
                      f"workload, fp64 NumPy oracle, {dt:.1f} s wall; BLAS threads {threads}, "
                      f"elementwise steps single-threaded"}


# Shortest warm-up by time: the shader clock ramps up over the first ~40 ms of
# sustained load, so warm-up continues past `--warmup` calls until this much
# wall time has passed.
MIN_WARMUP_MS = 200.0
WARMUP_DONE = {}   # label -> (calls, ms) of the warm-up actually run


def time_steps(step, steps: int, warmup: int, stream, label: str = "secondary"):
    """Warm up (at least `warmup` calls and at least MIN_WARMUP_MS of wall
    time), then time exactly `steps` calls between two synchronizations;
    returns (ms per step from HIP events on `stream`, ms per step of wall time)."""
    import torch
    t0 = time.perf_counter()
    calls = 0
    for _ in range(warmup):
        step()
        calls += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < MIN_WARMUP_MS:
        step()
        calls += 1
        torch.cuda.synchronize()
    WARMUP_DONE[label] = (calls, round((time.perf_counter() - t0) * 1e3, 1))
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    return ev0.elapsed_time(ev1) / steps, wall


def kernel_ms(hstu, step, steps: int, kernels):
    """Average launch time of each named kernel over `steps` further calls,
    from the events the library records around each launch."""
    import torch
    for k in kernels:
        hstu.timing_read(k)          # drop anything recorded before
    hstu.timing_enable(True)
    try:
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        out = {}
        for k in kernels:
            n, ms = hstu.timing_read(k)
            out[k] = ms / n if n else None
    finally:
        hstu.timing_enable(False)
    return out


def _attn_tensors(wl, dev):
    import torch
    t = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)  # noqa: E731
    d = dict(q=t(wl.q, torch.bfloat16), k=t(wl.k, torch.bfloat16), v=t(wl.v, torch.bfloat16),
             off=torch.from_numpy(wl.seq_offsets).to(dev),
             ts=torch.from_numpy(wl.timestamps).to(dev) if wl.timestamps is not None else None,
             pt=t(wl.pos_table, torch.float32) if wl.pos_table is not None else None,
             tt=t(wl.time_table, torch.float32) if wl.time_table is not None else None)
    if wl.d_o is not None:
        d["d_o"] = t(wl.d_o, torch.bfloat16)
    return d


def secondary_layers(hstu, name: str, steps: int, warmup: int, dev):
    """Tokens/s per layer of a layer workload (all its layers per step)."""
    import torch
    from workloads import make_workload
    wl = make_workload(name)
    x0 = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    off = torch.from_numpy(wl.seq_offsets).to(dev)
    ts = torch.from_numpy(wl.timestamps).to(dev) if wl.timestamps is not None else None
    keep, params = [], []
    for p in wl.layers:
        dv = {}
        for k in ("w_uvqk", "w_out"):
            dv[k] = torch.from_numpy(p[k]).to(dev).to(torch.bfloat16)
        for k in ("b_uvqk", "b_out", "ln_in_gamma", "ln_in_beta", "ln_out_gamma", "ln_out_beta",
                  "pos_table", "time_table"):
            dv[k] = None if p.get(k) is None else torch.from_numpy(p[k]).to(dev).to(torch.float32)
        keep.append(dv)
        params.append(hstu.make_layer_params(wl.embed_dim, wl.num_heads, wl.dqk, wl.dv, ln_eps=wl.ln_eps, **dv))
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)   # >= hstu_layer_workspace_size

    def step():
        x = x0
        for i, p in enumerate(params):
            x = hstu.layer_fwd(x, off, p, timestamps=ts, out=bufs[i & 1], workspace=ws)

    stream = torch.cuda.current_stream(dev)
    ms_ev, ms_wall = time_steps(step, steps, warmup, stream)
    ms = max(ms_ev, ms_wall)
    L = len(params)
    kern = kernel_ms(hstu, step, steps, ["attn_fwd", "layer_gemm_uvqk", "layer_gemm_out", "layer_norm"])
    per_layer = {k: (None if v is None else round(v * (1 if k != "layer_norm" else 2), 5))
                 for k, v in kern.items()}
    gemm_ms = (kern["layer_gemm_uvqk"] or 0) + (kern["layer_gemm_out"] or 0)
    return {
        "workload": f"{name}: {wl.note}",
        "tokens_per_s_per_layer": round(wl.total_tokens / (ms * 1e-3 / L), 1),
        "ms_per_layer": round(ms / L, 5),
        "layers": L,
        "total_tokens": wl.total_tokens,
        "kernel_ms_per_layer": per_layer,
        "gemm_tflops": round(wl.layer_gemm_flops() / (gemm_ms * 1e-3) / 1e12, 2) if gemm_ms else None,
        "attn_fwd_tflops": round(wl.attn_fwd_flops() / (kern["attn_fwd"] * 1e-3) / 1e12, 2)
        if kern["attn_fwd"] else None,
    }


def secondary_fwd_bwd(hstu, name: str, steps: int, warmup: int, dev):
    """Attention forward + backward of a training-step workload."""
    import torch
    from workloads import make_workload
    wl = make_workload(name)
    a = _attn_tensors(wl, dev)
    o = torch.empty_like(a["v"])
    grads = (torch.empty_like(a["q"]), torch.empty_like(a["k"]), torch.empty_like(a["v"]),
             torch.empty_like(a["pt"]) if a["pt"] is not None else None,
             torch.empty_like(a["tt"]) if a["tt"] is not None else None)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def fwd():
        hstu.attn_fwd(a["q"], a["k"], a["v"], a["off"], timestamps=a["ts"], pos_table=a["pt"],
                      time_table=a["tt"], alpha=wl.alpha, divisor=wl.divisor, out=o, workspace=ws)

    def bwd():
        hstu.attn_bwd(a["q"], a["k"], a["v"], a["d_o"], a["off"], timestamps=a["ts"], pos_table=a["pt"],
                      time_table=a["tt"], alpha=wl.alpha, divisor=wl.divisor, workspace=ws, out=grads)

    def step():
        fwd()
        bwd()

    stream = torch.cuda.current_stream(dev)
    ms_ev, ms_wall = time_steps(step, steps, warmup, stream)
    ms = max(ms_ev, ms_wall)
    kern = kernel_ms(hstu, step, steps, ["attn_fwd", "attn_bwd_kv", "attn_bwd_q"])
    F_f, F_b = wl.attn_fwd_flops(), wl.attn_bwd_flops()
    bwd_k = (kern["attn_bwd_kv"] or 0) + (kern["attn_bwd_q"] or 0)
    return {
        "workload": f"{name}: {wl.note}",
        "fwd_bwd_tflops": round((F_f + F_b) / (ms * 1e-3) / 1e12, 2),
        "ms_per_step": round(ms, 5),
        "total_tokens": wl.total_tokens,
        "kernel_ms": {k: (None if v is None else round(v, 5)) for k, v in kern.items()},
        "bwd_kernels_tflops": round(F_b / (bwd_k * 1e-3) / 1e12, 2) if bwd_k else None,
        "fwd_kernel_tflops": round(F_f / (kern["attn_fwd"] * 1e-3) / 1e12, 2) if kern["attn_fwd"] else None,
    }


def secondary_layer_fwd_bwd(hstu, name: str, steps: int, warmup: int, dev):
    """One layer forward + backward (a training step's layer) of a layer
    workload with an upstream gradient. Credited flops: the forward's and,
    for the backward, the attention backward plus two GEMMs per forward GEMM
    (the backward's recompute of the forward is not credited)."""
    import torch
    from workloads import make_workload
    wl = make_workload(name)
    p = wl.layers[0]
    dvt = {}
    for k in ("w_uvqk", "w_out"):
        dvt[k] = torch.from_numpy(p[k]).to(dev).to(torch.bfloat16)
    for k in ("b_uvqk", "b_out", "ln_in_gamma", "ln_in_beta", "ln_out_gamma", "ln_out_beta",
              "pos_table", "time_table"):
        dvt[k] = None if p.get(k) is None else torch.from_numpy(p[k]).to(dev).to(torch.float32)
    params = hstu.make_layer_params(wl.embed_dim, wl.num_heads, wl.dqk, wl.dv, ln_eps=wl.ln_eps, **dvt)
    x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    d_out = torch.from_numpy(wl.d_o).to(dev).to(torch.bfloat16)
    off = torch.from_numpy(wl.seq_offsets).to(dev)
    ts = torch.from_numpy(wl.timestamps).to(dev) if wl.timestamps is not None else None
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device=dev)   # >= either workspace size
    dx_, grads = hstu.layer_bwd(x, d_out, off, params, timestamps=ts, dx=dx, workspace=ws)

    def fwd():
        hstu.layer_fwd(x, off, params, timestamps=ts, out=y, workspace=ws)

    def bwd():
        hstu.layer_bwd(x, d_out, off, params, timestamps=ts, dx=dx, grads=grads, workspace=ws)

    def step():
        fwd()
        bwd()

    stream = torch.cuda.current_stream(dev)
    ms_f = max(time_steps(fwd, steps, warmup, stream))
    ms_b = max(time_steps(bwd, steps, warmup, stream))
    ms = max(time_steps(step, steps, warmup, stream))
    kern = kernel_ms(hstu, bwd, steps, ["attn_fwd", "attn_bwd_kv", "attn_bwd_q", "layer_gemm_uvqk",
                                        "layer_gemm_out", "layer_norm"])
    F_f = wl.attn_fwd_flops() + wl.layer_gemm_flops()
    F_b = wl.attn_bwd_flops() + 2.0 * wl.layer_gemm_flops()
    return {
        "workload": f"{name}: {wl.note}",
        "tokens_per_s": round(wl.total_tokens / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 5),
        "fwd_ms": round(ms_f, 5),
        "bwd_ms": round(ms_b, 5),
        "credited_tflops": round((F_f + F_b) / (ms * 1e-3) / 1e12, 2),
        "total_tokens": wl.total_tokens,
        "bwd_kernel_ms": {k: (None if v is None else round(v, 5)) for k, v in kern.items()},
    }


def secondary_candidates(hstu, name: str, steps: int, warmup: int, dev):
    """Candidate scoring against cached histories: candidates/s and
    causal-effective TFLOP/s (each candidate attends its history plus itself:
    512 flop per (candidate, key) pair per head at d = 128)."""
    import torch
    from workloads import make_workload
    wl = make_workload(name)
    c = wl.cand
    bf = torch.bfloat16
    t = lambda a, dt=None: torch.from_numpy(a).to(dev) if dt is None else torch.from_numpy(a).to(dev).to(dt)
    q, k, v = t(c["q"], bf), t(c["k"], bf), t(c["v"], bf)
    kh, vh = t(wl.k, bf), t(wl.v, bf)
    coff, hoff = t(c["offsets"]), t(wl.seq_offsets)
    ts, cts = t(wl.timestamps), t(c["timestamps"])
    pt, tt = t(wl.pos_table, torch.float32), t(wl.time_table, torch.float32)
    out = torch.empty_like(v)
    m = np.diff(c["offsets"])
    mmax = int(m.max())
    ws = torch.empty(max(1, hstu.attn_cand_workspace_size(wl.num_heads, wl.dqk, wl.num_seqs, wl.total_tokens, mmax)),
                     dtype=torch.uint8, device=dev)

    def step():
        hstu.attn_fwd_candidates(q, k, v, coff, kh, vh, hoff, timestamps=ts, cand_timestamps=cts,
                                 pos_table=pt, time_table=tt, max_candidates=mmax, out=out, workspace=ws)

    stream = torch.cuda.current_stream(dev)
    ms_ev, ms_wall = time_steps(step, steps, warmup, stream)
    ms = max(ms_ev, ms_wall)
    kern = kernel_ms(hstu, step, steps, ["attn_cand"])["attn_cand"]
    pairs = float(np.sum(m * (np.diff(wl.seq_offsets) + 1))) * wl.num_heads
    F = pairs * 2.0 * (wl.dqk + wl.dv)
    return {
        "workload": f"{name}: {wl.note}",
        "candidates_per_s": round(float(m.sum()) / (ms * 1e-3), 1),
        "tflops": round(F / (ms * 1e-3) / 1e12, 2),
        "ms_per_step": round(ms, 5),
        "kernel_ms": round(kern, 5) if kern else None,
        "kernel_tflops": round(F / (kern * 1e-3) / 1e12, 2) if kern else None,
    }


def secondary_head(hstu, name: str, steps: int, warmup: int, dev):
    """Final RMSNorm + tied retrieval head: token rows/s, TFLOP/s of the
    logits GEMM (2 D flop per (row, item) pair) and its bf16 logits write rate."""
    import torch
    from workloads import make_workload
    wl = make_workload(name)
    h = wl.head
    x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    table = torch.from_numpy(h["table"]).to(dev).to(torch.bfloat16)
    gamma = None if h["gamma"] is None else torch.from_numpy(h["gamma"]).to(dev)
    rows, vocab = x.shape[0], table.shape[0]
    out = torch.empty((rows, vocab), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(hstu.head_workspace_size(rows, wl.embed_dim), dtype=torch.uint8, device=dev)

    def step():
        hstu.head_fwd(x, table, gamma=gamma, eps=h["eps"], out=out, workspace=ws)

    stream = torch.cuda.current_stream(dev)
    ms_ev, ms_wall = time_steps(step, steps, warmup, stream)
    ms = max(ms_ev, ms_wall)
    kern = kernel_ms(hstu, step, steps, ["head_rms_norm", "head_gemm"])
    F = 2.0 * rows * vocab * wl.embed_dim
    kg = kern["head_gemm"]
    return {
        "workload": f"{name}: {wl.note}",
        "rows_per_s": round(rows / (ms * 1e-3), 1),
        "tflops": round(F / (ms * 1e-3) / 1e12, 2),
        "ms_per_step": round(ms, 5),
        "kernel_ms": {k: (round(v, 5) if v else None) for k, v in kern.items()},
        "gemm_tflops": round(F / (kg * 1e-3) / 1e12, 2) if kg else None,
        "gemm_logits_write_gbs": round(rows * vocab * 2 / (kg * 1e-3) / 1e9, 1) if kg else None,
    }


def secondary_stochastic_length(hstu, name: str, steps: int, warmup: int, dev):
    """Stochastic Length: one step = the keyed selection (new offsets and
    gather index) plus the gathers of the kept token rows and timestamps.
    Input tokens/s, and the step's algorithmic bytes (keys read once, index
    written once and read by both gathers, rows and timestamps read and
    written once) per second."""
    import torch
    from workloads import make_workload
    wl = make_workload(name)
    L = wl.sl["max_len"]
    off = torch.from_numpy(wl.seq_offsets).to(dev)
    keys = torch.from_numpy(wl.sl["keys"].view(np.int32)).to(dev)
    x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    ts = torch.from_numpy(wl.timestamps).to(dev)
    T = wl.total_tokens
    new_off = torch.empty(wl.num_seqs + 1, dtype=torch.int64, device=dev)
    idx = torch.empty(T, dtype=torch.int64, device=dev)
    xo = torch.empty_like(x)
    tso = torch.empty_like(ts)
    count = new_off[-1:]

    def step():
        hstu.stochastic_length(off, keys, L, new_offsets=new_off, gather_index=idx)
        hstu.gather_rows(x, idx, count, T, out=xo)
        hstu.gather_rows(ts, idx, count, T, out=tso)

    stream = torch.cuda.current_stream(dev)
    ms_ev, ms_wall = time_steps(step, steps, warmup, stream)
    ms = max(ms_ev, ms_wall)
    kern = kernel_ms(hstu, step, steps, ["sl_select", "gather_rows"])
    Tn = int(np.minimum(wl.lengths, L).sum())
    row = wl.embed_dim * 2 + 8
    nbytes = 4 * T + 8 * Tn + 2 * 8 * Tn + 2 * row * Tn
    return {
        "workload": f"{name}: {wl.note}",
        "input_tokens_per_s": round(T / (ms * 1e-3), 1),
        "kept_tokens": Tn,
        "ms_per_step": round(ms, 5),
        "algorithmic_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "kernel_ms": {k: (round(v, 5) if v else None) for k, v in kern.items()},
    }


SECONDARY = ("layer_stack", "layer_jagged", "attn_fwd_bwd", "layer_fwd_bwd", "candidates", "head",
             "stochastic_length")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c3", help="attention-forward workload of the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default=",".join(SECONDARY),
                    help="comma-separated secondary figures to run (default: all)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="print per-kernel averages and derived figures of rocprofv3 --pmc CSV files and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters, COUNTER_KERNELS), indent=1))
        return

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
    a = _attn_tensors(wl, dev)
    out = torch.empty_like(a["v"])
    ws = torch.empty(hstu.attn_workspace_size(wl.num_heads, wl.dqk, wl.dv, torch.bfloat16,
                                              wl.num_seqs, wl.total_tokens), dtype=torch.uint8,
                     device=dev)

    def step():
        hstu.attn_fwd(a["q"], a["k"], a["v"], a["off"], timestamps=a["ts"], pos_table=a["pt"],
                      time_table=a["tt"], alpha=wl.alpha, divisor=wl.divisor, out=out, workspace=ws)

    stream = torch.cuda.current_stream(dev)   # the stream every kernel is launched on
    ms_events, ms_wall = time_steps(step, args.steps, args.warmup, stream, label="headline")
    ms_step = max(ms_events, ms_wall)
    kern = kernel_ms(hstu, step, args.steps, ["attn_fwd"])["attn_fwd"]

    flops = wl.attn_fwd_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kern * 1e-3) / 1e12
    ctr = _counters()

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"calls": WARMUP_DONE["headline"][0], "ms": WARMUP_DONE["headline"][1],
                       "min_ms": MIN_WARMUP_MS},
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
        "tokens_per_s": round(wl.total_tokens / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": ctr["bytes_per_launch"] if ctr else None,
            # from the same counter summary (null once the kernel changed):
            # MFMA-busy cycles over all SIMDs' cycles, and the HBM bytes per
            # launch over this run's average launch time
            "mfma_util": ctr["mfma_busy_frac"] if ctr else None,
            "hbm_gbs": round(ctr["bytes_per_launch"] / (kern * 1e-3) / 1e9, 1) if ctr else None,
            "kernel": f"attn_fwd_bf16_kernel<{wl.dqk},{wl.dv}>",
            "algorithmic_flops_per_launch": flops,
            "avg_launch_ms": round(kern, 5),
            "kernel_sha256_16": kernel_hash(),
        },
    }
    if not args.no_secondary:
        runs = {
            "layer_stack": lambda: secondary_layers(hstu, "c1", args.steps, args.warmup, dev),
            "layer_jagged": lambda: secondary_layers(hstu, "c2", max(5, args.steps // 5),
                                                     max(2, args.warmup // 10), dev),
            "attn_fwd_bwd": lambda: secondary_fwd_bwd(hstu, "c4", args.steps, args.warmup, dev),
            "layer_fwd_bwd": lambda: secondary_layer_fwd_bwd(hstu, "c5", max(5, args.steps // 5),
                                                             max(2, args.warmup // 10), dev),
            "candidates": lambda: secondary_candidates(hstu, "c6", max(5, args.steps // 2),
                                                       max(5, args.warmup // 4), dev),
            "head": lambda: secondary_head(hstu, "c7", max(5, args.steps // 4), max(5, args.warmup // 10), dev),
            "stochastic_length": lambda: secondary_stochastic_length(hstu, "c8", args.steps,
                                                                     max(5, args.warmup // 4), dev),
        }
        wanted = [w for w in args.secondary.split(",") if w]
        unknown = sorted(set(wanted) - set(runs))
        if unknown:
            ap.error(f"unknown secondary figure(s): {unknown}")
        res["secondary"] = {w: runs[w]() for w in wanted}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
