"""Shared helpers of the tests: device transfer of workload arrays and the
error measure of the tolerance rule  max|gpu - ref| <= tol * max|ref|."""

import numpy as np

TOL_F32 = 1e-5
TOL_BF16 = 1e-2


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(denom, 1e-300))


def to_dev(a, dtype=None, device="cuda:0"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def attn_inputs_on_device(wl, device="cuda:0"):
    """q, k, v, offsets, timestamps and tables of an attention workload as
    device tensors (bf16 or fp32 per the workload)."""
    import torch
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = dict(q=to_dev(wl.q, dt, device), k=to_dev(wl.k, dt, device), v=to_dev(wl.v, dt, device),
               seq_offsets=to_dev(wl.seq_offsets, None, device))
    out["timestamps"] = None if wl.timestamps is None else to_dev(wl.timestamps, None, device)
    out["pos_table"] = None if wl.pos_table is None else to_dev(wl.pos_table, torch.float32, device)
    out["time_table"] = None if wl.time_table is None else to_dev(wl.time_table, torch.float32, device)
    if wl.d_o is not None:
        out["d_o"] = to_dev(wl.d_o, dt, device)
    return out
