"""The oracle's layer stack evaluated with every stored activation rounded to
bfloat16 (test infrastructure).

The stack workload prescribes bf16 weights and activations with fp32
accumulation. A GPU pipeline that stores LN(X), G = SiLU(Z), O, Y and X' in
bf16 between its steps therefore differs from the all-fp64 oracle by the
rounding of those stores, and that difference compounds over layers. This
module evaluates the same layers with the oracle's own functions (LayerNorm,
SiLU, attention), in fp64, rounding to bf16 (nearest, ties to even) at exactly
those five points -- nothing else of the GPU path is imitated. The gap between
this pipeline and the fp64 stack is the part of the error that storage
precision alone causes, whatever the kernels do.
"""

from __future__ import annotations

import numpy as np

from oracle import oracle as orc
from workloads.generators import round_to_bf16


def _bf16(x: np.ndarray) -> np.ndarray:
    return round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def layer_fwd_bf16_storage(x, p: dict, seq_offsets, *, num_heads: int, dqk: int, dv: int,
                           timestamps=None, eps: float = 1e-6):
    """One layer of ``oracle.layer_fwd`` with LN(X), G, O, Y and X' rounded to
    bf16 where the GPU path stores them."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    H = num_heads
    xn = _bf16(orc.layer_norm(x, p["ln_in_gamma"], p["ln_in_beta"], eps))
    z = xn @ np.asarray(p["w_uvqk"], np.float64).T
    if p.get("b_uvqk") is not None:
        z = z + np.asarray(p["b_uvqk"], np.float64)
    g = _bf16(orc.silu(z))
    u = g[:, 0:H * dv]
    v = g[:, H * dv:2 * H * dv].reshape(T, H, dv)
    q = g[:, 2 * H * dv:2 * H * dv + H * dqk].reshape(T, H, dqk)
    k = g[:, 2 * H * dv + H * dqk:].reshape(T, H, dqk)
    o = _bf16(orc.attn_fwd(q, k, v, seq_offsets, pos_table=p.get("pos_table"), time_table=p.get("time_table"),
                           timestamps=timestamps).reshape(T, H * dv))
    y = _bf16(orc.layer_norm(o, p["ln_out_gamma"], p["ln_out_beta"], eps) * u)
    out = x + y @ np.asarray(p["w_out"], np.float64).T
    if p.get("b_out") is not None:
        out = out + np.asarray(p["b_out"], np.float64)
    return _bf16(out)


def stack_errors(wl):
    """Per number of layers L = 1 .. len(wl.layers): (the bf16-storage stack's
    output after L layers, the fp64 stack's output after L layers, and the
    error max|a - b| / max|b| between them)."""
    h64 = np.asarray(wl.x, np.float64)
    hbf = np.asarray(wl.x, np.float64)
    out = []
    for p in wl.layers:
        h64, _ = orc.layer_fwd(h64, p, wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk, dv=wl.dv,
                               timestamps=wl.timestamps, eps=wl.ln_eps)
        hbf = layer_fwd_bf16_storage(hbf, p, wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk, dv=wl.dv,
                                     timestamps=wl.timestamps, eps=wl.ln_eps)
        err = float(np.max(np.abs(hbf - h64)) / np.max(np.abs(h64)))
        out.append((hbf.copy(), h64.copy(), err))
    return out
