"""GPU parity at the relative-bias bucket edges (time buckets
floor(log2(1 + dt)) clamped to Bt - 1, position buckets min(i - j, Bp - 1)):
the forward (both work-list kernels and the fp32 kernel), the backward's key
and query passes and bias-table gradients, and candidate scoring, on inputs
where every output element is one pair's bias term (q = k = 0 or one-hot,
one-hot values; tests/bucket_edge_inputs.py). Pairs sit on the edges
2^k - 1 / 2^k - 2 in the 32-bit and the 64-bit gap ranges, and blocks of pairs
with one, two and many time buckets take the kernels' constant-bias,
compare-and-select and per-pair paths. tests/test_bucket_edge_fixture.py
shows on the CPU that any of the plausible bucket slips moves these outputs
by more than twice the tolerance."""

import numpy as np
import pytest

from tests import bucket_edge_inputs as E
from tests.helpers import TOL_BF16, TOL_F32, rel_err, to_dev
from tests.test_bucket_edge_fixture import (bwd_inputs, cand_inputs, fwd_inputs, oracle_bwd, oracle_cand,
                                            oracle_fwd)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _dev_all(a, dtype):
    import torch
    out = {}
    for key, x in a.items():
        if x is None:
            out[key] = None
        elif key in ("seq_offsets", "timestamps", "cand_offsets", "cand_timestamps"):
            out[key] = to_dev(x)
        elif key in ("pos_table", "time_table"):
            out[key] = to_dev(x, torch.float32)
        else:
            out[key] = to_dev(x, dtype)
    return out


@pytest.mark.parametrize("Bp,Bt,scale", E.CONFIGS)
@pytest.mark.parametrize("kind", ["short", "long", "f32"])
def test_forward_bucket_edges(hstu, kind, Bp, Bt, scale):
    """kind short: the work list is short (the key-range-split kernel);
    long: 600 empty sequences appended (one wave group per item); f32: the
    fp32 kernel."""
    import torch
    a = fwd_inputs(Bp, Bt, scale)
    ref = oracle_fwd(a)
    if kind == "long":
        off = a["seq_offsets"]
        a["seq_offsets"] = np.concatenate([off, np.full(600, off[-1], off.dtype)])
    d = _dev_all(a, torch.float32 if kind == "f32" else torch.bfloat16)
    print(f"forward edges: kind {kind} Bp {Bp} Bt {Bt} scale {scale}", flush=True)
    o = hstu.attn_fwd(d["q"], d["k"], d["v"], d["seq_offsets"], timestamps=d["timestamps"],
                      pos_table=d["pos_table"], time_table=d["time_table"], divisor=E.DIVISOR)
    torch.cuda.synchronize()
    err = rel_err(o.float().cpu().numpy(), ref)
    print(f"  err {err:.2e}")
    assert err <= (TOL_F32 if kind == "f32" else TOL_BF16)


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("variant", ["A", "B", "C"])
def test_backward_bucket_edges(hstu, variant, cfg):
    """A: dq = dS pair by pair (query pass); B: dk = dS^T pair by pair (key
    pass); C: one edge pair per row drives the bias-table gradients. Every
    gradient against the oracle."""
    import torch
    Bp, Bt, scale = E.CONFIGS[cfg]
    a = bwd_inputs(variant, Bp, Bt, scale)
    ref = oracle_bwd(a)
    d = _dev_all(a, torch.bfloat16)
    print(f"backward edges: variant {variant} Bp {Bp} Bt {Bt} scale {scale}", flush=True)
    got = hstu.attn_bwd(d["q"], d["k"], d["v"], d["d_o"], d["seq_offsets"], timestamps=d["timestamps"],
                        pos_table=d["pos_table"], time_table=d["time_table"], divisor=E.DIVISOR)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv", "d_pos", "d_time"), got, ref):
        g = g.float().cpu().numpy()
        if np.max(np.abs(r)) == 0:
            assert np.all(g == 0), name
            continue
        err = rel_err(g, r)
        print(f"  {name} err {err:.2e}")
        assert err <= TOL_BF16, name


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_candidate_bucket_edges(hstu, cfg):
    import torch
    Bp, Bt, scale = E.CONFIGS[cfg]
    a = cand_inputs(Bp, Bt, scale)
    ref = oracle_cand(a)
    d = _dev_all(a, torch.bfloat16)
    print(f"candidate edges: Bp {Bp} Bt {Bt} scale {scale}", flush=True)
    o = hstu.attn_fwd_candidates(d["q_c"], d["k_c"], d["v_c"], d["cand_offsets"], d["k_hist"], d["v_hist"],
                                 d["seq_offsets"], timestamps=d["timestamps"], cand_timestamps=d["cand_timestamps"],
                                 pos_table=d["pos_table"], time_table=d["time_table"], divisor=E.DIVISOR)
    torch.cuda.synchronize()
    err = rel_err(o.float().cpu().numpy(), ref)
    print(f"  err {err:.2e}")
    assert err <= TOL_BF16
