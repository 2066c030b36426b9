"""GPU parity of hstu_layer_bwd (one HSTU layer's input and parameter
gradients) against the fp64 oracle's chain-rule backward, through the C ABI.
Every gradient tensor is held to the bf16 tolerance separately."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import TOL_BF16, rel_err, to_dev
from workloads import make_workload

pytestmark = pytest.mark.gpu

PARAM_KEYS = ("w_uvqk", "b_uvqk", "w_out", "b_out", "ln_in_gamma", "ln_in_beta", "ln_out_gamma",
              "ln_out_beta", "pos_table", "time_table")


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _dev_params(hstu, wl, p):
    import torch
    keep = {}
    for name in ("w_uvqk", "w_out"):
        keep[name] = to_dev(p[name], torch.bfloat16)
    for name in ("b_uvqk", "b_out", "ln_in_gamma", "ln_in_beta", "ln_out_gamma", "ln_out_beta",
                 "pos_table", "time_table"):
        keep[name] = None if p.get(name) is None else to_dev(p[name], torch.float32)
    params = hstu.make_layer_params(wl.embed_dim, wl.num_heads, wl.dqk, wl.dv, ln_eps=wl.ln_eps, **keep)
    return params, keep


def _gpu_bwd(hstu, wl, p, x=None, d_out=None, off=None, ts=None):
    import torch
    params, keep = _dev_params(hstu, wl, p)
    x = to_dev(wl.x if x is None else x, torch.bfloat16)
    d_out = to_dev(wl.d_o if d_out is None else d_out, torch.bfloat16)
    off = to_dev(wl.seq_offsets if off is None else off)
    ts = wl.timestamps if ts is None else ts
    ts = None if ts is None else to_dev(ts)
    dx, grads = hstu.layer_bwd(x, d_out, off, params, timestamps=ts)
    torch.cuda.synchronize()
    return dx.float().cpu().numpy(), {k: v.cpu().numpy() for k, v in grads.items()}


def _oracle(wl, p, x=None, d_out=None, off=None, ts=None):
    return orc.layer_bwd(wl.x if x is None else x, p, wl.seq_offsets if off is None else off,
                         wl.d_o if d_out is None else d_out, num_heads=wl.num_heads, dqk=wl.dqk,
                         dv=wl.dv, timestamps=wl.timestamps if ts is None else ts, eps=wl.ln_eps)


def _compare(label, got, ref):
    gdx, gg = got
    rdx, rg = ref
    errs = {"dx": rel_err(gdx, rdx)}
    assert set(gg) == set(rg), (sorted(gg), sorted(rg))
    for k in rg:
        assert np.all(np.isfinite(gg[k])), f"{label}: {k} not finite"
        errs[k] = rel_err(gg[k], rg[k])
    print(label, " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL_BF16, f"{label}: {k} error {e:.3e}"


def test_reduced_jagged_layer_backward(hstu):
    """7 ragged sequences (lengths 1 to 159), pos + time bias, every gradient."""
    wl = make_workload("c5_small")
    p = wl.layers[0]
    _compare("c5_small", _gpu_bwd(hstu, wl, p), _oracle(wl, p))


def test_full_size_layer_backward(hstu):
    """32 sequences log-uniform in [64, 2048] (20074 tokens), D 512, H 4, d 128,
    pos + time bias: every element of every gradient against the oracle."""
    wl = make_workload("c5")
    p = wl.layers[0]
    _compare("c5", _gpu_bwd(hstu, wl, p), _oracle(wl, p))


def test_nonzero_linear_biases_and_affine_norms(hstu):
    """Linear biases and LayerNorm affine parameters away from their b = 0,
    gamma = 1, beta = 0 initial values, and no time table."""
    wl = make_workload("c5_small")
    rng = np.random.default_rng(41)
    p = dict(wl.layers[0])
    D, n1, hv = wl.embed_dim, p["w_uvqk"].shape[0], p["w_out"].shape[1]
    p["b_uvqk"] = (0.1 * rng.standard_normal(n1)).astype(np.float32)
    p["b_out"] = (0.1 * rng.standard_normal(D)).astype(np.float32)
    p["ln_in_gamma"] = (1 + 0.2 * rng.standard_normal(D)).astype(np.float32)
    p["ln_in_beta"] = (0.2 * rng.standard_normal(D)).astype(np.float32)
    p["ln_out_gamma"] = (1 + 0.2 * rng.standard_normal(hv)).astype(np.float32)
    p["ln_out_beta"] = (0.2 * rng.standard_normal(hv)).astype(np.float32)
    p["time_table"] = None
    _compare("biased, no time table", _gpu_bwd(hstu, wl, p, ts=None), _oracle(wl, p, ts=None))


def test_empty_batch_zero_gradients(hstu):
    """No tokens: every parameter gradient is exactly zero."""
    import torch
    wl = make_workload("c5_small")
    p = wl.layers[0]
    params, keep = _dev_params(hstu, wl, p)
    x = torch.empty((0, wl.embed_dim), dtype=torch.bfloat16, device="cuda:0")
    off = to_dev(np.zeros(3, np.int64))
    dx, grads = hstu.layer_bwd(x, x.clone(), off, params,
                               timestamps=torch.empty(0, dtype=torch.int64, device="cuda:0"))
    torch.cuda.synchronize()
    for k, v in grads.items():
        assert not torch.any(v != 0), k


def test_deterministic(hstu):
    wl = make_workload("c5_small")
    p = wl.layers[0]
    a = _gpu_bwd(hstu, wl, p)
    b = _gpu_bwd(hstu, wl, p)
    assert np.array_equal(a[0], b[0])
    for k in a[1]:
        assert np.array_equal(a[1][k], b[1][k]), k


def test_wider_layer_backward_d1024_h8(hstu):
    """D = 1024 with 8 heads of 128: the 1024-wide LayerNorm backward and the
    weight-gradient GEMMs at another width, 5 ragged sequences."""
    from workloads.generators import _layer_recipe
    wl = _layer_recipe("wide_bwd", 37, lengths=[130, 1, 0, 257, 64], num_layers=1, D=1024, H=8, time=True,
                       backward=True)
    p = wl.layers[0]
    _compare("D 1024 H 8", _gpu_bwd(hstu, wl, p), _oracle(wl, p))
