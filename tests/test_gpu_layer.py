"""GPU parity of hstu_layer_fwd (one HSTU layer, and a stack of them) against
the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import TOL_BF16, rel_err, to_dev
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _dev_layer(hstu, wl, p):
    """Device copies of one layer's parameters and the hstu_layer_params_t
    (the tensors are returned so they outlive the call)."""
    import torch
    keep = {}
    for name in ("w_uvqk", "w_out"):
        keep[name] = to_dev(p[name], torch.bfloat16)
    for name in ("b_uvqk", "b_out", "ln_in_gamma", "ln_in_beta", "ln_out_gamma", "ln_out_beta",
                 "pos_table", "time_table"):
        keep[name] = None if p.get(name) is None else to_dev(p[name], torch.float32)
    params = hstu.make_layer_params(wl.embed_dim, wl.num_heads, wl.dqk, wl.dv, ln_eps=wl.ln_eps,
                                    **{k: v for k, v in keep.items()})
    return params, keep


def _run_stack(hstu, wl, layers=None, want_intermediates=False):
    import torch
    layers = wl.layers if layers is None else layers
    x = to_dev(wl.x, torch.bfloat16)
    off = to_dev(wl.seq_offsets)
    ts = None if wl.timestamps is None else to_dev(wl.timestamps)
    T = wl.total_tokens
    H, d = wl.num_heads, wl.dqk
    inter = {}
    for li, p in enumerate(layers):
        params, keep = _dev_layer(hstu, wl, p)
        g = torch.empty((T, H * 4 * d), dtype=torch.bfloat16, device=x.device) if want_intermediates else None
        o = torch.empty((T, H * d), dtype=torch.bfloat16, device=x.device) if want_intermediates else None
        x = hstu.layer_fwd(x, off, params, timestamps=ts, uvqk_out=g, o_out=o)
        if want_intermediates:
            inter[li] = (g, o)
    torch.cuda.synchronize()
    out = x.float().cpu().numpy()
    if want_intermediates:
        inter = {k: (g.float().cpu().numpy(), o.float().cpu().numpy()) for k, (g, o) in inter.items()}
    return out, inter


def test_one_layer_reduced_jagged_with_intermediates(hstu):
    wl = make_workload("c2_small")
    out, inter = _run_stack(hstu, wl, want_intermediates=True)
    ref, parts = orc.layer_fwd(wl.x, wl.layers[0], wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk,
                               dv=wl.dv, timestamps=wl.timestamps, eps=wl.ln_eps)
    g, o = inter[0]
    e_g, e_o, e_x = rel_err(g, parts["uvqk"]), rel_err(o, parts["o"]), rel_err(out, ref)
    print(f"c2_small: uvqk {e_g:.2e}  o {e_o:.2e}  x' {e_x:.2e}")
    assert e_g <= TOL_BF16 and e_o <= TOL_BF16 and e_x <= TOL_BF16


def test_two_layer_stack_ragged(hstu):
    wl = make_workload("c1_small")
    out, _ = _run_stack(hstu, wl)
    ref = orc.stack_fwd(wl.x, wl.layers, wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk,
                        dv=wl.dv, timestamps=wl.timestamps, eps=wl.ln_eps)
    err = rel_err(out, ref)
    print(f"c1_small stack err {err:.2e}")
    assert err <= TOL_BF16


def test_zero_output_projection_returns_input_bitwise(hstu):
    wl = make_workload("c2_small")
    p = dict(wl.layers[0])
    p["w_out"] = np.zeros_like(p["w_out"])
    out, _ = _run_stack(hstu, wl, layers=[p])
    assert np.array_equal(out, wl.x)


def test_nonzero_biases_and_affine_norms(hstu):
    wl = make_workload("c2_small")
    rng = np.random.default_rng(21)
    p = dict(wl.layers[0])
    for name in ("b_uvqk", "b_out", "ln_in_beta", "ln_out_beta"):
        p[name] = (0.1 * rng.standard_normal(p[name].shape)).astype(np.float32)
    for name in ("ln_in_gamma", "ln_out_gamma"):
        p[name] = (1 + 0.2 * rng.standard_normal(p[name].shape)).astype(np.float32)
    out, _ = _run_stack(hstu, wl, layers=[p])
    ref, _ = orc.layer_fwd(wl.x, p, wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk, dv=wl.dv,
                           timestamps=wl.timestamps, eps=wl.ln_eps)
    assert rel_err(out, ref) <= TOL_BF16


def test_four_layer_stack_full_size(hstu):
    """The 4-layer, 8 x 1024-token stack at full size.

    - Each layer against the oracle layer applied to the same input (the
      previous GPU layer's bf16 output), at the bf16 tolerance.
    - The whole stack against the all-fp64 stack. The workload stores every
      activation in bf16 between steps, and that storage alone moves the
      oracle's own stack e_s = 1.7e-2 from fp64 after four layers (the oracle
      evaluated with LN(X), G, O, Y, X' rounded where they are stored,
      tests/bf16_storage.py; pinned on the CPU by tests/test_stack_precision.py).
      The bound is that storage error plus the bf16 tolerance that each layer's
      kernels are held to: e_s + 1e-2, computed here from the emulation, not
      picked by hand.
    """
    import torch
    from tests.bf16_storage import stack_errors
    wl = make_workload("c1")
    x_gpu = to_dev(wl.x, torch.bfloat16)
    off = to_dev(wl.seq_offsets)
    ts = None if wl.timestamps is None else to_dev(wl.timestamps)
    for li, p in enumerate(wl.layers):
        params, keep = _dev_layer(hstu, wl, p)
        x_in = x_gpu.float().cpu().numpy()
        x_gpu = hstu.layer_fwd(x_gpu, off, params, timestamps=ts)
        torch.cuda.synchronize()
        ref, _ = orc.layer_fwd(x_in, p, wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk, dv=wl.dv,
                               timestamps=wl.timestamps, eps=wl.ln_eps)
        err = rel_err(x_gpu.float().cpu().numpy(), ref)
        print(f"c1 layer {li}: err {err:.2e} (same input)")
        assert err <= TOL_BF16
    got = x_gpu.float().cpu().numpy()
    emu, ref64, e_s = stack_errors(wl)[-1]
    bound = e_s + TOL_BF16
    err = rel_err(got, ref64)
    print(f"c1 4-layer end-to-end vs fp64: {err:.2e}; bound {bound:.2e} = bf16-storage error {e_s:.2e} + "
          f"{TOL_BF16:.0e}; vs the bf16-storage stack: {rel_err(got, emu):.2e}")
    assert err <= bound


def test_jagged_layer_full_size_every_row(hstu):
    """One layer over the 64-sequence jagged batch at full size (49 404 tokens,
    lengths log-uniform in [32, 4096]): every output row against the oracle."""
    wl = make_workload("c2")
    out, _ = _run_stack(hstu, wl)
    assert np.all(np.isfinite(out))
    ref, _ = orc.layer_fwd(wl.x, wl.layers[0], wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk, dv=wl.dv,
                           timestamps=wl.timestamps, eps=wl.ln_eps)
    err = rel_err(out, ref)
    print(f"c2 every row: err {err:.2e} over {out.shape[0]} rows")
    assert err <= TOL_BF16


def test_wider_layer_d1024_h8(hstu):
    """D = 1024 with 8 heads of 128 (H dv = 1024, G 4096 wide): the 1024-wide
    LayerNorms and both GEMM shapes at another width, 5 ragged sequences."""
    from workloads.generators import _layer_recipe
    wl = _layer_recipe("wide", 31, lengths=[130, 1, 0, 257, 64], num_layers=1, D=1024, H=8, time=True)
    got, _ = _run_stack(hstu, wl)
    ref, _ = orc.layer_fwd(wl.x, wl.layers[0], wl.seq_offsets, num_heads=wl.num_heads, dqk=wl.dqk, dv=wl.dv,
                           timestamps=wl.timestamps, eps=wl.ln_eps)
    err = rel_err(got, ref)
    print(f"D 1024 H 8 layer err {err:.2e}")
    assert err <= TOL_BF16
