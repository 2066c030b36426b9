"""GPU parity of hstu_head_fwd (final RMSNorm + tied retrieval head) against
the fp64 oracle, through the C ABI: every logit of the reduced case, sampled
rows and item columns of the 8192 x 200000 case, and the tied-weight
self-retrieval property at full size."""

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


@pytest.fixture(scope="module")
def c7():
    return make_workload("c7")


def _run(hstu, x, table, gamma, eps):
    import torch
    out = hstu.head_fwd(to_dev(x, torch.bfloat16), to_dev(table, torch.bfloat16),
                        gamma=None if gamma is None else to_dev(gamma, torch.float32), eps=eps)
    torch.cuda.synchronize()
    return out


def test_reduced_head_every_logit(hstu):
    """300 rows x 1000 items (ragged against 256 x 256 tiles), gamma away from ones."""
    wl = make_workload("c7_small")
    h = wl.head
    got = _run(hstu, wl.x, h["table"], h["gamma"], h["eps"]).float().cpu().numpy()
    ref = orc.head_fwd(wl.x, h["table"], h["gamma"], h["eps"])
    err = rel_err(got, ref)
    print("c7_small", f"{err:.2e}")
    assert got.shape == ref.shape
    assert err <= TOL_BF16


def test_null_gamma_is_ones(hstu):
    import torch
    wl = make_workload("c7_small")
    h = wl.head
    a = _run(hstu, wl.x, h["table"], None, h["eps"])
    b = _run(hstu, wl.x, h["table"], np.ones(wl.embed_dim, np.float32), h["eps"])
    assert torch.equal(a, b)


def test_full_size_sampled_rows_and_items(hstu, c7):
    """8192 x 200000 logits in the launch configuration of the benchmark:
    48 whole rows (every item) and 48 whole item columns (every row)."""
    import torch
    h = c7.head
    out = _run(hstu, c7.x, h["table"], h["gamma"], h["eps"])
    rng = np.random.default_rng(77)
    rows = np.concatenate([[0, c7.x.shape[0] - 1], rng.choice(c7.x.shape[0], 46, replace=False)])
    cols = np.concatenate([[0, h["table"].shape[0] - 1], rng.choice(h["table"].shape[0], 46, replace=False)])
    got_r = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref_r = orc.head_fwd(c7.x[rows], h["table"], h["gamma"], h["eps"])
    got_c = out[:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
    ref_c = orc.head_fwd(c7.x, h["table"][cols], h["gamma"], h["eps"])
    er, ec = rel_err(got_r, ref_r), rel_err(got_c, ref_c)
    print("c7 rows", f"{er:.2e}", "cols", f"{ec:.2e}")
    assert er <= TOL_BF16 and ec <= TOL_BF16
    assert bool(torch.isfinite(out).all())


def test_tied_self_retrieval_at_full_size(hstu, c7):
    """Tied weights: token rows that are the table's own rows score their own
    item highest (Cauchy-Schwarz, with the table's near-equal row norms)."""
    import torch
    h = c7.head
    ids = np.random.default_rng(78).integers(0, h["table"].shape[0], size=8192)
    table = to_dev(h["table"], torch.bfloat16)
    x = table[torch.from_numpy(ids).cuda()].contiguous()
    out = hstu.head_fwd(x, table, eps=h["eps"])
    best = out.float().argmax(dim=1).cpu().numpy()
    assert np.array_equal(best, ids)


def test_empty_inputs_launch_nothing(hstu):
    import torch
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda:0")
    t = torch.zeros((64, 512), dtype=torch.bfloat16, device="cuda:0")
    assert hstu.head_fwd(x, t).shape == (0, 64)
    out = torch.full((5, 0), 1.0, dtype=torch.bfloat16, device="cuda:0")
    x5 = torch.ones((5, 512), dtype=torch.bfloat16, device="cuda:0")
    e = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda:0")
    assert hstu.head_fwd(x5, e, out=out).shape == (5, 0)


def test_rejects_vocab_not_multiple_of_eight(hstu):
    import torch
    x = torch.ones((4, 512), dtype=torch.bfloat16, device="cuda:0")
    t = torch.ones((12, 512), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(hstu.HstuError):
        hstu.head_fwd(x, t)


def test_deterministic(hstu):
    import torch
    wl = make_workload("c7_small")
    h = wl.head
    a = _run(hstu, wl.x, h["table"], h["gamma"], h["eps"])
    b = _run(hstu, wl.x, h["table"], h["gamma"], h["eps"])
    assert torch.equal(a, b)


def test_dim_1024_with_strided_rows_and_logits(hstu):
    """dim 1024 (the other built width): x a column view of a wider buffer,
    logits written into a buffer whose rows are padded past the vocabulary."""
    import torch
    rng = np.random.default_rng(79)
    rows, dim, vocab = 130, 1024, 520
    xw = (rng.standard_normal((rows, dim + 64)) * rng.uniform(0.1, 4.0, (rows, 1))).astype(np.float32)
    table = (0.02 * rng.standard_normal((vocab, dim))).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(dim)).astype(np.float32)
    xd = to_dev(xw, torch.bfloat16)[:, 32:32 + dim]
    out_buf = torch.full((rows, vocab + 24), -5.0, dtype=torch.bfloat16, device="cuda:0")
    out = out_buf[:, :vocab]
    hstu.head_fwd(xd, to_dev(table, torch.bfloat16), gamma=to_dev(gamma, torch.float32), eps=1e-6, out=out)
    torch.cuda.synchronize()
    xr = xd.float().cpu().numpy()
    tr = to_dev(table, torch.bfloat16).float().cpu().numpy()
    ref = orc.head_fwd(xr, tr, gamma, 1e-6)
    err = rel_err(out.float().cpu().numpy(), ref)
    print(f"dim 1024 strided err {err:.2e}")
    assert err <= TOL_BF16
    assert bool((out_buf[:, vocab:] == -5.0).all())   # padding untouched


def test_looping_workgroups_ragged_rows_and_padded_logits(hstu):
    """600 rows x 24008 items at dim 512: 3 x 94 tiles of 256 x 256, more
    than the compute units, so workgroups loop over tiles and request the next
    tile's first stage before storing the current one; rows and items ragged
    against the tiles, logits written into rows padded past the vocabulary.
    Every logit against the oracle."""
    import torch
    rng = np.random.default_rng(83)
    rows, dim, vocab = 600, 512, 24008
    x = (rng.standard_normal((rows, dim)) * rng.uniform(0.1, 4.0, (rows, 1))).astype(np.float32)
    table = (0.02 * rng.standard_normal((vocab, dim))).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(dim)).astype(np.float32)
    xd = to_dev(x, torch.bfloat16)
    td = to_dev(table, torch.bfloat16)
    out_buf = torch.full((rows, vocab + 40), -5.0, dtype=torch.bfloat16, device="cuda:0")
    out = out_buf[:, :vocab]
    hstu.head_fwd(xd, td, gamma=to_dev(gamma, torch.float32), eps=1e-6, out=out)
    torch.cuda.synchronize()
    ref = orc.head_fwd(xd.float().cpu().numpy(), td.float().cpu().numpy(), gamma, 1e-6)
    err = rel_err(out.float().cpu().numpy(), ref)
    print(f"looping head err {err:.2e}")
    assert err <= TOL_BF16
    assert bool((out_buf[:, vocab:] == -5.0).all())   # padding untouched
