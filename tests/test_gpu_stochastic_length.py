"""GPU parity of hstu_stochastic_length and hstu_gather_rows against the
oracle, through the C ABI: the shortened batch's offsets and gather index
bit for bit, and the gathered token rows and timestamps byte for byte."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import to_dev
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _keys_dev(keys):
    return to_dev(np.ascontiguousarray(keys, np.uint32).view(np.int32))


def _select(hstu, off, keys, L):
    import torch
    new_off, idx = hstu.stochastic_length(to_dev(np.asarray(off, np.int64)), _keys_dev(keys), L)
    torch.cuda.synchronize()
    new_off = new_off.cpu().numpy()
    return new_off, idx[:int(new_off[-1])].cpu().numpy()


def _check_workload(hstu, wl):
    import torch
    L = wl.sl["max_len"]
    ref_off, ref_idx = orc.stochastic_length(wl.seq_offsets, wl.sl["keys"], L)
    off_d = to_dev(wl.seq_offsets)
    new_off, idx = hstu.stochastic_length(off_d, _keys_dev(wl.sl["keys"]), L)
    T = wl.total_tokens
    x = to_dev(wl.x, torch.bfloat16)
    ts = to_dev(wl.timestamps)
    count = new_off[-1:]
    xs = hstu.gather_rows(x, idx, count, T)
    tss = hstu.gather_rows(ts, idx, count, T)
    torch.cuda.synchronize()
    got_off = new_off.cpu().numpy()
    Tn = int(got_off[-1])
    assert np.array_equal(got_off, ref_off)
    assert np.array_equal(idx[:Tn].cpu().numpy(), ref_idx)
    xb = x.view(torch.int16).cpu().numpy()
    assert np.array_equal(xs[:Tn].view(torch.int16).cpu().numpy(), xb[ref_idx])
    assert np.array_equal(tss[:Tn].cpu().numpy(), wl.timestamps[ref_idx])
    return Tn


def test_reduced_batch_with_ties_and_lengths_around_the_cap(hstu):
    """Lengths 5000, 0, 1, 300, 299, 301, 77, 2049 at cap 300; one sequence
    with 16 distinct keys, one with every key equal."""
    Tn = _check_workload(hstu, make_workload("c8_small"))
    assert Tn == 300 + 0 + 1 + 300 + 299 + 300 + 77 + 300


def test_full_size_batch(hstu):
    """64 sequences log-uniform in [64, 16384] (127956 tokens), cap 2048."""
    wl = make_workload("c8")
    Tn = _check_workload(hstu, wl)
    assert Tn == int(np.minimum(wl.lengths, 2048).sum())


@pytest.mark.parametrize("L", [0, 1, 2, 5000, 1 << 40])
def test_caps_from_zero_to_beyond_every_length(hstu, L):
    wl = make_workload("c8_small")
    got = _select(hstu, wl.seq_offsets, wl.sl["keys"], L)
    ref = orc.stochastic_length(wl.seq_offsets, wl.sl["keys"], L)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_empty_batches(hstu):
    import torch
    new_off, _ = hstu.stochastic_length(torch.zeros(1, dtype=torch.int64, device="cuda:0"),
                                        torch.zeros(0, dtype=torch.int32, device="cuda:0"), 4)
    assert new_off.cpu().tolist() == [0]
    got = _select(hstu, [0, 0, 0, 0], np.zeros(0, np.uint32), 4)
    assert got[0].tolist() == [0, 0, 0, 0] and got[1].size == 0


def test_extreme_keys_and_single_long_sequence(hstu):
    """One 70000-token sequence: keys 0 and 0xFFFFFFFF mixed with random ones."""
    rng = np.random.default_rng(90)
    n = 70000
    keys = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    keys[rng.choice(n, 500, replace=False)] = 0
    keys[rng.choice(n, 3000, replace=False)] = 0xFFFFFFFF
    for L in (499, 500, 501, 66999, 67000, 67001):
        got = _select(hstu, [0, n], keys, L)
        ref = orc.stochastic_length([0, n], keys, L)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), L


def test_gather_skips_out_of_range_indices_and_respects_max_rows(hstu):
    import torch
    src = torch.arange(40, dtype=torch.int32, device="cuda:0").reshape(10, 4)
    index = torch.tensor([3, -1, 10, 0, 9, 5], dtype=torch.int64, device="cuda:0")
    count = torch.tensor([6], dtype=torch.int64, device="cuda:0")
    out = torch.full((5, 4), -7, dtype=torch.int32, device="cuda:0")
    hstu.gather_rows(src, index, count, 5, out=out)
    o = out.cpu().numpy()
    s = src.cpu().numpy()
    assert np.array_equal(o[0], s[3]) and np.all(o[1] == -7) and np.all(o[2] == -7)
    assert np.array_equal(o[3], s[0]) and np.array_equal(o[4], s[9])


def test_deterministic(hstu):
    wl = make_workload("c8_small")
    a = _select(hstu, wl.seq_offsets, wl.sl["keys"], 300)
    b = _select(hstu, wl.seq_offsets, wl.sl["keys"], 300)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
