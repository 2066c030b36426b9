"""GPU parity of hstu_attn_fwd against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import TOL_BF16, TOL_F32, attn_inputs_on_device, rel_err, to_dev
from workloads import make_workload
from workloads.generators import _attn_recipe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _run(hstu, wl, **kw):
    import torch
    d = attn_inputs_on_device(wl)
    o = hstu.attn_fwd(d["q"], d["k"], d["v"], d["seq_offsets"], timestamps=d["timestamps"],
                      pos_table=d["pos_table"], time_table=d["time_table"], alpha=wl.alpha,
                      divisor=wl.divisor, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def _oracle(wl):
    return orc.attn_fwd(wl.q, wl.k, wl.v, wl.seq_offsets, alpha=wl.alpha, divisor=wl.divisor,
                        pos_table=wl.pos_table, time_table=wl.time_table, timestamps=wl.timestamps)


def test_fp32_workload_n256(hstu):
    wl = make_workload("c0")
    err = rel_err(_run(hstu, wl), _oracle(wl))
    print(f"c0 fp32 rel err {err:.3e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("name", ["c3_small", "c4_small"])
def test_bf16_reduced_workloads(hstu, name):
    wl = make_workload(name)
    err = rel_err(_run(hstu, wl), _oracle(wl))
    print(f"{name} bf16 rel err {err:.3e}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_dims_and_options(hstu, d, dtype):
    wl = _attn_recipe("dims", 100 + d, [300, 5, 129], 2, d, dtype=dtype, Bp=40, Bt=20)
    wl.alpha, wl.divisor = 0.75, 0.0
    err = rel_err(_run(hstu, wl), _oracle(wl))
    assert err <= (TOL_BF16 if dtype == "bf16" else TOL_F32), err
    wl.divisor = 77.0
    err = rel_err(_run(hstu, wl), _oracle(wl))
    assert err <= (TOL_BF16 if dtype == "bf16" else TOL_F32), err


def test_no_bias_and_large_position_table(hstu):
    wl = _attn_recipe("nobias", 7, [700, 260], 2, 128, time=False, pos=False)
    assert rel_err(_run(hstu, wl), _oracle(wl)) <= TOL_BF16
    # more than 1024 position buckets: entries past the LDS-staged part come from HBM
    wl = _attn_recipe("bigpos", 8, [1500], 1, 64, time=True, Bp=2000, Bt=200, table_std=0.5)
    assert rel_err(_run(hstu, wl), _oracle(wl)) <= TOL_BF16


def test_empty_and_single_token_sequences(hstu):
    wl = _attn_recipe("edge", 9, [0, 1, 0, 0, 2, 0], 3, 64)
    assert rel_err(_run(hstu, wl), _oracle(wl)) <= TOL_BF16
    wl = _attn_recipe("allempty", 9, [0, 0], 3, 64)
    out = _run(hstu, wl)
    assert out.shape == (0, 3, 64)


def test_large_and_mixed_score_ranges(hstu):
    """Scores far outside the polynomial SiLU range (exact path), and a batch
    where only some rows are large (per-row choice between the two forms)."""
    wl = _attn_recipe("large", 12, [400, 77], 2, 128, qkv_std=1.0, table_std=1.0)
    assert rel_err(_run(hstu, wl), _oracle(wl)) <= TOL_BF16
    wl = _attn_recipe("mixed", 13, [640], 2, 128)
    wl.q = wl.q.copy()
    wl.q[::7] *= 4.0                         # every 7th row has a 4x larger norm
    assert rel_err(_run(hstu, wl), _oracle(wl)) <= TOL_BF16


@pytest.mark.parametrize("d", [32, 64, 128])
def test_short_and_long_work_lists(hstu, d):
    """The same long, ragged sequences as a short work list (under 512 items:
    the kernel whose workgroups split each item's key range between two wave
    groups and add the halves' fp32 sums through LDS) and, padded with 600
    empty sequences, as a long one (one wave group per item). Both match the
    oracle and differ from each other by the order of one fp32 addition only.
    The 4100-token sequence walks key tiles past the 32-tile window of the
    per-block bias classification, in both halves."""
    import dataclasses
    lengths = [1500, 700, 513, 512, 90, 4100, 641]
    wl = _attn_recipe("pad", 300 + d, lengths, 2, d)
    ref = _oracle(wl)
    short = _run(hstu, wl)
    off = np.asarray(wl.seq_offsets)
    padded = dataclasses.replace(wl, seq_offsets=np.concatenate([off, np.full(600, off[-1], off.dtype)]))
    long_ = _run(hstu, padded)
    assert rel_err(short, ref) <= TOL_BF16
    assert rel_err(long_, ref) <= TOL_BF16
    assert rel_err(short, long_) <= 2.0 ** -6   # two bf16 ulps of the largest output


def test_split_kernel_edge_items(hstu):
    """Short work list (key-range-split kernel) with items whose second half
    has no tile (sequences of at most 64 tokens), a spare step (a last query
    tile of 65..128 rows), exactly one tile each, and an empty sequence."""
    wl = _attn_recipe("splitedge", 41, [64, 1, 65, 128, 129, 193, 0, 257, 320], 3, 64)
    assert rel_err(_run(hstu, wl), _oracle(wl)) <= TOL_BF16


def test_many_short_sequences(hstu):
    """5000 sequences of 0..9 tokens: more sequences than the work-list
    builder keeps in LDS, so its counters and scans go through global memory;
    a long list (one wave group per item)."""
    lengths = np.random.default_rng(77).integers(0, 10, size=5000).tolist()
    wl = _attn_recipe("many", 78, lengths, 2, 32)
    assert rel_err(_run(hstu, wl), _oracle(wl)) <= TOL_BF16


@pytest.mark.parametrize("seed", range(8))
def test_random_batches(hstu, seed):
    """Seeded random batches: 1-12 sequences of 0-1500 tokens, 1-4 heads, head
    dims 32/64/128, position and time biases on or off with random bucket
    counts (beyond the 1024 position buckets staged in LDS for one seed in
    four), score scale alpha and divisor. Odd seeds append 600 empty sequences,
    so the long-list kernel runs; even seeds take the short-list kernel."""
    import dataclasses
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 13))
    lengths = np.floor(np.exp(rng.uniform(0.0, np.log(1501.0), size=B))).astype(int) - 1
    H = int(rng.choice([1, 2, 4]))
    d = int(rng.choice([32, 64, 128]))
    pos, time = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    Bp = int(rng.choice([16, 128, 1500])) if seed % 4 == 3 else int(rng.choice([16, 128]))
    Bt = int(rng.choice([8, 32, 64]))
    wl = _attn_recipe(f"rand{seed}", 2000 + seed, lengths.tolist(), H, d, pos=pos, time=time, Bp=Bp, Bt=Bt,
                      table_std=float(rng.choice([0.02, 0.5])))
    wl.alpha = float(rng.choice([1.0, 0.5]))
    wl.divisor = float(rng.choice([0.0, 300.0]))
    if seed % 2 == 1:
        off = np.asarray(wl.seq_offsets)
        wl = dataclasses.replace(wl, seq_offsets=np.concatenate([off, np.full(600, off[-1], off.dtype)]))
    err = rel_err(_run(hstu, wl), _oracle(wl))
    print(f"seed {seed}: B {B} H {H} d {d} pos {pos} time {time} Bp {Bp} Bt {Bt} err {err:.2e}")
    assert err <= TOL_BF16


def test_nan_in_neighbour_sequence_does_not_leak(hstu):
    import torch
    wl = _attn_recipe("nan", 10, [200, 150, 90], 2, 128)
    d = attn_inputs_on_device(wl)
    for name in ("q", "k", "v"):
        d[name][200:350] = float("nan")
    o = hstu.attn_fwd(d["q"], d["k"], d["v"], d["seq_offsets"], timestamps=d["timestamps"],
                      pos_table=d["pos_table"], time_table=d["time_table"])
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    ref = _oracle(wl)
    keep = np.r_[0:200, 350:440]
    assert np.all(np.isfinite(o[keep]))
    assert rel_err(o[keep], ref[keep]) <= TOL_BF16


def test_causality_bitwise_and_determinism(hstu):
    import torch
    wl = _attn_recipe("causal", 11, [500], 2, 128)
    d = attn_inputs_on_device(wl)
    args = dict(timestamps=d["timestamps"], pos_table=d["pos_table"], time_table=d["time_table"])
    base = hstu.attn_fwd(d["q"], d["k"], d["v"], d["seq_offsets"], **args).clone()
    again = hstu.attn_fwd(d["q"], d["k"], d["v"], d["seq_offsets"], **args)
    torch.cuda.synchronize()
    assert torch.equal(base, again)
    g = torch.Generator(device="cpu").manual_seed(5)
    for cut in (0, 63, 200, 383):
        q, k, v = d["q"].clone(), d["k"].clone(), d["v"].clone()
        ts = d["timestamps"].clone()
        sl = slice(cut + 1, 500)
        for t in (q, k, v):
            t[sl] += (torch.randn(t[sl].shape, generator=g) * 3).to(t.device, t.dtype)
        ts[sl] += torch.randint(0, 10**6, ts[sl].shape, generator=g).to(ts.device)
        o = hstu.attn_fwd(q, k, v, d["seq_offsets"], timestamps=ts, pos_table=d["pos_table"],
                          time_table=d["time_table"])
        torch.cuda.synchronize()
        assert torch.equal(o[:cut + 1], base[:cut + 1]), cut


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_full_size_every_element(hstu, name):
    """Full-size workloads in the launch configuration the benchmark times
    (4 x 8192 tokens with 8 heads; 32 jagged sequences with 4 heads): every
    output element against the whole oracle."""
    wl = make_workload(name)
    o = _run(hstu, wl)
    assert np.all(np.isfinite(o))
    err = rel_err(o, _oracle(wl))
    print(f"{name} every element: rel err {err:.3e}")
    assert err <= TOL_BF16


def _clamped(off, T):
    """The documented reading of a malformed offsets array (include/hstu.h):
    c(b) = min(max(0, off[0..b]), T)."""
    return np.minimum(np.maximum.accumulate(np.maximum(np.asarray(off, np.int64), 0)), T)


@pytest.mark.parametrize("raw", [
    [0, 300, 200, 700, 100],        # a decreasing step and an offset past T
    [-40, 120, 90, 500],            # a negative offset
    [0, 100, 60],                   # offsets ending before T: later tokens belong to no sequence
])
def test_malformed_offsets_are_clamped(hstu, raw):
    """The kernels read a clamped copy of the offsets, so a malformed array
    neither faults nor moves a read out of the T tokens: the result equals
    the oracle on the clamped offsets, for every token that the clamped batch
    covers."""
    import dataclasses
    T = 500
    wl = _attn_recipe("malformed", 51, [T], 2, 64)
    c = _clamped(raw, T)
    lo, hi = int(c[0]), int(c[-1])
    got = _run(hstu, dataclasses.replace(wl, seq_offsets=np.asarray(raw, np.int64)))
    part = dataclasses.replace(wl, q=wl.q[lo:hi], k=wl.k[lo:hi], v=wl.v[lo:hi], timestamps=wl.timestamps[lo:hi],
                               seq_offsets=c - lo)
    ref = _oracle(part)
    err = rel_err(got[lo:hi], ref)
    print(f"offsets {raw} -> {c.tolist()}: err {err:.2e}")
    assert err <= TOL_BF16
