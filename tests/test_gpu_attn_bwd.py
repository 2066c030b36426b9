"""GPU parity of hstu_attn_bwd (dQ, dK, dV and the bias-table gradients)
against the fp64 oracle's hand-derived gradients, through the C ABI. Each
gradient tensor is held to the bf16 tolerance separately."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import TOL_BF16, attn_inputs_on_device, rel_err, to_dev
from workloads import make_workload
from workloads.generators import exponential_timestamps, normal, offsets_from_lengths, round_to_bf16

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "d_pos", "d_time")


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _gpu_bwd(hstu, inp, alpha=1.0, divisor=0.0):
    import torch
    out = hstu.attn_bwd(inp["q"], inp["k"], inp["v"], inp["d_o"], inp["seq_offsets"],
                        timestamps=inp["timestamps"], pos_table=inp["pos_table"],
                        time_table=inp["time_table"], alpha=alpha, divisor=divisor)
    torch.cuda.synchronize()
    return [None if t is None else t.float().cpu().numpy() for t in out]


def _oracle_bwd(q, k, v, d_o, off, ts, pt, tt, alpha=1.0, divisor=0.0):
    return orc.attn_bwd(q, k, v, d_o, off, pos_table=pt, time_table=tt, timestamps=ts,
                        alpha=alpha, divisor=divisor)


def _compare(got, ref, label):
    errs = {}
    for name, g, r in zip(NAMES, got, ref):
        assert (g is None) == (r is None), f"{label}: {name} presence"
        if r is None:
            continue
        assert np.all(np.isfinite(g)), f"{label}: {name} not finite"
        errs[name] = rel_err(g, r)
    print(label, " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL_BF16, f"{label}: {name} error {e:.3e}"
    return errs


def _synthetic(lengths, H, d, *, seed, pos=True, time=True, Bp=128, Bt=128, table_std=0.02, qkv_std=None):
    """A seeded attention-backward input in the workload recipe's shape."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    std = 1.0 / np.sqrt(d) if qkv_std is None else qkv_std
    q, k, v = (round_to_bf16(normal(rng, (T, H, d), std)) for _ in range(3))
    d_o = round_to_bf16(normal(rng, (T, H, d), 1.0))
    ts = exponential_timestamps(rng, lengths) if time else None
    pt = normal(rng, (H, Bp), table_std) if pos else None
    tt = normal(rng, (H, Bt), table_std) if time else None
    return q, k, v, d_o, off, ts, pt, tt


def _dev(q, k, v, d_o, off, ts, pt, tt):
    import torch
    return dict(q=to_dev(q, torch.bfloat16), k=to_dev(k, torch.bfloat16), v=to_dev(v, torch.bfloat16),
                d_o=to_dev(d_o, torch.bfloat16), seq_offsets=to_dev(off),
                timestamps=None if ts is None else to_dev(ts),
                pos_table=None if pt is None else to_dev(pt, torch.float32),
                time_table=None if tt is None else to_dev(tt, torch.float32))


def test_reduced_jagged_all_gradients(hstu):
    wl = make_workload("c4_small")
    got = _gpu_bwd(hstu, attn_inputs_on_device(wl))
    ref = _oracle_bwd(wl.q, wl.k, wl.v, wl.d_o, wl.seq_offsets, wl.timestamps, wl.pos_table, wl.time_table)
    _compare(got, ref, "c4_small")


def test_full_size_jagged_all_gradients(hstu):
    """32 sequences, lengths log-uniform in [64, 2048], H 4, d 128: every
    element of every gradient against the oracle."""
    wl = make_workload("c4")
    got = _gpu_bwd(hstu, attn_inputs_on_device(wl))
    ref = _oracle_bwd(wl.q, wl.k, wl.v, wl.d_o, wl.seq_offsets, wl.timestamps, wl.pos_table, wl.time_table)
    _compare(got, ref, "c4")
    # every pair adds its dS to exactly one entry of each table
    assert np.allclose(got[3].sum(axis=1), got[4].sum(axis=1), rtol=1e-3, atol=1e-3 * np.abs(got[3]).max())


@pytest.mark.parametrize("d", [32, 64, 128])
def test_head_dims_scale_and_divisor(hstu, d):
    args = _synthetic([300, 65, 1, 190], 3, d, seed=100 + d)
    got = _gpu_bwd(hstu, _dev(*args), alpha=0.7, divisor=512.0)
    ref = _oracle_bwd(*args, alpha=0.7, divisor=512.0)
    _compare(got, ref, f"d={d} alpha 0.7 divisor 512")


@pytest.mark.parametrize("pos,time", [(False, False), (True, False), (False, True)])
def test_bias_subsets(hstu, pos, time):
    args = _synthetic([333, 97, 260], 2, 128, seed=7, pos=pos, time=time)
    got = _gpu_bwd(hstu, _dev(*args))
    ref = _oracle_bwd(*args)
    _compare(got, ref, f"pos={pos} time={time}")


def test_empty_and_single_token_sequences(hstu):
    args = _synthetic([0, 1, 129, 0, 2, 128, 1], 2, 64, seed=9)
    got = _gpu_bwd(hstu, _dev(*args))
    ref = _oracle_bwd(*args)
    _compare(got, ref, "empty/single")


def test_large_position_table_and_wide_gaps(hstu):
    """1024 position buckets (every pair of a long sequence in its own bucket
    near the diagonal) and timestamps with gaps spanning many time buckets."""
    q, k, v, d_o, off, ts, pt, tt = _synthetic([1100, 400], 2, 128, seed=11, Bp=1024, table_std=0.3)
    rng = np.random.default_rng(5)
    ts = np.concatenate([np.cumsum(rng.integers(0, 1 << 20, n)) for n in (1100, 400)]).astype(np.int64)
    args = (q, k, v, d_o, off, ts, pt, tt)
    got = _gpu_bwd(hstu, _dev(*args))
    ref = _oracle_bwd(*args)
    _compare(got, ref, "Bp=1024, wide gaps")


def test_long_sequence(hstu):
    """A 4160-token sequence: a key tile walks 130 query blocks, so the key
    pass refills its table of block classes (64 blocks at a time) twice, and
    the time gaps grow past 2^22 seconds (buckets up to 22)."""
    args = _synthetic([4160, 65], 1, 128, seed=17)
    got = _gpu_bwd(hstu, _dev(*args))
    ref = _oracle_bwd(*args)
    _compare(got, ref, "n=4160")


def test_large_scores(hstu):
    """Scores of a few tens (q, k ~ N(0, 1)): SiLU' saturates on both sides."""
    args = _synthetic([300, 200], 2, 64, seed=13, qkv_std=1.0)
    got = _gpu_bwd(hstu, _dev(*args))
    ref = _oracle_bwd(*args)
    _compare(got, ref, "large scores")


def test_deterministic(hstu):
    wl = make_workload("c4_small")
    inp = attn_inputs_on_device(wl)
    a = _gpu_bwd(hstu, inp)
    b = _gpu_bwd(hstu, inp)
    for name, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), name


def test_query_gradient_ignores_later_tokens(hstu):
    """dQ_i reads only keys and values j <= i: changing k and v of tokens 300
    and later leaves dQ of the first 300 rows bitwise unchanged (masked pairs
    enter the products as exact zeros)."""
    import torch
    q, k, v, d_o, off, ts, pt, tt = _synthetic([400], 2, 128, seed=17)
    inp = _dev(q, k, v, d_o, off, ts, pt, tt)
    a = _gpu_bwd(hstu, inp)
    k2, v2 = k.copy(), v.copy()
    k2[300:] += 0.5
    v2[300:] -= 0.25
    inp2 = dict(inp, k=to_dev(round_to_bf16(k2), torch.bfloat16), v=to_dev(round_to_bf16(v2), torch.bfloat16))
    b = _gpu_bwd(hstu, inp2)
    assert np.array_equal(a[0][:300], b[0][:300])


def test_malformed_offsets_are_clamped(hstu):
    """Offsets [0, 250, 120, 900] over 300 tokens read as their clamped copy
    [0, 250, 250, 300] (include/hstu.h): every gradient equals the oracle's on
    the clamped batch."""
    q, k, v, d_o, _, ts, pt, tt = _synthetic([300], 2, 128, seed=23)
    raw = np.array([0, 250, 120, 900], np.int64)
    clamped = np.array([0, 250, 250, 300], np.int64)
    got = _gpu_bwd(hstu, _dev(q, k, v, d_o, raw, ts, pt, tt))
    ref = _oracle_bwd(q, k, v, d_o, clamped, ts, pt, tt)
    _compare(got, ref, "malformed offsets")
