"""GPU parity of hstu_attn_fwd_candidates (candidate scoring against a
history with cached keys and values) against the fp64 oracle, through the C
ABI."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import TOL_BF16, rel_err, to_dev
from workloads import make_workload
from workloads.generators import offsets_from_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _gpu(hstu, wl, c=None, pos=True, time=True, alpha=1.0, divisor=0.0):
    import torch
    c = wl.cand if c is None else c
    bf = torch.bfloat16
    out = hstu.attn_fwd_candidates(
        to_dev(c["q"], bf), to_dev(c["k"], bf), to_dev(c["v"], bf), to_dev(c["offsets"]),
        to_dev(wl.k, bf), to_dev(wl.v, bf), to_dev(wl.seq_offsets),
        timestamps=to_dev(wl.timestamps) if time else None,
        cand_timestamps=to_dev(c["timestamps"]) if time else None,
        pos_table=to_dev(wl.pos_table, torch.float32) if pos else None,
        time_table=to_dev(wl.time_table, torch.float32) if time else None, alpha=alpha, divisor=divisor)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _ref(wl, c=None, pos=True, time=True, alpha=1.0, divisor=0.0):
    c = wl.cand if c is None else c
    return orc.attn_fwd_candidates(c["q"], c["k"], c["v"], c["offsets"], wl.k, wl.v, wl.q, wl.seq_offsets,
                                   alpha=alpha, divisor=divisor, pos_table=wl.pos_table if pos else None,
                                   time_table=wl.time_table if time else None,
                                   timestamps=wl.timestamps if time else None,
                                   cand_timestamps=c["timestamps"] if time else None)


def test_reduced_ragged_histories_all_candidates(hstu):
    """Histories of 300, 0, 77, 1 and 140 tokens with 5, 3, 0, 130 and 64
    candidates (two candidate tiles in one sequence), both biases."""
    wl = make_workload("c6_small")
    err = rel_err(_gpu(hstu, wl), _ref(wl))
    print(f"c6_small err {err:.2e}")
    assert err <= TOL_BF16


def test_histories_across_the_chunk_size(hstu):
    """Histories of 2047, 2048, 2049, 4100, 0 and 6000 tokens (one to three
    history chunks of 2048 keys, partial outputs summed across chunks) with
    3, 1, 130, 2, 5 and 64 candidates, both biases; every candidate."""
    from workloads.generators import _cand_recipe
    wl = _cand_recipe("chunks", 19, lengths=[2047, 2048, 2049, 4100, 0, 6000], cands=[3, 1, 130, 2, 5, 64],
                      H=2, d=128)
    err = rel_err(_gpu(hstu, wl), _ref(wl))
    print(f"chunked histories err {err:.2e}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("pos,time", [(False, False), (True, False), (False, True)])
def test_bias_subsets_scale_and_divisor(hstu, pos, time):
    wl = make_workload("c6_small")
    err = rel_err(_gpu(hstu, wl, pos=pos, time=time, alpha=0.7, divisor=200.0),
                  _ref(wl, pos=pos, time=time, alpha=0.7, divisor=200.0))
    print(f"pos={pos} time={time} err {err:.2e}")
    assert err <= TOL_BF16


def test_full_size_sampled_candidates(hstu):
    """16 histories log-uniform in [1024, 8192] with 1024 candidates each: the
    GPU scores all 16384; 32 candidates of every sequence (both ends of each
    128-candidate workgroup tile, the rest drawn with a fixed seed) are
    checked against the oracle, which scores each candidate on its own (the
    full oracle takes minutes)."""
    wl = make_workload("c6")
    got = _gpu(hstu, wl)
    c = wl.cand
    coff = c["offsets"]
    rng = np.random.default_rng(61)
    pick = []
    per = []
    for b in range(coff.size - 1):
        lo, hi = int(coff[b]), int(coff[b + 1])
        chosen = {lo, hi - 1}
        for t0 in range(lo, hi, 128):
            chosen |= {t0, min(t0 + 127, hi - 1)}
        chosen = sorted(chosen)[:18]
        rest = np.setdiff1d(np.arange(lo, hi), chosen)
        chosen = sorted(set(chosen) | set(rng.choice(rest, size=32 - len(chosen), replace=False).tolist()))
        pick += chosen
        per.append(len(chosen))
    pick = np.array(pick)
    per = np.array(per)
    sub = dict(offsets=offsets_from_lengths(per), q=c["q"][pick], k=c["k"][pick], v=c["v"][pick],
               timestamps=c["timestamps"][pick])
    ref = _ref(wl, c=sub)
    err = rel_err(got[pick], ref)
    print(f"c6 sampled err {err:.2e} over {pick.size} candidates")
    assert err <= TOL_BF16


def test_candidates_do_not_see_each_other_bitwise(hstu):
    """Changing candidate 2's q, k, v leaves every other candidate's output
    bitwise unchanged (its self term is masked out for the others)."""
    wl = make_workload("c6_small")
    base = _gpu(hstu, wl)
    c = dict(wl.cand)
    for key in ("q", "k", "v"):
        c[key] = c[key].copy()
        c[key][2] = -c[key][2] + 0.5
    other = _gpu(hstu, wl, c=c)
    keep = [i for i in range(base.shape[0]) if i != 2]
    assert np.array_equal(base[keep], other[keep])
    assert not np.array_equal(base[2], other[2])


def test_single_candidate_equals_forward_last_row(hstu):
    """One candidate after a history equals the forward's last row on
    (history ++ candidate), both computed on the GPU."""
    import torch
    wl = make_workload("c6_small")
    b = 0
    h0, h1 = int(wl.seq_offsets[b]), int(wl.seq_offsets[b + 1])
    c = wl.cand
    j = int(c["offsets"][b])
    cat = lambda hist, cand: np.concatenate([hist[h0:h1], cand[j:j + 1]])
    q = cat(wl.q, c["q"])   # the history's q rows do not enter the last row
    ts = np.concatenate([wl.timestamps[h0:h1], c["timestamps"][j:j + 1]])
    bf = torch.bfloat16
    o = hstu.attn_fwd(to_dev(q, bf), to_dev(cat(wl.k, c["k"]), bf), to_dev(cat(wl.v, c["v"]), bf),
                      to_dev(np.array([0, h1 - h0 + 1], np.int64)), timestamps=to_dev(ts),
                      pos_table=to_dev(wl.pos_table, torch.float32),
                      time_table=to_dev(wl.time_table, torch.float32))
    torch.cuda.synchronize()
    fwd_last = o.float().cpu().numpy()[-1]
    sub = dict(offsets=np.array([0, 1], np.int64), q=c["q"][j:j + 1], k=c["k"][j:j + 1], v=c["v"][j:j + 1],
               timestamps=c["timestamps"][j:j + 1])
    wl1 = make_workload("c6_small")
    wl1.seq_offsets = np.array([0, h1 - h0], np.int64)
    wl1.k, wl1.v, wl1.q, wl1.timestamps = wl.k[h0:h1], wl.v[h0:h1], wl.q[h0:h1], wl.timestamps[h0:h1]
    cand = _gpu(hstu, wl1, c=sub)[0]
    assert rel_err(cand, fwd_last) <= TOL_BF16


def test_deterministic(hstu):
    wl = make_workload("c6_small")
    assert np.array_equal(_gpu(hstu, wl), _gpu(hstu, wl))


def test_malformed_offsets_are_clamped(hstu):
    """History offsets [0, 150, 60, 10**9] over 300 tokens and candidate
    offsets [0, 3, 1, 12] over 10 candidates read as their clamped copies
    [0, 150, 150, 300] and [0, 3, 3, 10] (include/hstu.h): every candidate
    equals the oracle's score on the clamped batch."""
    import dataclasses
    from workloads.generators import _cand_recipe
    wl = _cand_recipe("malformed", 29, lengths=[150, 0, 150], cands=[3, 0, 7], H=2, d=64)
    ref = _ref(wl)
    c = dict(wl.cand, offsets=np.array([0, 3, 1, 12], np.int64))
    got = _gpu(hstu, dataclasses.replace(wl, seq_offsets=np.array([0, 150, 60, 10 ** 9], np.int64)), c=c)
    err = rel_err(got, ref)
    print(f"malformed offsets err {err:.2e}")
    assert err <= TOL_BF16
