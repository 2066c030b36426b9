"""The bucket-edge inputs (tests/bucket_edge_inputs.py) are sensitive enough:
on the CPU, planting a plausible slip of the bucket functions in the oracle
moves its outputs -- the forward, each backward variant and the candidate
scores that the GPU edge tests compare -- by more than twice the bf16
tolerance. A kernel with such a slip therefore fails those GPU tests.

Slips planted: floor(log2(dt)) or floor(log2(2 + dt)) for the time bucket
instead of floor(log2(1 + dt)); |dt| instead of max(dt, 0) for negative
gaps; the time clamp at Bt - 2; the position bucket one off in either
direction."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests import bucket_edge_inputs as E
from tests.helpers import TOL_BF16, rel_err
from workloads.generators import offsets_from_lengths

_TRUE_TB, _TRUE_PB = orc.time_bucket, orc.pos_bucket

TIME_SLIPS = {
    "log2(dt)": lambda dt, nb: _TRUE_TB(np.asarray(dt) - 1, nb),
    "log2(2+dt)": lambda dt, nb: _TRUE_TB(np.asarray(dt) + 1, nb),
    "abs(dt)": lambda dt, nb: _TRUE_TB(np.abs(np.asarray(dt)), nb),
    "clamp Bt-2": lambda dt, nb: np.minimum(_TRUE_TB(dt, nb), nb - 2),
}
POS_SLIPS = {
    "pos-1": lambda d, nb: _TRUE_PB(np.asarray(d) - 1, nb),
    "pos+1": lambda d, nb: _TRUE_PB(np.asarray(d) + 1, nb),
}


def fwd_inputs(Bp, Bt, scale):
    lengths, ts = E.edge_batch()
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    pt, tt = E.tables(Bp, Bt, scale)
    z = np.zeros((T, E.H, E.D), np.float32)
    return dict(q=z, k=z, v=E.one_hot(lengths), seq_offsets=off, timestamps=ts, pos_table=pt, time_table=tt)


def bwd_inputs(variant, Bp, Bt, scale, seed=3):
    """A: q = 0, k = v = I, dO = +-1 (dq is dS pair by pair, query pass);
    B: q = v = I, k = 0, dO = +-1 (dk is dS transposed, key pass);
    C: q = k = 0, v = I, dO_i = e_j(i) for one partner j(i) <= i per row, the
    partner whose gap to i is an edge where there is one (table gradients)."""
    lengths, ts = E.edge_batch()
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    pt, tt = E.tables(Bp, Bt, scale)
    rng = np.random.default_rng(seed)
    I = E.one_hot(lengths)
    z = np.zeros_like(I)
    if variant == "C":
        def partner(b, i):
            t = ts[off[b]:off[b + 1]]
            dt = t[i] - t[:i + 1] + 1
            edge = np.flatnonzero((dt > 1) & ((dt & (dt - 1)) == 0))         # 1 + dt a power of two
            return int(edge[rng.integers(0, edge.size)]) if edge.size else int(rng.integers(0, i + 1))
        d_o = np.zeros_like(I)
        for b in range(len(lengths)):
            for i in range(int(lengths[b])):
                d_o[off[b] + i, :, partner(b, i)] = 1.0
        q, k = z, z
    else:
        d_o = rng.choice(np.array([-1.0, 1.0], np.float32), size=I.shape).astype(np.float32)
        q, k = (z, I) if variant == "A" else (I, z)
    return dict(q=q, k=k, v=I, d_o=d_o, seq_offsets=off, timestamps=ts, pos_table=pt, time_table=tt)


def cand_inputs(Bp, Bt, scale):
    hl, hts, cm, cts = E.cand_edge_batch()
    hoff, coff = offsets_from_lengths(hl), offsets_from_lengths(cm)
    Th, Tc = int(hoff[-1]), int(coff[-1])
    pt, tt = E.tables(Bp, Bt, scale)
    zc = np.zeros((Tc, E.H, E.D), np.float32)
    vc = zc.copy()
    vc[:, :, E.D - 1] = 1.0
    return dict(q_c=zc, k_c=zc, v_c=vc, cand_offsets=coff, k_hist=np.zeros((Th, E.H, E.D), np.float32),
                v_hist=E.one_hot(hl), q_hist=np.zeros((Th, E.H, E.D), np.float32), seq_offsets=hoff,
                timestamps=hts, cand_timestamps=cts, pos_table=pt, time_table=tt)


def oracle_fwd(a):
    return orc.attn_fwd(a["q"], a["k"], a["v"], a["seq_offsets"], pos_table=a["pos_table"],
                        time_table=a["time_table"], timestamps=a["timestamps"], divisor=E.DIVISOR)


def oracle_bwd(a):
    return orc.attn_bwd(a["q"], a["k"], a["v"], a["d_o"], a["seq_offsets"], pos_table=a["pos_table"],
                        time_table=a["time_table"], timestamps=a["timestamps"], divisor=E.DIVISOR)


def oracle_cand(a):
    return orc.attn_fwd_candidates(a["q_c"], a["k_c"], a["v_c"], a["cand_offsets"], a["k_hist"], a["v_hist"],
                                   a["q_hist"], a["seq_offsets"], pos_table=a["pos_table"],
                                   time_table=a["time_table"], timestamps=a["timestamps"],
                                   cand_timestamps=a["cand_timestamps"], divisor=E.DIVISOR)


def test_edges_present():
    """Pairs sit exactly on the edges 2^k - 1 / 2^k - 2 for k across the
    narrow and the wide range, and some gaps are negative."""
    lengths, ts = E.edge_batch()
    off = offsets_from_lengths(lengths)
    ks_hit, neg = set(), False
    for b in range(len(lengths)):
        t = ts[off[b]:off[b + 1]]
        g = (t[:, None] - t[None, :])[np.tril_indices(t.size)]
        neg |= bool(np.any(g < 0))
        for k in range(1, 41):
            if np.any(g == (1 << k) - 1) and np.any(g == (1 << k) - 2):
                ks_hit.add(k)
    assert neg
    assert {2, 5, 10, 11, 20, 30, 31, 33, 34}.issubset(ks_hit), sorted(ks_hit)


@pytest.mark.parametrize("Bp,Bt,scale", E.CONFIGS)
def test_slips_move_the_forward(monkeypatch, Bp, Bt, scale):
    a = fwd_inputs(Bp, Bt, scale)
    ref = oracle_fwd(a)
    for name, slip in list(TIME_SLIPS.items()) + list(POS_SLIPS.items()):
        if name == "clamp Bt-2" and Bt > 40:
            continue            # gaps here reach bucket 41 at most: the clamp is not reached
        with monkeypatch.context() as m:
            m.setattr(orc, "time_bucket" if name in TIME_SLIPS else "pos_bucket", slip)
            err = rel_err(oracle_fwd(a), ref)
        assert err > 2 * TOL_BF16, (name, err)


@pytest.mark.parametrize("variant,grad", [("A", 0), ("B", 1), ("C", 3), ("C", 4)])
@pytest.mark.parametrize("cfg", [0, 1])
def test_slips_move_the_backward(monkeypatch, variant, grad, cfg):
    Bp, Bt, scale = E.CONFIGS[cfg]
    a = bwd_inputs(variant, Bp, Bt, scale)
    ref = oracle_bwd(a)[grad]
    slips = dict(TIME_SLIPS)
    if grad != 4:
        slips.update(POS_SLIPS)
    for name, slip in slips.items():
        if grad == 3 and name in ("abs(dt)", "clamp Bt-2"):
            continue            # time-only slips do not move the position-table gradient
        if name == "clamp Bt-2" and Bt > 40:
            continue
        with monkeypatch.context() as m:
            m.setattr(orc, "time_bucket" if name in TIME_SLIPS else "pos_bucket", slip)
            err = rel_err(oracle_bwd(a)[grad], ref)
        assert err > 2 * TOL_BF16, (variant, grad, name, err)


@pytest.mark.parametrize("cfg", [0, 1])
def test_slips_move_the_candidates(monkeypatch, cfg):
    Bp, Bt, scale = E.CONFIGS[cfg]
    a = cand_inputs(Bp, Bt, scale)
    ref = oracle_cand(a)
    for name, slip in list(TIME_SLIPS.items()) + list(POS_SLIPS.items()):
        if name == "clamp Bt-2" and Bt > 40:
            continue
        with monkeypatch.context() as m:
            m.setattr(orc, "time_bucket" if name in TIME_SLIPS else "pos_bucket", slip)
            err = rel_err(oracle_cand(a), ref)
        assert err > 2 * TOL_BF16, (name, err)
