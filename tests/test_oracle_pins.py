"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with a copy of itself: each check uses an
independent form (pure-Python loops, a dense transcription of the pages'
exported expression, a closed form, a textbook routine, an invariant or a
hand-worked example). Each is chosen so that a plausible mistake in the
oracle (a dropped bias term, a wrong sign or index, a mask before instead of
after the SiLU, a transposed operand, a wrong divisor) fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from oracle import brute as B
from workloads import make_workload
from workloads.generators import exponential_timestamps, offsets_from_lengths


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _tiny_case(seed, lengths, H=2, d=3, dv=4, Bp=5, Bt=6, time=True, pos=True):
    rng = np.random.default_rng(seed)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, dv))
    do = rng.standard_normal((T, H, dv))
    ts = rng.integers(0, 40, size=T).astype(np.int64) + 10**9 if time else None
    pt = rng.standard_normal((H, Bp)) * 0.5 if pos else None
    tt = rng.standard_normal((H, Bt)) * 0.5 if time else None
    return dict(q=q, k=k, v=v, do=do, off=off, ts=ts, pt=pt, tt=tt)


# ----------------------------------------------------------------------------
# bucket functions
# ----------------------------------------------------------------------------
def test_time_bucket_golden_edges(golden_dir):
    with open(os.path.join(golden_dir, "time_bucket_edges.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got_o = int(O.time_bucket(np.array([c["dt"]], np.int64), c["Bt"])[0])
        got_b = B.time_bucket(c["dt"], c["Bt"])
        assert got_o == c["bucket"], c
        assert got_b == c["bucket"], c


def test_time_bucket_matches_log2_on_range():
    dt = np.arange(-50, 300000, dtype=np.int64)
    ref = np.array([0 if x <= 0 else int(math.floor(math.log2(1 + x))) for x in dt.tolist()])
    assert np.array_equal(O.time_bucket(dt, 128), ref)
    assert np.array_equal(O.time_bucket(dt, 9), np.minimum(ref, 8))


def test_pos_bucket_clamps():
    d = np.arange(0, 300, dtype=np.int64)
    assert np.array_equal(O.pos_bucket(d, 64), np.minimum(d, 63))
    assert all(B.pos_bucket(int(x), 64) == min(int(x), 63) for x in d)


# ----------------------------------------------------------------------------
# forward: brute force, the pages' dense expression, hand-worked example
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("alpha,divisor", [(1.0, 0.0), (0.7, 0.0), (1.3, 5.0)])
def test_fwd_matches_brute_force_loops(alpha, divisor):
    c = _tiny_case(0, [5, 0, 1, 8, 3])
    ref = B.attn_fwd(c["q"], c["k"], c["v"], c["off"], alpha, divisor, c["pt"], c["tt"], c["ts"])
    got = O.attn_fwd(c["q"], c["k"], c["v"], c["off"], alpha=alpha, divisor=divisor,
                     pos_table=c["pt"], time_table=c["tt"], timestamps=c["ts"], row_block=3)
    assert _rel(got, ref) < 1e-12


def test_fwd_matches_dense_transcription_of_exported_block():
    """One sequence, no bias, alpha 1, divisor n: the exported block computes
    (silu(q @ k^T) / t).tril() @ v per head; write it densely and compare."""
    rng = np.random.default_rng(1)
    n, H, d = 37, 3, 8
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    ref = np.zeros((n, H, d))
    for h in range(H):
        s = q[:, h] @ k[:, h].T
        a = np.tril(s / (1.0 + np.exp(-s)) / n)
        ref[:, h] = a @ v[:, h]
    got = O.attn_fwd(q, k, v, np.array([0, n]), row_block=10)
    assert _rel(got, ref) < 1e-13


def test_fwd_hand_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "worked_example_n2.json")) as f:
        g = json.load(f)
    q = np.array(g["q"]).reshape(2, 1, 1)
    k = np.array(g["k"]).reshape(2, 1, 1)
    v = np.array(g["v"]).reshape(2, 1, 1)
    pt = np.array(g["pos_table"]).reshape(1, 2)
    got = O.attn_fwd(q, k, v, np.array([0, 2]), pos_table=pt)

    def silu(x):
        return x / (1.0 + math.exp(-x))

    for i, key in enumerate(["O0", "O1"]):
        exp = sum(silu(x) * c * vv for x, c, vv in g["expected_terms"][key])
        assert abs(got[i, 0, 0] - exp) < 1e-15 * max(1.0, abs(exp))


def test_fwd_rows_match_full():
    c = _tiny_case(2, [40, 77], H=2, d=5, dv=3, Bp=16, Bt=10)
    full = O.attn_fwd(c["q"], c["k"], c["v"], c["off"], pos_table=c["pt"],
                      time_table=c["tt"], timestamps=c["ts"])
    rows = [0, 1, 39, 76, 50]
    got = O.attn_fwd_rows(c["q"], c["k"], c["v"], c["off"], 1, 1, rows, pos_table=c["pt"],
                          time_table=c["tt"], timestamps=c["ts"])
    assert _rel(got, full[40 + np.array(rows), 1]) < 1e-13


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_zero_qk_zero_bias_gives_exact_zero():
    rng = np.random.default_rng(3)
    T, H = 50, 2
    q = np.zeros((T, H, 4))
    v = rng.standard_normal((T, H, 6))
    ts = np.sort(rng.integers(0, 10**6, size=T))
    out = O.attn_fwd(q, q, v, np.array([0, 20, 50]), pos_table=np.zeros((H, 8)),
                     time_table=np.zeros((H, 8)), timestamps=ts)
    assert np.all(out == 0.0)


def test_constant_bias_gives_prefix_sum():
    """q = k = 0, P == c: O_i = SiLU(c)/n * sum_{j<=i} v_j (cumulative sum)."""
    rng = np.random.default_rng(4)
    n, H, c = 33, 2, 0.37
    v = rng.standard_normal((n, H, 5))
    q = np.zeros((n, H, 3))
    got = O.attn_fwd(q, q, v, np.array([0, n]), pos_table=np.full((H, 7), c), row_block=8)
    silu_c = c / (1.0 + math.exp(-c))
    ref = silu_c / n * np.cumsum(v, axis=0)
    assert _rel(got, ref) < 1e-13


def test_position_bias_is_causal_convolution():
    """q = k = 0, no time bias: O = causal convolution of v with
    w_m = SiLU(P[h, min(m, Bp-1)]) / n (numpy.convolve, truncated)."""
    rng = np.random.default_rng(5)
    n, H, Bp = 60, 2, 9
    v = rng.standard_normal((n, H, 4))
    pt = rng.standard_normal((H, Bp))
    q = np.zeros((n, H, 2))
    got = O.attn_fwd(q, q, v, np.array([0, n]), pos_table=pt, row_block=16)
    for h in range(H):
        m = np.arange(n)
        p = pt[h][np.minimum(m, Bp - 1)]
        w = p / (1.0 + np.exp(-p)) / n
        for e in range(4):
            ref = np.convolve(w, v[:, h, e])[:n]
            assert _rel(got[:, h, e], ref) < 1e-13


def test_identical_timestamps_reduce_to_position_only():
    """All timestamps equal: every time bucket is 0, so the time bias is the
    constant Tt[h, 0], which equals folding it into every position bucket."""
    c = _tiny_case(6, [30, 12], Bp=8, Bt=5)
    ts = np.full(42, 1_700_000_000, np.int64)
    got = O.attn_fwd(c["q"], c["k"], c["v"], c["off"], pos_table=c["pt"],
                     time_table=c["tt"], timestamps=ts)
    ref = O.attn_fwd(c["q"], c["k"], c["v"], c["off"], pos_table=c["pt"] + c["tt"][:, :1])
    assert _rel(got, ref) < 1e-13


def test_time_gaps_on_bucket_edges():
    """Timestamps spaced so every gap of each pair sits exactly on a bucket
    edge (2**k - 1); a bucket off by one shows as a different table entry."""
    H, n = 1, 6
    ts = np.array([0, 1, 4, 11, 26, 57], np.int64)   # gaps to the previous: 1, 3, 7, 15, 31
    tt = np.arange(10, dtype=np.float64)[None, :] * 0.1
    q = np.zeros((n, H, 1))
    v = np.eye(n).reshape(n, H, n)
    got = O.attn_fwd(q, q, v, np.array([0, n]), time_table=tt, timestamps=ts, divisor=1.0)
    for i in range(n):
        for j in range(n):
            if j > i:
                assert got[i, 0, j] == 0.0
                continue
            bkt = int(math.floor(math.log2(1 + ts[i] - ts[j])))
            x = tt[0, bkt]
            assert abs(got[i, 0, j] - x / (1 + math.exp(-x))) < 1e-15


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_causality_bitwise():
    c = _tiny_case(7, [25, 31], Bp=12, Bt=12)
    base = O.attn_fwd(c["q"], c["k"], c["v"], c["off"], pos_table=c["pt"],
                      time_table=c["tt"], timestamps=c["ts"])
    rng = np.random.default_rng(70)
    for cut in [0, 7, 24, 25 + 13]:
        q, k, v, ts = (c[x].copy() for x in ("q", "k", "v", "ts"))
        seq_end = 25 if cut < 25 else 56
        sl = slice(cut + 1, seq_end)
        q[sl] += rng.standard_normal(q[sl].shape) * 10
        k[sl] += rng.standard_normal(k[sl].shape) * 10
        v[sl] += rng.standard_normal(v[sl].shape) * 10
        ts[sl] += rng.integers(0, 10**7, size=ts[sl].shape)
        pert = O.attn_fwd(q, k, v, c["off"], pos_table=c["pt"], time_table=c["tt"], timestamps=ts)
        start = 0 if cut < 25 else 25
        assert np.array_equal(pert[start:cut + 1], base[start:cut + 1])


def test_linear_in_v_and_divisor_scaling():
    c = _tiny_case(8, [19, 40])
    args = dict(pos_table=c["pt"], time_table=c["tt"], timestamps=c["ts"])
    v2 = np.random.default_rng(80).standard_normal(c["v"].shape)
    f = lambda v, **kw: O.attn_fwd(c["q"], c["k"], v, c["off"], **args, **kw)  # noqa: E731
    lhs = f(2.5 * c["v"] - 0.75 * v2)
    rhs = 2.5 * f(c["v"]) - 0.75 * f(v2)
    assert _rel(lhs, rhs) < 1e-13
    assert _rel(3.0 * f(c["v"], divisor=3.0), 11.0 * f(c["v"], divisor=11.0)) < 1e-14
    # per-sequence divisor: each sequence scales with its own length
    fixed = f(c["v"], divisor=1.0)
    per = f(c["v"])
    assert _rel(per[:19] * 19, fixed[:19]) < 1e-14
    assert _rel(per[19:] * 40, fixed[19:]) < 1e-14


def test_jagged_batch_equals_sequences_alone_and_heads_commute():
    c = _tiny_case(9, [11, 0, 23, 5])
    full = O.attn_fwd(c["q"], c["k"], c["v"], c["off"], pos_table=c["pt"],
                      time_table=c["tt"], timestamps=c["ts"])
    off = c["off"]
    for b in range(len(off) - 1):
        s = slice(off[b], off[b + 1])
        n = off[b + 1] - off[b]
        alone = O.attn_fwd(c["q"][s], c["k"][s], c["v"][s], np.array([0, n]), pos_table=c["pt"],
                           time_table=c["tt"], timestamps=c["ts"][s])
        assert np.array_equal(alone, full[s])
    perm = [1, 0]
    pp = O.attn_fwd(c["q"][:, perm], c["k"][:, perm], c["v"][:, perm], off,
                    pos_table=c["pt"][perm], time_table=c["tt"][perm], timestamps=c["ts"])
    assert np.array_equal(pp, full[:, perm])


def test_mask_is_applied_after_silu():
    """A huge negative score on a future pair must give exactly 0 (mask after
    SiLU), and a finite pre-activation on past pairs must not be touched."""
    n = 4
    q = np.zeros((n, 1, 1))
    k = np.zeros((n, 1, 1))
    q[0, 0, 0], k[3, 0, 0] = 1e300, -1e300   # S_03 = -inf (j > i, masked)
    v = np.ones((n, 1, 1))
    out = O.attn_fwd(q, k, v, np.array([0, n]))
    assert np.all(np.isfinite(out))


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
def test_bwd_matches_brute_force_loops():
    c = _tiny_case(10, [4, 1, 0, 6], H=2, d=3, dv=2, Bp=4, Bt=5)
    for alpha, divisor in [(1.0, 0.0), (0.8, 3.0)]:
        ref = B.attn_bwd(c["q"], c["k"], c["v"], c["do"], c["off"], alpha, divisor,
                         c["pt"], c["tt"], c["ts"])
        got = O.attn_bwd(c["q"], c["k"], c["v"], c["do"], c["off"], alpha=alpha, divisor=divisor,
                         pos_table=c["pt"], time_table=c["tt"], timestamps=c["ts"], row_block=2)
        for g, r in zip(got, ref):
            assert _rel(g, r) < 1e-12


def _fd_check(q, k, v, do, off, pt, tt, ts, alpha=1.0, divisor=0.0, h=1e-6, tol=1e-6):
    kw = dict(alpha=alpha, divisor=divisor, pos_table=pt, time_table=tt, timestamps=ts)
    an = O.attn_bwd(q, k, v, do, off, **kw)

    def loss(q_, k_, v_, pt_, tt_):
        o = O.attn_fwd(q_, k_, v_, off, alpha=alpha, divisor=divisor, pos_table=pt_,
                       time_table=tt_, timestamps=ts)
        return float(np.sum(o * do))

    arrays = [q, k, v, pt, tt]
    for which, arr in enumerate(arrays):
        if arr is None:
            continue
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = [a.copy() if a is not None else None for a in arrays]
            minus = [a.copy() if a is not None else None for a in arrays]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert _rel(fd, an[which]) < tol, which


def test_bwd_finite_differences_small_random():
    c = _tiny_case(11, [3, 5], H=2, d=2, dv=3, Bp=3, Bt=4)
    _fd_check(c["q"], c["k"], c["v"], c["do"], c["off"], c["pt"], c["tt"], c["ts"], alpha=0.9)


def test_bwd_finite_differences_three_token_slice_of_c4():
    """The first three tokens of the jagged fwd+bwd workload's sequence 0 as a
    standalone n = 3 sequence (its own divisor 3), all heads, both tables."""
    wl = make_workload("c4")
    s = slice(0, 3)
    args = [np.asarray(a[s], np.float64) for a in (wl.q, wl.k, wl.v, wl.d_o)]
    _fd_check(*args, np.array([0, 3]), np.asarray(wl.pos_table, np.float64),
              np.asarray(wl.time_table, np.float64), wl.timestamps[s])


def test_bwd_dv_is_a_transpose_times_do_and_table_sums_agree():
    rng = np.random.default_rng(12)
    n, H, d = 21, 2, 4
    q, k, v, do = (rng.standard_normal((n, H, d)) for _ in range(4))
    ts = np.sort(rng.integers(0, 5000, size=n)).astype(np.int64)
    pt = rng.standard_normal((H, 6)) * 0.3
    tt = rng.standard_normal((H, 8)) * 0.3
    dq, dk, dv, dP, dTt = O.attn_bwd(q, k, v, do, np.array([0, n]), pos_table=pt,
                                     time_table=tt, timestamps=ts, row_block=5)
    # rebuild A densely from the pages' expression plus the bias terms
    for h in range(H):
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        s = q[:, h] @ k[:, h].T + pt[h][np.clip(i - j, 0, 5)]
        gap = np.maximum(ts[:, None] - ts[None, :], 0)
        s = s + tt[h][np.minimum(np.floor(np.log2(1 + gap)).astype(int), 7)]
        sig = 1 / (1 + np.exp(-s))
        a = np.tril(s * sig) / n
        assert _rel(dv[:, h], a.T @ do[:, h]) < 1e-13
        ds = np.tril((do[:, h] @ v[:, h].T) * sig * (1 + s * (1 - sig))) / n
        assert abs(dP[h].sum() - ds.sum()) < 1e-12 * max(1, abs(ds).sum())
        assert abs(dTt[h].sum() - ds.sum()) < 1e-12 * max(1, abs(ds).sum())
        assert _rel(dq[:, h], ds @ k[:, h]) < 1e-13
        assert _rel(dk[:, h], ds.T @ q[:, h]) < 1e-13


# ----------------------------------------------------------------------------
# layer
# ----------------------------------------------------------------------------
def _tiny_layer(seed, T_lengths, D=6, H=2, d=3, time=True):
    rng = np.random.default_rng(seed)
    off = offsets_from_lengths(T_lengths)
    T = int(off[-1])
    n_uvqk = H * 4 * d
    p = dict(
        w_uvqk=rng.standard_normal((n_uvqk, D)) * 0.5, b_uvqk=rng.standard_normal(n_uvqk) * 0.1,
        w_out=rng.standard_normal((D, H * d)) * 0.5, b_out=rng.standard_normal(D) * 0.1,
        ln_in_gamma=1 + 0.1 * rng.standard_normal(D), ln_in_beta=0.1 * rng.standard_normal(D),
        ln_out_gamma=1 + 0.1 * rng.standard_normal(H * d),
        ln_out_beta=0.1 * rng.standard_normal(H * d),
        pos_table=rng.standard_normal((H, 4)) * 0.2,
        time_table=rng.standard_normal((H, 5)) * 0.2 if time else None)
    x = rng.standard_normal((T, D))
    ts = np.sort(rng.integers(0, 100, size=T)).astype(np.int64) if time else None
    return x, p, off, ts


def test_layer_matches_brute_force_loops():
    x, p, off, ts = _tiny_layer(13, [4, 0, 3])
    ref = B.layer_fwd(x, p, off, 2, 3, 3, timestamps=ts)
    got, _ = O.layer_fwd(x, p, off, num_heads=2, dqk=3, dv=3, timestamps=ts)
    assert _rel(got, ref) < 1e-12


def test_stack_matches_brute_force_layers_in_turn():
    """A two-layer stack is the brute-force layer loops applied twice, the
    second on the first's output."""
    x, p1, off, ts = _tiny_layer(19, [5, 1, 3])
    _, p2, _, _ = _tiny_layer(23, [5, 1, 3])
    mid = B.layer_fwd(x, p1, off, 2, 3, 3, timestamps=ts)
    ref = B.layer_fwd(np.array(mid), p2, off, 2, 3, 3, timestamps=ts)
    got = O.stack_fwd(x, [p1, p2], off, num_heads=2, dqk=3, dv=3, timestamps=ts)
    assert _rel(got, ref) < 1e-12


def test_stack_with_zero_output_projections_is_identity():
    x, p, off, ts = _tiny_layer(29, [4, 2])
    p = dict(p)
    p["w_out"] = np.zeros_like(p["w_out"])
    if p.get("b_out") is not None:
        p["b_out"] = np.zeros_like(p["b_out"])
    got = O.stack_fwd(x, [p, p, p], off, num_heads=2, dqk=3, dv=3, timestamps=ts)
    assert np.array_equal(got, x)


def test_layer_rows_match_full_layer():
    x, p, off, ts = _tiny_layer(17, [6, 0, 9])
    full, _ = O.layer_fwd(x, p, off, num_heads=2, dqk=3, dv=3, timestamps=ts)
    rows = [0, 5, 6, 14, 10]
    got = O.layer_fwd_rows(x, p, off, rows, num_heads=2, dqk=3, dv=3, timestamps=ts)
    assert _rel(got, full[rows]) < 1e-13


def test_layer_zero_out_projection_is_identity():
    x, p, off, ts = _tiny_layer(14, [5, 4])
    p["w_out"] = np.zeros_like(p["w_out"])
    p["b_out"] = np.zeros_like(p["b_out"])
    got, _ = O.layer_fwd(x, p, off, num_heads=2, dqk=3, dv=3, timestamps=ts)
    assert np.array_equal(got, x)


def test_layer_zero_u_gate_adds_only_output_bias():
    x, p, off, ts = _tiny_layer(15, [5, 4])
    H, d = 2, 3
    p["w_uvqk"][0:H * d] = 0.0     # U columns (first block of the u|v|q|k split)
    p["b_uvqk"][0:H * d] = 0.0
    got, inter = O.layer_fwd(x, p, off, num_heads=H, dqk=d, dv=d, timestamps=ts)
    assert np.all(inter["uvqk"][:, :H * d] == 0.0)
    assert np.array_equal(got, x + p["b_out"])


def test_layer_norm_of_constant_row_is_beta():
    beta = np.array([0.5, -1.0, 2.0])
    out = O.layer_norm(np.full((4, 3), 7.25), np.array([3.0, 4.0, 5.0]), beta, 1e-6)
    assert np.array_equal(out, np.broadcast_to(beta, (4, 3)))


def test_layer_split_order_u_v_q_k():
    """Put a distinct constant in each of the four column blocks' biases with
    zero weights: u, v, q and k come out as SiLU of their own constant."""
    x, p, off, ts = _tiny_layer(16, [3])
    H, d = 2, 3
    p["w_uvqk"][:] = 0.0
    for blk, c in enumerate([0.1, 0.2, 0.3, 0.4]):
        p["b_uvqk"][blk * H * d:(blk + 1) * H * d] = c
    _, inter = O.layer_fwd(x, p, off, num_heads=H, dqk=d, dv=d, timestamps=ts)
    for blk, c in enumerate([0.1, 0.2, 0.3, 0.4]):
        block = inter["uvqk"][:, blk * H * d:(blk + 1) * H * d]
        assert np.allclose(block, c / (1 + math.exp(-c)), rtol=0, atol=1e-16)


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def test_generators_are_deterministic_and_shaped():
    a, b = make_workload("c3_small"), make_workload("c3_small")
    for name in ("q", "k", "v", "timestamps", "pos_table", "time_table", "seq_offsets"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c0 = make_workload("c0")
    assert c0.q.shape == (256, 2, 32) and c0.pos_table.shape == (2, 64)
    c2 = make_workload("c2_small")
    assert c2.x.shape == (c2.total_tokens, 512)
    assert c2.layers[0]["w_uvqk"].shape == (2048, 512)
    assert c2.layers[0]["w_out"].shape == (512, 512)
    # timestamps are non-decreasing inside each sequence and start at t0
    off = c2.seq_offsets
    for b_ in range(c2.num_seqs):
        t = c2.timestamps[off[b_]:off[b_ + 1]]
        if t.size:
            assert t[0] == 1_700_000_000 and np.all(np.diff(t) >= 0)


def test_exponential_timestamps_mean_gap():
    rng = np.random.default_rng(0)
    ts = exponential_timestamps(rng, [200000])
    gap = np.diff(ts).mean()
    assert 3550 < gap < 3650   # floor() lowers the mean by ~0.5 s


# ----------------------------------------------------------------------------
# layer backward
# ----------------------------------------------------------------------------
def _layer_loss(x, p, off, ts, d_out, H, d, eps=1e-6):
    out, _ = O.layer_fwd(x, p, off, num_heads=H, dqk=d, dv=d, timestamps=ts, eps=eps)
    return float(np.sum(out * d_out))


@pytest.mark.parametrize("time", [True, False])
def test_layer_bwd_finite_differences(time):
    """Every entry of X and of every parameter (both norms, both projections
    and their biases, both bias tables) against central differences of
    sum(X' * dOut), fp64, h = 1e-6, two jagged sequences."""
    H, d, D = 2, 3, 6
    x, p, off, ts = _tiny_layer(31, [3, 4], D=D, H=H, d=d, time=time)
    rng = np.random.default_rng(32)
    d_out = rng.standard_normal(x.shape)
    dx, grads = O.layer_bwd(x, p, off, d_out, num_heads=H, dqk=d, dv=d, timestamps=ts)
    h = 1e-6

    def fd_of(get, put):
        base = get().copy()
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            for sgn in (1, -1):
                a = base.copy()
                a[idx] += sgn * h
                put(a)
                fd[idx] += sgn * _layer_loss(x_cur[0], p, off, ts, d_out, H, d)
            fd[idx] /= 2 * h
        put(base)
        return fd

    x_cur = [x.copy()]
    fd = fd_of(lambda: x_cur[0], lambda a: x_cur.__setitem__(0, a))
    assert _rel(fd, dx) < 1e-6
    for key in ("w_uvqk", "b_uvqk", "w_out", "b_out", "ln_in_gamma", "ln_in_beta",
                "ln_out_gamma", "ln_out_beta", "pos_table", "time_table"):
        if p.get(key) is None:
            assert ("d_" + key) not in grads
            continue
        fd = fd_of(lambda k=key: p[k], lambda a, k=key: p.__setitem__(k, a))
        assert _rel(fd, grads["d_" + key]) < 1e-6, key


def test_layer_norm_bwd_rows_are_mean_free_and_orthogonal_to_xhat():
    """LN's input gradient has zero mean and, with eps = 0 and gamma = 1, is
    orthogonal to the normalised row (the projection of the upstream gradient
    onto the complement of span{1, xhat}, scaled by 1/sigma)."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((7, 16)) * 3 + 1
    dy = rng.standard_normal((7, 16))
    dx, dg, db = O.layer_norm_bwd(x, np.ones(16), dy, 0.0)
    mu = x.mean(1, keepdims=True)
    xhat = (x - mu) / np.sqrt(((x - mu) ** 2).mean(1, keepdims=True))
    assert np.abs(dx.sum(1)).max() < 1e-12
    assert np.abs((dx * xhat).sum(1)).max() < 1e-10
    assert np.allclose(db, dy.sum(0)) and np.allclose(dg, (dy * xhat).sum(0))


def test_layer_bwd_zero_out_projection_leaves_only_residual_and_weight_grads():
    """W_out = 0: dX = dOut exactly, and every gradient upstream of the output
    projection (norms, W_uvqk, tables) is exactly zero, while d_W_out = dOut^T Y."""
    H, d, D = 2, 3, 6
    x, p, off, ts = _tiny_layer(34, [5, 2], D=D, H=H, d=d)
    p["w_out"] = np.zeros_like(p["w_out"])
    d_out = np.random.default_rng(35).standard_normal(x.shape)
    dx, grads = O.layer_bwd(x, p, off, d_out, num_heads=H, dqk=d, dv=d, timestamps=ts)
    assert np.array_equal(dx, d_out)
    for key in ("d_w_uvqk", "d_b_uvqk", "d_ln_in_gamma", "d_ln_in_beta", "d_ln_out_gamma",
                "d_ln_out_beta", "d_pos_table", "d_time_table"):
        assert not np.any(grads[key]), key
    _, inter = O.layer_fwd(x, p, off, num_heads=H, dqk=d, dv=d, timestamps=ts)
    assert _rel(grads["d_w_out"], d_out.T @ inter["y"]) < 1e-13
    assert _rel(grads["d_b_out"], d_out.sum(0)) < 1e-13


# ----------------------------------------------------------------------------
# candidate scoring against a cached history
# ----------------------------------------------------------------------------
def _cand_case(seed, hist_lengths, cand_counts, H=2, d=3, Bp=5, Bt=6):
    rng = np.random.default_rng(seed)
    hoff = offsets_from_lengths(hist_lengths)
    coff = offsets_from_lengths(cand_counts)
    Th, Tc = int(hoff[-1]), int(coff[-1])
    qh, kh, vh = (rng.standard_normal((Th, H, d)) for _ in range(3))
    qc, kc, vc = (rng.standard_normal((Tc, H, d)) for _ in range(3))
    ts = np.concatenate([np.sort(rng.integers(0, 2000, n)) for n in hist_lengths]).astype(np.int64)
    cts = np.concatenate([np.full(m, 2100 + 7 * i) for i, m in enumerate(cand_counts)]).astype(np.int64)
    pt = rng.standard_normal((H, Bp)) * 0.3
    tt = rng.standard_normal((H, Bt)) * 0.3
    return dict(qc=qc, kc=kc, vc=vc, coff=coff, kh=kh, vh=vh, qh=qh, hoff=hoff, ts=ts, cts=cts, pt=pt, tt=tt)


def _cand(c, **kw):
    return O.attn_fwd_candidates(c["qc"], c["kc"], c["vc"], c["coff"], c["kh"], c["vh"], c["qh"], c["hoff"],
                                 pos_table=c["pt"], time_table=c["tt"], timestamps=c["ts"],
                                 cand_timestamps=c["cts"], **kw)


def test_candidates_equal_appending_each_one_to_its_history_by_brute_force():
    """Each candidate's output against the pure-Python loops of the forward on
    (history ++ [candidate]) -- an independent transcription of the pages'
    expression -- for several histories, including an empty one."""
    c = _cand_case(51, [4, 0, 6], [2, 3, 1])
    got = _cand(c, alpha=0.8)
    for b in range(3):
        h0, h1 = int(c["hoff"][b]), int(c["hoff"][b + 1])
        for j in range(int(c["coff"][b]), int(c["coff"][b + 1])):
            cat = lambda hist, cand: np.concatenate([hist[h0:h1], cand[j:j + 1]])
            ts = np.concatenate([c["ts"][h0:h1], c["cts"][j:j + 1]])
            ref = B.attn_fwd(cat(c["qh"], c["qc"]), cat(c["kh"], c["kc"]), cat(c["vh"], c["vc"]),
                             np.array([0, h1 - h0 + 1]), 0.8, 0.0, c["pt"], c["tt"], ts)
            assert _rel(got[j], ref[-1]) < 1e-12


def test_candidates_do_not_see_each_other():
    """Changing one candidate's q, k, v leaves every other candidate's output
    bitwise unchanged; permuting candidates permutes outputs."""
    c = _cand_case(52, [5, 3], [4, 3])
    base = _cand(c)
    c2 = dict(c)
    for key in ("qc", "kc", "vc"):
        c2[key] = c[key].copy()
        c2[key][1] += 3.0
    other = _cand(c2)
    keep = [i for i in range(base.shape[0]) if i != 1]
    assert np.array_equal(base[keep], other[keep])
    perm = np.array([2, 0, 3, 1, 5, 6, 4])
    c3 = dict(c, qc=c["qc"][perm], kc=c["kc"][perm], vc=c["vc"][perm], cts=c["cts"][perm])
    assert _rel(_cand(c3), base[perm]) < 1e-13


def test_candidates_with_zero_history_are_self_attention_of_one_token():
    """No history: O_c = SiLU(alpha q.k + P[0] + Tt[0]) v_c / 1, a closed form."""
    c = _cand_case(53, [0], [3], H=1, d=4)
    got = _cand(c, alpha=1.3)
    s = 1.3 * np.einsum("thd,thd->th", c["qc"], c["kc"]) + c["pt"][0, 0] + c["tt"][0, 0]
    ref = (s / (1 + np.exp(-s)))[..., None] * c["vc"]
    assert _rel(got, ref) < 1e-13


# ----------------------------------------------------------------------------
# final RMSNorm and tied retrieval head
# ----------------------------------------------------------------------------
def test_head_matches_torch_rms_norm_and_linear():
    """The library's own RMSNorm and bias-free linear map, in float64 on the CPU."""
    import torch
    rng = np.random.default_rng(70)
    x = rng.standard_normal((37, 64)) * rng.uniform(0.01, 3.0, size=(37, 1))
    gamma = 1 + 0.3 * rng.standard_normal(64)
    table = 0.02 * rng.standard_normal((301, 64))
    eps = 1e-6
    ref = torch.nn.functional.linear(
        torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(gamma), eps),
        torch.from_numpy(table)).numpy()
    got = O.head_fwd(x, table, gamma, eps)
    assert got.shape == (37, 301)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_rms_norm_constant_row_and_unit_rms():
    """eps = 0: a constant row c maps to sign(c) * gamma; any nonzero row has
    mean square exactly 1 with gamma = 1; a zero row stays zero (eps > 0)."""
    rng = np.random.default_rng(71)
    gamma = rng.standard_normal(32)
    for c in (3.5, -0.25):
        np.testing.assert_allclose(O.rms_norm(np.full((1, 32), c), gamma, 0.0)[0], np.sign(c) * gamma,
                                   rtol=1e-14)
    y = O.rms_norm(rng.standard_normal((9, 32)) * 7.0, None, 0.0)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-13)
    z = O.rms_norm(np.zeros((2, 32)), gamma, 1e-6)
    assert np.all(z == 0.0)


def test_head_scale_invariance_and_sign():
    """eps = 0: scaling a token row by s > 0 leaves its logits unchanged, a
    negative s negates them (the norm divides by the root mean square, not by
    the variance about the mean)."""
    rng = np.random.default_rng(72)
    x = rng.standard_normal((5, 48)) + 2.0
    table = rng.standard_normal((20, 48))
    gamma = rng.uniform(0.5, 1.5, 48)
    base = O.head_fwd(x, table, gamma, 0.0)
    np.testing.assert_allclose(O.head_fwd(13.0 * x, table, gamma, 0.0), base, rtol=1e-12)
    np.testing.assert_allclose(O.head_fwd(-0.5 * x, table, gamma, 0.0), -base, rtol=1e-12)


def test_head_with_basis_table_is_a_gather_of_the_normalised_row():
    """Table row i = unit vector e_{p(i)}: logit i is feature p(i) of the normalised row."""
    rng = np.random.default_rng(73)
    D = 16
    x = rng.standard_normal((4, D))
    gamma = rng.standard_normal(D)
    perm = rng.permutation(D)
    table = np.eye(D)[perm]
    y = O.rms_norm(x, gamma, 1e-6)
    np.testing.assert_array_equal(O.head_fwd(x, table, gamma, 1e-6), y[:, perm])


def test_tied_head_retrieves_each_token_own_item():
    """Tied weights: tokens are rows of the same table the head scores
    against. With equal-norm rows, gamma = 1 and eps = 0, the own item's logit
    is sqrt(D) * |e| (Cauchy-Schwarz maximum) and it is the arg max."""
    rng = np.random.default_rng(74)
    V, D, r = 500, 64, 0.3
    table = rng.standard_normal((V, D))
    table *= r / np.linalg.norm(table, axis=1, keepdims=True)
    ids = rng.integers(0, V, size=40)
    logits = O.head_fwd(table[ids], table, None, 0.0)
    np.testing.assert_allclose(logits[np.arange(40), ids], math.sqrt(D) * r, rtol=1e-12)
    assert np.array_equal(logits.argmax(axis=1), ids)


# ----------------------------------------------------------------------------
# Stochastic Length
# ----------------------------------------------------------------------------
def _kept_by_counting(keys, s, e, L):
    """Brute force: token i of [s, e) is kept iff fewer than L tokens of its
    sequence have a smaller (key, position) pair."""
    out = []
    for i in range(s, e):
        smaller = sum(1 for j in range(s, e) if (int(keys[j]), j) < (int(keys[i]), i))
        if smaller < L:
            out.append(i)
    return out


def test_stochastic_length_matches_pairwise_counting():
    rng = np.random.default_rng(80)
    lengths = [0, 1, 7, 8, 9, 30, 3, 64]
    off = offsets_from_lengths(lengths)
    keys = rng.integers(0, 1 << 32, size=int(off[-1]), dtype=np.uint64).astype(np.uint32)
    keys[off[5]:off[6]] %= 4                     # heavy ties in one sequence
    keys[off[7]:off[7] + 10] = 0xFFFFFFFF        # ties at the largest key
    L = 8
    new_off, idx = O.stochastic_length(off, keys, L)
    assert np.array_equal(new_off, offsets_from_lengths(np.minimum(lengths, L)))
    want = []
    for b in range(len(lengths)):
        want += _kept_by_counting(keys, int(off[b]), int(off[b + 1]), L)
    assert np.array_equal(idx, np.array(want, np.int64))


def test_stochastic_length_short_sequences_and_zero_cap():
    off = offsets_from_lengths([3, 0, 5])
    keys = np.arange(8, dtype=np.uint32)[::-1].copy()
    new_off, idx = O.stochastic_length(off, keys, 5)
    assert np.array_equal(new_off, off) and np.array_equal(idx, np.arange(8))
    new_off, idx = O.stochastic_length(off, keys, 0)
    assert np.array_equal(new_off, np.zeros(4, np.int64)) and idx.size == 0
    # all keys equal: the first L positions of each long sequence
    new_off, idx = O.stochastic_length(off, np.zeros(8, np.uint32), 2)
    assert np.array_equal(idx, [0, 1, 3, 4])
    # strictly decreasing keys: the last L positions
    new_off, idx = O.stochastic_length(off, keys, 2)
    assert np.array_equal(idx, [1, 2, 6, 7])


def test_stochastic_length_is_a_uniform_subsample():
    """Independent uniform keys: each of the n positions is kept with
    probability L / n, and the kept set's first position follows the
    hypergeometric minimum, P(first >= m) = C(n - m, L) / C(n, L)."""
    rng = np.random.default_rng(81)
    n, L, draws = 40, 10, 4000
    off = np.array([0, n], np.int64)
    counts = np.zeros(n)
    firsts = np.zeros(n + 1)
    for _ in range(draws):
        keys = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
        _, idx = O.stochastic_length(off, keys, L)
        assert idx.size == L and np.all(np.diff(idx) > 0)
        counts[idx] += 1
        firsts[idx[0]] += 1
    p = L / n
    sd = math.sqrt(p * (1 - p) / draws)
    assert np.all(np.abs(counts / draws - p) < 5 * sd)
    for m in (1, 3, 6):
        exact = math.comb(n - m, L) / math.comb(n, L)
        seen = firsts[m:].sum() / draws
        assert abs(seen - exact) < 5 * math.sqrt(exact * (1 - exact) / draws), (m, seen, exact)
