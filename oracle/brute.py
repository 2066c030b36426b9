"""Pure-Python loop restatement of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY. Every sum is an explicit loop over Python floats;
the bucket functions use integer shifts; no NumPy arithmetic is used. It is
the second, independent form the fp64 oracle is checked against on tiny
inputs (n <= 8, H <= 2, d <= 4).
"""

from __future__ import annotations

import math


def _silu(x: float) -> float:
    if x < -700.0:
        return -0.0
    return x / (1.0 + math.exp(-x))


def _sig(x: float) -> float:
    if x < -700.0:
        return 0.0
    return 1.0 / (1.0 + math.exp(-x))


def pos_bucket(delta: int, nb: int) -> int:
    """min(i - j, nb - 1) for i - j >= 0."""
    return min(max(int(delta), 0), nb - 1)


def time_bucket(dt: int, nb: int) -> int:
    """min(floor(log2(1 + max(dt, 0))), nb - 1) by counting right shifts."""
    x = 1 + max(int(dt), 0)
    c = -1
    while x > 0:
        x >>= 1
        c += 1
    return min(c, nb - 1)


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def _score(q, k, ts, pt, tt, o0, i, j, h, alpha):
    s = 0.0
    for d in range(len(q[o0 + i][h])):
        s += float(q[o0 + i][h][d]) * float(k[o0 + j][h][d])
    s *= alpha
    if pt is not None:
        s += float(pt[h][pos_bucket(i - j, len(pt[h]))])
    if tt is not None:
        s += float(tt[h][time_bucket(int(ts[o0 + i]) - int(ts[o0 + j]), len(tt[h]))])
    return s


def attn_fwd(q, k, v, seq_offsets, alpha=1.0, divisor=0.0, pos_table=None,
             time_table=None, timestamps=None):
    """O[t][h][e] by explicit loops over sequences, heads, rows and columns j <= i."""
    q, k, v = _tolist(q), _tolist(k), _tolist(v)
    off = [int(x) for x in _tolist(seq_offsets)]
    pt = None if pos_table is None else _tolist(pos_table)
    tt = None if time_table is None else _tolist(time_table)
    ts = None if timestamps is None else [int(x) for x in _tolist(timestamps)]
    T, H, dv = len(q), (len(q[0]) if q else 0), (len(v[0][0]) if v else 0)
    out = [[[0.0] * dv for _ in range(H)] for _ in range(T)]
    for b in range(len(off) - 1):
        o0, n = off[b], off[b + 1] - off[b]
        denom = float(n) if divisor <= 0 else float(divisor)
        for h in range(H):
            for i in range(n):
                for j in range(i + 1):
                    a = _silu(_score(q, k, ts, pt, tt, o0, i, j, h, alpha)) / denom
                    for e in range(dv):
                        out[o0 + i][h][e] += a * float(v[o0 + j][h][e])
    return out


def attn_bwd(q, k, v, d_o, seq_offsets, alpha=1.0, divisor=0.0, pos_table=None,
             time_table=None, timestamps=None):
    """(dq, dk, dv, dP, dTt) by explicit loops (same formulas as the oracle)."""
    q, k, v, d_o = _tolist(q), _tolist(k), _tolist(v), _tolist(d_o)
    off = [int(x) for x in _tolist(seq_offsets)]
    pt = None if pos_table is None else _tolist(pos_table)
    tt = None if time_table is None else _tolist(time_table)
    ts = None if timestamps is None else [int(x) for x in _tolist(timestamps)]
    T, H = len(q), (len(q[0]) if q else 0)
    dqk, dvd = len(q[0][0]), len(v[0][0])
    dq = [[[0.0] * dqk for _ in range(H)] for _ in range(T)]
    dk = [[[0.0] * dqk for _ in range(H)] for _ in range(T)]
    dv = [[[0.0] * dvd for _ in range(H)] for _ in range(T)]
    dP = None if pt is None else [[0.0] * len(pt[0]) for _ in range(H)]
    dTt = None if tt is None else [[0.0] * len(tt[0]) for _ in range(H)]
    for b in range(len(off) - 1):
        o0, n = off[b], off[b + 1] - off[b]
        denom = float(n) if divisor <= 0 else float(divisor)
        for h in range(H):
            for i in range(n):
                for j in range(i + 1):
                    s = _score(q, k, ts, pt, tt, o0, i, j, h, alpha)
                    sg = _sig(s)
                    a = s * sg / denom
                    da = 0.0
                    for e in range(dvd):
                        da += float(d_o[o0 + i][h][e]) * float(v[o0 + j][h][e])
                        dv[o0 + j][h][e] += a * float(d_o[o0 + i][h][e])
                    ds = da * sg * (1.0 + s * (1.0 - sg)) / denom
                    for e in range(dqk):
                        dq[o0 + i][h][e] += alpha * ds * float(k[o0 + j][h][e])
                        dk[o0 + j][h][e] += alpha * ds * float(q[o0 + i][h][e])
                    if dP is not None:
                        dP[h][pos_bucket(i - j, len(pt[h]))] += ds
                    if dTt is not None:
                        dTt[h][time_bucket(ts[o0 + i] - ts[o0 + j], len(tt[h]))] += ds
    return dq, dk, dv, dP, dTt


def layer_norm_row(x, gamma, beta, eps):
    n = len(x)
    mu = sum(float(a) for a in x) / n
    var = sum((float(a) - mu) ** 2 for a in x) / n
    r = 1.0 / math.sqrt(var + eps)
    return [(float(a) - mu) * r * float(g) + float(bb) for a, g, bb in zip(x, gamma, beta)]


def layer_fwd(x, params, seq_offsets, num_heads, dqk, dv, timestamps=None, eps=1e-6):
    """One HSTU layer by loops: LN -> x W_uvqk^T + b -> SiLU -> split u|v|q|k ->
    attention -> LN(o) * u -> x + y W_out^T + b_out."""
    x = _tolist(x)
    W1 = _tolist(params["w_uvqk"])
    b1 = _tolist(params["b_uvqk"])
    W2 = _tolist(params["w_out"])
    b2 = _tolist(params["b_out"])
    H = num_heads
    T, D = len(x), len(x[0])
    g = []
    for t in range(T):
        xn = layer_norm_row(x[t], params["ln_in_gamma"], params["ln_in_beta"], eps)
        row = []
        for o in range(len(W1)):
            z = float(b1[o])
            for c in range(D):
                z += xn[c] * float(W1[o][c])
            row.append(_silu(z))
        g.append(row)
    u = [row[0:H * dv] for row in g]
    vv = [[row[H * dv + hh * dv:H * dv + (hh + 1) * dv] for hh in range(H)] for row in g]
    base_q = 2 * H * dv
    qq = [[row[base_q + hh * dqk:base_q + (hh + 1) * dqk] for hh in range(H)] for row in g]
    base_k = base_q + H * dqk
    kk = [[row[base_k + hh * dqk:base_k + (hh + 1) * dqk] for hh in range(H)] for row in g]
    o = attn_fwd(qq, kk, vv, seq_offsets, pos_table=params.get("pos_table"),
                 time_table=params.get("time_table"), timestamps=timestamps)
    out = []
    for t in range(T):
        flat = [o[t][hh][e] for hh in range(H) for e in range(dv)]
        yn = layer_norm_row(flat, params["ln_out_gamma"], params["ln_out_beta"], eps)
        y = [yn[c] * u[t][c] for c in range(H * dv)]
        row = []
        for r in range(D):
            acc = float(b2[r])
            for c in range(H * dv):
                acc += y[c] * float(W2[r][c])
            row.append(float(x[t][r]) + acc)
        out.append(row)
    return out
