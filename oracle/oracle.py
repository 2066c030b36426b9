"""Plain fp64 NumPy oracle of the HSTU layer's hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports, calls or falls back to this module.

Sources, cited by page title and section:

* neurarch "HSTU (Generative Recommender)" model card, section "Exported
  PyTorch", ``HSTUBlock``: the fused u|v|q|k projection and its split order,
  the per-head views, and the pointwise aggregation -- SiLU of q.k^T divided
  by the sequence length, lower-triangular (causal, diagonal kept) mask taken
  after the SiLU, then multiplied by v. No softmax.
* neurarch model card, section "Structure", and the neurarch graph JSON of
  the same model (its "norm" and "head" nodes): the final RMSNorm (eps 1e-6)
  and the tied, bias-free retrieval head.
* briansu.co explainer, section 6 "Why it works": Stochastic Length (random
  shortening of long training histories) and M-FALCON (candidate scoring
  with the history's keys and values reused).
* briansu.co "HSTU: Hierarchical Sequential Transduction Units", section 3
  "How it works": the three steps of a layer (pointwise projection to
  U, V, Q, K; spatial aggregation by pointwise SiLU attention with relative
  position and time biases; gated pointwise transformation).
* daiwk.github.io HSTU reproduction notes, section "core formula" and the
  flowchart of "background and main changes": U, V, Q, K = SiLU(Norm(X) W),
  causal pointwise aggregation with relative bias, post-pooling
  normalisation, U gate, output projection with residual.

Where the pages leave a step open, the reading used here is stated in the
function's docstring (bucket functions, divisor, norm placement, SiLU on all
four projections).
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------
def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), in float64.

    For x below about -709, e^-x overflows to inf and the quotient is -0.0,
    which is the correctly rounded result.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def pos_bucket(delta: np.ndarray, num_buckets: int) -> np.ndarray:
    """Relative-position bucket of the distance delta = i - j >= 0.

    The pages name a relative position bias (briansu.co explainer, section 3)
    without its bucketing; the reading used is one bucket per distance,
    clamped: min(i - j, num_buckets - 1). Negative distances (masked pairs)
    map to bucket 0; their value never reaches the output.
    """
    d = np.asarray(delta, dtype=np.int64)
    return np.minimum(np.maximum(d, 0), num_buckets - 1)


def _floor_log2_of_positive(x: np.ndarray) -> np.ndarray:
    """floor(log2(x)) for int64 x >= 1, exactly.

    np.frexp(x) returns (m, e) with x = m * 2**e and 0.5 <= m < 1, so
    floor(log2(x)) = e - 1, exact whenever x converts to float64 without
    rounding (x < 2**53). Larger entries are done with Python's int.bit_length.
    """
    x = np.asarray(x, dtype=np.int64)
    _, e = np.frexp(x.astype(np.float64))
    out = e.astype(np.int64) - 1
    big = x >= (1 << 53)
    if np.any(big):
        flat = out.reshape(-1)
        for idx in np.flatnonzero(big.reshape(-1)):
            flat[idx] = int(x.reshape(-1)[idx]).bit_length() - 1
    return out


def time_bucket(dt: np.ndarray, num_buckets: int) -> np.ndarray:
    """Relative-time bucket of the timestamp gap dt = t_i - t_j (int64 seconds).

    The pages name a time-aware relative bias (briansu.co explainer, sections
    1 and 3) without its bucketing; the reading used is a log2 bucket of the
    gap: min(floor(log2(1 + max(dt, 0))), num_buckets - 1), computed exactly
    in integers (no floating-point log2 ties at powers of two). Gaps are
    clamped below 2**62 so that 1 + dt cannot overflow int64.
    """
    d = np.asarray(dt, dtype=np.int64)
    d = np.clip(d, 0, (1 << 62))
    return np.minimum(_floor_log2_of_positive(d + 1), num_buckets - 1)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _pre_activation(qb, kb, i0, i1, h, alpha, pos_table, time_table, ts_b):
    """S = alpha * q_i . k_j + P[h, pos(i-j)] + Tt[h, time(t_i - t_j)] for
    rows i in [i0, i1) and columns j in [0, i1) of one sequence and head.
    Returns (S, causal_mask, I, J)."""
    S = alpha * (qb[i0:i1] @ kb[:i1].T)
    I = np.arange(i0, i1, dtype=np.int64)[:, None]
    J = np.arange(0, i1, dtype=np.int64)[None, :]
    if pos_table is not None:
        S = S + pos_table[h][pos_bucket(I - J, pos_table.shape[1])]
    if time_table is not None:
        dt = ts_b[i0:i1][:, None] - ts_b[:i1][None, :]
        S = S + time_table[h][time_bucket(dt, time_table.shape[1])]
    return S, (J <= I), I, J


def _check_attn_args(q, k, v, seq_offsets, pos_table, time_table, timestamps):
    T, H, dqk = q.shape
    assert k.shape == (T, H, dqk), "k must match q"
    assert v.shape[:2] == (T, H), "v must be [T, H, dv]"
    off = np.asarray(seq_offsets, dtype=np.int64)
    assert off[0] == 0 and off[-1] == T and np.all(np.diff(off) >= 0), "bad seq_offsets"
    if time_table is not None:
        assert timestamps is not None, "time bias needs timestamps"
    if pos_table is not None:
        assert pos_table.shape[0] == H
    if time_table is not None:
        assert time_table.shape[0] == H
    return off


def attn_fwd(q, k, v, seq_offsets, *, alpha: float = 1.0, divisor: float = 0.0,
             pos_table=None, time_table=None, timestamps=None,
             row_block: int = 512) -> np.ndarray:
    """Causal pointwise aggregated attention over a jagged batch, float64.

    q, k: [T, H, dqk]; v: [T, H, dv]; seq_offsets: int64 [B+1];
    pos_table: [H, Bp] or None; time_table: [H, Bt] or None (needs int64
    timestamps [T]). For sequence b of length n and head h, with positions
    i, j inside the sequence:

        S_ij = alpha q_i.k_j + P[h, pos(i-j)] + Tt[h, time(t_i - t_j)]
        A_ij = SiLU(S_ij) / N   for j <= i,   0 for j > i
        O_i  = sum_j A_ij v_j

    N is n (per-sequence length; ``divisor <= 0``) or the constant
    ``divisor``. The neurarch exported block divides by its (padded) length
    and masks with a lower triangle after the SiLU; with jagged sequences the
    reading used is each sequence's own length. Returns O as float64
    [T, H, dv].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    pos_table, time_table = _f64(pos_table), _f64(time_table)
    off = _check_attn_args(q, k, v, seq_offsets, pos_table, time_table, timestamps)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    T, H, _ = q.shape
    dv = v.shape[2]
    out = np.zeros((T, H, dv), dtype=np.float64)
    for b in range(off.size - 1):
        o0, n = int(off[b]), int(off[b + 1] - off[b])
        if n == 0:
            continue
        denom = float(n) if divisor <= 0 else float(divisor)
        ts_b = None if ts is None else ts[o0:o0 + n]
        for h in range(H):
            qb, kb, vb = q[o0:o0 + n, h], k[o0:o0 + n, h], v[o0:o0 + n, h]
            for i0 in range(0, n, row_block):
                i1 = min(n, i0 + row_block)
                S, causal, _, _ = _pre_activation(qb, kb, i0, i1, h, alpha,
                                                  pos_table, time_table, ts_b)
                A = np.where(causal, silu(S), 0.0) / denom
                out[o0 + i0:o0 + i1, h] = A @ vb[:i1]
    return out


def attn_fwd_rows(q, k, v, seq_offsets, b: int, h: int, rows: Sequence[int], *,
                  alpha: float = 1.0, divisor: float = 0.0, pos_table=None,
                  time_table=None, timestamps=None) -> np.ndarray:
    """Selected output rows O_i (positions inside sequence b, head h), float64
    [len(rows), dv], each computed on its own from the definition in
    ``attn_fwd``. Cost O(i * d) per row, for sampled checks at full size."""
    off = np.asarray(seq_offsets, dtype=np.int64)
    o0, n = int(off[b]), int(off[b + 1] - off[b])
    denom = float(n) if divisor <= 0 else float(divisor)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    res = []
    for i in rows:
        i = int(i)
        assert 0 <= i < n
        qi = np.asarray(q[o0 + i, h], dtype=np.float64)
        kj = np.asarray(k[o0:o0 + i + 1, h], dtype=np.float64)
        vj = np.asarray(v[o0:o0 + i + 1, h], dtype=np.float64)
        s = alpha * (kj @ qi)
        j = np.arange(i + 1, dtype=np.int64)
        if pos_table is not None:
            pt = np.asarray(pos_table, dtype=np.float64)
            s = s + pt[h][pos_bucket(i - j, pt.shape[1])]
        if time_table is not None:
            tt = np.asarray(time_table, dtype=np.float64)
            dt = ts[o0 + i] - ts[o0:o0 + i + 1]
            s = s + tt[h][time_bucket(dt, tt.shape[1])]
        res.append((silu(s) / denom) @ vj)
    return np.array(res, dtype=np.float64).reshape(len(res), v.shape[2])


def attn_bwd(q, k, v, d_o, seq_offsets, *, alpha: float = 1.0, divisor: float = 0.0,
             pos_table=None, time_table=None, timestamps=None, row_block: int = 512):
    """Gradients of sum(O * dO) for ``attn_fwd``, float64, derived by hand.

    With sig = 1/(1+e^-S) and SiLU'(S) = sig (1 + S (1 - sig)), over pairs
    j <= i of the same sequence:

        dA_ij = dO_i . v_j
        dS_ij = dA_ij SiLU'(S_ij) / N
        dv_j  = sum_i A_ij dO_i            dq_i = alpha sum_j dS_ij k_j
        dk_j  = alpha sum_i dS_ij q_i
        dP[h, beta]  = sum of dS_ij over pairs with position bucket beta
        dTt[h, gam]  = sum of dS_ij over pairs with time bucket gam

    Offsets and timestamps are not differentiated. Returns
    (dq, dk, dv, d_pos_table or None, d_time_table or None).
    """
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    pos_table, time_table = _f64(pos_table), _f64(time_table)
    off = _check_attn_args(q, k, v, seq_offsets, pos_table, time_table, timestamps)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    T, H, _ = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dP = None if pos_table is None else np.zeros_like(pos_table)
    dTt = None if time_table is None else np.zeros_like(time_table)
    for b in range(off.size - 1):
        o0, n = int(off[b]), int(off[b + 1] - off[b])
        if n == 0:
            continue
        denom = float(n) if divisor <= 0 else float(divisor)
        ts_b = None if ts is None else ts[o0:o0 + n]
        for h in range(H):
            qb, kb, vb = q[o0:o0 + n, h], k[o0:o0 + n, h], v[o0:o0 + n, h]
            dob = d_o[o0:o0 + n, h]
            for i0 in range(0, n, row_block):
                i1 = min(n, i0 + row_block)
                S, causal, I, J = _pre_activation(qb, kb, i0, i1, h, alpha,
                                                  pos_table, time_table, ts_b)
                sig = sigmoid(S)
                A = np.where(causal, S * sig, 0.0) / denom
                dA = dob[i0:i1] @ vb[:i1].T
                dS = np.where(causal, dA * sig * (1.0 + S * (1.0 - sig)), 0.0) / denom
                dv[o0:o0 + i1, h] += A.T @ dob[i0:i1]
                dq[o0 + i0:o0 + i1, h] += alpha * (dS @ kb[:i1])
                dk[o0:o0 + i1, h] += alpha * (dS.T @ qb[i0:i1])
                if dP is not None:
                    bk = pos_bucket(I - J, pos_table.shape[1])
                    dP[h] += np.bincount(bk[causal], weights=dS[causal],
                                         minlength=pos_table.shape[1])
                if dTt is not None:
                    dt = ts_b[i0:i1][:, None] - ts_b[:i1][None, :]
                    bk = time_bucket(dt, time_table.shape[1])
                    dTt[h] += np.bincount(bk[causal], weights=dS[causal],
                                          minlength=time_table.shape[1])
    return dq, dk, dv, dP, dTt


def attn_fwd_candidates(q_c, k_c, v_c, cand_offsets, k_hist, v_hist, q_hist, seq_offsets, *,
                        alpha: float = 1.0, divisor: float = 0.0, pos_table=None,
                        time_table=None, timestamps=None, cand_timestamps=None):
    """Candidate scoring against a history with cached keys and values, float64
    (M-FALCON, "micro-batched candidate scoring with KV reuse": briansu.co
    explainer, section 6 "Why it works"). The pages give no formula; the
    reading used here: candidate c of sequence b, with an n-token history,
    is scored exactly as if it alone were appended at position n, i.e. its
    output is the last row of ``attn_fwd`` applied to (history ++ [c]) -- it
    attends to every history token and to itself, never to another candidate,
    and is divided by n + 1 (or by the fixed divisor).

    History tensors are [T_h, H, d] with ``seq_offsets``; candidates are
    [T_c, H, d] with ``cand_offsets`` (same number of sequences). ``q_hist``
    only fills the history rows of the per-candidate sequences (their outputs
    are discarded). Returns O for the candidates, [T_c, H, dv].
    """
    q_c, k_c, v_c = _f64(q_c), _f64(k_c), _f64(v_c)
    k_hist, v_hist, q_hist = _f64(k_hist), _f64(v_hist), _f64(q_hist)
    hoff = np.asarray(seq_offsets, dtype=np.int64)
    coff = np.asarray(cand_offsets, dtype=np.int64)
    ts = None if timestamps is None else np.asarray(timestamps, dtype=np.int64)
    cts = None if cand_timestamps is None else np.asarray(cand_timestamps, dtype=np.int64)
    out = np.zeros_like(v_c)
    H = q_c.shape[1]
    for b in range(hoff.size - 1):
        h0, h1 = int(hoff[b]), int(hoff[b + 1])
        for c in range(int(coff[b]), int(coff[b + 1])):
            sl = lambda hist, cand: np.concatenate([hist[h0:h1], cand[c:c + 1]], axis=0)
            t_seq = None if ts is None else np.concatenate([ts[h0:h1], cts[c:c + 1]])
            qs, ks, vs = sl(q_hist, q_c), sl(k_hist, k_c), sl(v_hist, v_c)
            # the appended row only (attn_fwd_rows evaluates attn_fwd's rows one by one)
            for hh in range(H):
                out[c, hh] = attn_fwd_rows(qs, ks, vs, np.array([0, h1 - h0 + 1]), 0, hh, [h1 - h0],
                                           alpha=alpha, divisor=divisor, pos_table=pos_table,
                                           time_table=time_table, timestamps=t_seq)[0]
    return out


# ----------------------------------------------------------------------------
# layer
# ----------------------------------------------------------------------------
def layer_norm(x, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm over the last axis: (x - mean) / sqrt(biased var + eps) * gamma + beta
    (the ``nn.LayerNorm`` of the neurarch exported block)."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def layer_fwd(x, params: dict, seq_offsets, *, num_heads: int, dqk: int, dv: int,
              timestamps=None, eps: float = 1e-6, alpha: float = 1.0,
              divisor: float = 0.0):
    """One HSTU layer, float64.

    Steps (daiwk reproduction notes, flowchart and core formula; briansu.co
    explainer, section 3):

      1. G = SiLU(LN(X; g1, b1) W_uvqk^T + b_uvqk), split along features as
         u | v | q | k (the split order of the neurarch exported block), each
         viewed per head as [T, H, d]. SiLU goes on all four projections.
      2. O = attn_fwd(q, k, v) with this layer's bias tables.
      3. Y = LN(O; g2, b2) * u, the norm taken over all H*dv features of a
         token (post-pooling normalisation, then the U gate).
      4. X' = X + Y W_out^T + b_out (output projection with residual; no norm
         after the residual).

    Weights use the nn.Linear layout: W_uvqk [H(2dv+2dqk), D], W_out [D, H dv].
    Returns (X', dict of the intermediates uvqk, o, y).
    """
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    H = num_heads
    xn = layer_norm(x, params["ln_in_gamma"], params["ln_in_beta"], eps)
    z = xn @ _f64(params["w_uvqk"]).T
    if params.get("b_uvqk") is not None:
        z = z + _f64(params["b_uvqk"])
    g = silu(z)
    u = g[:, 0:H * dv]
    vv = g[:, H * dv:2 * H * dv].reshape(T, H, dv)
    qq = g[:, 2 * H * dv:2 * H * dv + H * dqk].reshape(T, H, dqk)
    kk = g[:, 2 * H * dv + H * dqk:2 * H * dv + 2 * H * dqk].reshape(T, H, dqk)
    o = attn_fwd(qq, kk, vv, seq_offsets, alpha=alpha, divisor=divisor,
                 pos_table=params.get("pos_table"), time_table=params.get("time_table"),
                 timestamps=timestamps).reshape(T, H * dv)
    y = layer_norm(o, params["ln_out_gamma"], params["ln_out_beta"], eps) * u
    out = x + y @ _f64(params["w_out"]).T
    if params.get("b_out") is not None:
        out = out + _f64(params["b_out"])
    return out, {"uvqk": g, "o": o, "y": y}


def layer_fwd_rows(x, params: dict, seq_offsets, rows, *, num_heads: int, dqk: int, dv: int,
                   timestamps=None, eps: float = 1e-6, alpha: float = 1.0, divisor: float = 0.0):
    """Rows ``rows`` (global token indices) of ``layer_fwd``'s output, float64.

    The projection G is formed for every token (later rows attend to all
    earlier ones); the attention, post-pooling norm, gate and output projection
    are then evaluated only for the requested rows, each from the same
    definitions as ``layer_fwd``. Returns [len(rows), D].
    """
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    H = num_heads
    off = np.asarray(seq_offsets, dtype=np.int64)
    xn = layer_norm(x, params["ln_in_gamma"], params["ln_in_beta"], eps)
    z = xn @ _f64(params["w_uvqk"]).T
    if params.get("b_uvqk") is not None:
        z = z + _f64(params["b_uvqk"])
    g = silu(z)
    u = g[:, 0:H * dv]
    vv = g[:, H * dv:2 * H * dv].reshape(T, H, dv)
    qq = g[:, 2 * H * dv:2 * H * dv + H * dqk].reshape(T, H, dqk)
    kk = g[:, 2 * H * dv + H * dqk:2 * H * dv + 2 * H * dqk].reshape(T, H, dqk)
    rows = np.asarray(rows, dtype=np.int64)
    seq_of = np.searchsorted(off, rows, side="right") - 1
    out = np.zeros((rows.size, D), dtype=np.float64)
    for b in np.unique(seq_of):
        sel = np.flatnonzero(seq_of == b)
        pos = rows[sel] - off[b]
        o = np.concatenate([attn_fwd_rows(qq, kk, vv, off, int(b), h, pos, alpha=alpha,
                                          divisor=divisor, pos_table=params.get("pos_table"),
                                          time_table=params.get("time_table"),
                                          timestamps=timestamps) for h in range(H)], axis=1)
        y = layer_norm(o, params["ln_out_gamma"], params["ln_out_beta"], eps) * u[rows[sel]]
        r = x[rows[sel]] + y @ _f64(params["w_out"]).T
        if params.get("b_out") is not None:
            r = r + _f64(params["b_out"])
        out[sel] = r
    return out


def layer_norm_bwd(x, gamma, d_y, eps: float):
    """Gradients of y = LN(x) * gamma + beta (over the last axis) for upstream
    d_y, float64: with xhat = (x - mean) / sqrt(var + eps), g = d_y * gamma,
        dx = (g - mean(g) - xhat * mean(g * xhat)) / sqrt(var + eps)
    (mean over the normalised axis), d_gamma = sum over rows of d_y * xhat,
    d_beta = sum over rows of d_y. Returns (dx, d_gamma, d_beta)."""
    x = np.asarray(x, dtype=np.float64)
    d_y = np.asarray(d_y, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xhat = (x - mu) * rstd
    g = d_y * _f64(gamma)
    dx = (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True)) * rstd
    return dx, (d_y * xhat).sum(axis=0), d_y.sum(axis=0)


def layer_bwd(x, params: dict, seq_offsets, d_out, *, num_heads: int, dqk: int, dv: int,
              timestamps=None, eps: float = 1e-6, alpha: float = 1.0, divisor: float = 0.0):
    """Gradients of sum(X' * d_out) for ``layer_fwd``, float64, by the chain
    rule through its four steps in reverse (the layer of the daiwk
    reproduction notes' flowchart and core formula, trained at every position
    as their core formula describes):

      4. X' = X + Y W_out^T + b_out:  d_b_out = sum_t d_out,
         d_W_out = d_out^T Y,  dY = d_out W_out,  and d_out reaches X directly.
      3. Y = LN(O; g2, b2) * u:  du = dY * LN(O),  then ``layer_norm_bwd`` of
         O with upstream dY * u gives dO, d_g2, d_b2.
      2. O = attention(q, k, v):  ``attn_bwd`` gives dq, dk, dv and the bias
         tables' gradients.
      1. G = SiLU(Z), Z = LN(X; g1, b1) W_uvqk^T + b_uvqk:  dG = [du|dv|dq|dk]
         (the split order), dZ = dG * SiLU'(Z) with SiLU'(z) = sig(z) (1 +
         z (1 - sig(z))),  d_b_uvqk = sum_t dZ,  d_W_uvqk = dZ^T LN(X),
         d LN(X) = dZ W_uvqk, then ``layer_norm_bwd`` of X.

    Returns (dX, dict of parameter gradients with the keys of ``params``
    prefixed "d_"; a table absent from ``params`` has no gradient entry).
    """
    x = np.asarray(x, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    T, D = x.shape
    H = num_heads
    w_uvqk, w_out = _f64(params["w_uvqk"]), _f64(params["w_out"])
    # forward, keeping what the backward reads
    xn = layer_norm(x, params["ln_in_gamma"], params["ln_in_beta"], eps)
    z = xn @ w_uvqk.T
    if params.get("b_uvqk") is not None:
        z = z + _f64(params["b_uvqk"])
    g = silu(z)
    c_v, c_q, c_k = H * dv, 2 * H * dv, 2 * H * dv + H * dqk
    u = g[:, 0:c_v]
    vv = g[:, c_v:c_q].reshape(T, H, dv)
    qq = g[:, c_q:c_k].reshape(T, H, dqk)
    kk = g[:, c_k:c_k + H * dqk].reshape(T, H, dqk)
    attn_kw = dict(alpha=alpha, divisor=divisor, pos_table=params.get("pos_table"),
                   time_table=params.get("time_table"), timestamps=timestamps)
    o = attn_fwd(qq, kk, vv, seq_offsets, **attn_kw).reshape(T, H * dv)
    on = layer_norm(o, params["ln_out_gamma"], params["ln_out_beta"], eps)
    y = on * u
    grads = {}
    # 4. output projection and residual
    grads["d_b_out"] = d_out.sum(axis=0)
    grads["d_w_out"] = d_out.T @ y
    d_y = d_out @ w_out
    # 3. post-pooling norm and U gate
    d_u = d_y * on
    d_o, grads["d_ln_out_gamma"], grads["d_ln_out_beta"] = layer_norm_bwd(
        o, params["ln_out_gamma"], d_y * u, eps)
    # 2. attention
    dq, dk, dvv, dP, dTt = attn_bwd(qq, kk, vv, d_o.reshape(T, H, dv), seq_offsets, **attn_kw)
    if params.get("pos_table") is not None:
        grads["d_pos_table"] = dP
    if params.get("time_table") is not None:
        grads["d_time_table"] = dTt
    # 1. projection with SiLU, input norm
    d_g = np.concatenate([d_u, dvv.reshape(T, H * dv), dq.reshape(T, H * dqk),
                          dk.reshape(T, H * dqk)], axis=1)
    sig = sigmoid(z)
    d_z = d_g * sig * (1.0 + z * (1.0 - sig))
    grads["d_b_uvqk"] = d_z.sum(axis=0)
    grads["d_w_uvqk"] = d_z.T @ xn
    d_x_ln, grads["d_ln_in_gamma"], grads["d_ln_in_beta"] = layer_norm_bwd(
        x, params["ln_in_gamma"], d_z @ w_uvqk, eps)
    return d_out + d_x_ln, grads


def stack_fwd(x, layers, seq_offsets, *, num_heads: int, dqk: int, dv: int,
              timestamps=None, eps: float = 1e-6):
    """A stack of HSTU layers applied in order (the neurarch model card lists
    four blocks between the embedding and the final norm). Returns the last
    layer's output, float64."""
    h = np.asarray(x, dtype=np.float64)
    for p in layers:
        h, _ = layer_fwd(h, p, seq_offsets, num_heads=num_heads, dqk=dqk, dv=dv,
                         timestamps=timestamps, eps=eps)
    return h


# ----------------------------------------------------------------------------
# final norm and retrieval head
# ----------------------------------------------------------------------------
def rms_norm(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis, float64: x / sqrt(mean(x^2) + eps) * gamma.

    The norm between the last HSTU block and the head in the neurarch model
    card (structure table row "RMSNorm", 512 features; the exported code
    builds ``nn.RMSNorm(512)``; the neurarch graph JSON's "norm" node gives
    eps 1e-6). Unlike
    LayerNorm no mean is subtracted and there is no shift. gamma None means
    ones (the initial value)."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * _f64(gamma)


def head_fwd(x, table, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """Catalogue logits of the retrieval head, float64:
        logits[t, i] = sum_d RMSNorm(x)[t, d] * table[i, d].

    The neurarch model card's head maps 512 features to 200000 item logits
    with a bias-free linear map (structure table row "Retrieval Head";
    exported code ``nn.Linear(512, 200000, bias=False)``), and the neurarch
    graph JSON's "head" node marks its weights as tied, read here as: the [vocab, D] weight is
    the token-embedding table itself. A subset of items is scored by passing
    those rows of the table."""
    return rms_norm(x, gamma, eps) @ _f64(table).T


# ----------------------------------------------------------------------------
# Stochastic Length
# ----------------------------------------------------------------------------
def stochastic_length(seq_offsets, keys, max_len: int):
    """Random shortening of long histories (Stochastic Length, named in the
    briansu.co explainer, section 6 "Why it works", as what makes training
    cheap; the pages give no procedure, the reading here): a sequence of n <= max_len
    tokens is kept whole; a longer one keeps a uniformly random subset of
    max_len tokens in their original order. The randomness is passed in: one
    32-bit key per token, and a sequence keeps the max_len tokens whose
    (key, position in the sequence) pairs are smallest -- with independent
    uniform keys, every max_len-subset is equally likely.

    Returns (new_offsets int64 [B+1], gather_index int64 [T']): output token
    r of the shortened batch is input token gather_index[r]."""
    off = np.asarray(seq_offsets, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.uint32)
    if max_len < 0:
        raise ValueError("max_len must be >= 0")
    new_off = [0]
    picked = []
    for b in range(off.size - 1):
        s, e = int(off[b]), int(off[b + 1])
        n = e - s
        if n <= max_len:
            keep = np.arange(n, dtype=np.int64)
        else:
            order = np.lexsort((np.arange(n), keys[s:e]))     # by key, then by position
            keep = np.sort(order[:max_len]).astype(np.int64)
        picked.append(s + keep)
        new_off.append(new_off[-1] + keep.size)
    idx = np.concatenate(picked) if picked else np.zeros(0, np.int64)
    return np.asarray(new_off, np.int64), idx.astype(np.int64)
