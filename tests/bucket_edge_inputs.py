"""Seeded inputs that make every relative-bias bucket decision visible in the
output (test infrastructure; random draws and constructions only).

With q = k = 0 the score of a pair is its bias alone, and with one-hot values
(v_j = e_j, at most 128 tokens per sequence, d = 128) every output element is
one pair's SiLU(P[pos] + Tt[time]) / N. The timestamps put many pairs exactly
on bucket edges -- time gaps of 2^k - 1 (first gap of bucket k) and 2^k - 2
(last gap of bucket k - 1) -- in narrow (< 2^31) and wide (> 2^31) ranges,
with query and key blocks arranged so that a 32 x 32 block of pairs can have
one time bucket, two adjacent time buckets, or many; some sequences run
backwards in time (negative gaps, bucket 0). The tables have well-separated
neighbouring entries, so a pair placed one bucket off changes its output by
far more than the tolerance.
"""

from __future__ import annotations

import numpy as np

from workloads.generators import offsets_from_lengths

T0 = 1_700_000_000
D = 128                      # head dim = one-hot width: sequences hold at most 128 tokens
H = 2
DIVISOR = 128.0              # one fixed divisor, so that every sequence's pairs weigh alike


def _edge_steps(rng, count, klo, khi):
    """Increments 2^k - 1, 2^k - 2 or 2^k with k uniform in [klo, khi]."""
    k = rng.integers(klo, khi + 1, size=count)
    sub = rng.integers(0, 3, size=count)          # 1, 2 or 0 below the power of two
    return (np.left_shift(np.int64(1), k.astype(np.int64)) - np.where(sub == 2, 0, sub + 1)).astype(np.int64)


def _two_bucket_block_times(K):
    """128 tokens whose 32 x 32 blocks below the diagonal span exactly two time
    buckets around the edge 2^K - 1 (and 2^(K+1) - 1), with pairs on both
    sides of each edge: keys 0..31 at t0 + j, keys 32..63 at t0 + 2^K + j,
    rows 64..95 at t0 + 2^K - 17 + (i - 64), rows 96..127 at t0 + 2^(K+1) - 17
    + (i - 96)."""
    i = np.arange(128, dtype=np.int64)
    t = np.empty(128, np.int64)
    t[:32] = T0 + i[:32]
    t[32:64] = T0 + (1 << K) + (i[32:64] - 32)
    t[64:96] = T0 + (1 << K) - 17 + (i[64:96] - 64)
    t[96:] = T0 + (1 << (K + 1)) - 17 + (i[96:] - 96)
    return t


def edge_batch(seed: int = 0):
    """Lengths and int64 timestamps of the edge batch (several sequences of
    at most 128 tokens, each built to exercise one family of edges)."""
    rng = np.random.default_rng(seed)
    seqs = []
    seqs.append(T0 + np.concatenate([[0], np.cumsum(_edge_steps(rng, 127, 0, 12))]))       # narrow edges
    seqs.append(T0 + np.concatenate([[0], np.cumsum(_edge_steps(rng, 127, 28, 40))]))      # wide edges
    seqs.append(_two_bucket_block_times(10))                                              # two buckets, narrow
    seqs.append(_two_bucket_block_times(33))                                              # two buckets, wide
    seqs.append(np.concatenate([np.full(64, T0), T0 + (1 << 20) + np.arange(64)]))        # one bucket per block
    seqs.append(T0 - np.concatenate([[0], np.cumsum(_edge_steps(rng, 99, 0, 20))]))        # backwards in time
    mixed = T0 + rng.permutation(np.concatenate([[0], np.cumsum(_edge_steps(rng, 76, 0, 34))]))
    seqs.append(mixed)                                                                    # unsorted
    seqs.append(T0 + np.array([0, (1 << 31) - 1, (1 << 31) - 2 + (1 << 31) - 1], np.int64))  # 3 tokens at 2^31 edges
    seqs.append(np.array([T0], np.int64))                                                 # one token
    lengths = np.array([len(s) for s in seqs], np.int64)
    assert lengths.max() <= D
    return lengths, np.concatenate(seqs).astype(np.int64)


def tables(Bp: int, Bt: int, scale: float = 1.0):
    """Position and time tables with well-separated neighbours: Tt cycles
    through 0.25, 0.75, 1.25 and P through -0.3, 0, 0.3 (head 1 in another
    phase), times `scale`. With scale 1 every bias lies in [-0.05, 1.55]
    (the kernels' polynomial SiLU range); with scale 3 beyond it."""
    p = np.array([[0.3 * (((b + h) % 3) - 1) for b in range(Bp)] for h in range(H)], np.float32)
    t = np.array([[0.25 + 0.5 * ((c + 2 * h) % 3) for c in range(Bt)] for h in range(H)], np.float32)
    return (scale * p).astype(np.float32), (scale * t).astype(np.float32)


def one_hot(lengths, column_of=None):
    """[T, H, D] with token j of every sequence set to e_j (or e_column_of(b, j))."""
    off = offsets_from_lengths(lengths)
    x = np.zeros((int(off[-1]), H, D), np.float32)
    for b in range(len(lengths)):
        for j in range(int(lengths[b])):
            c = j if column_of is None else column_of(b, j)
            x[off[b] + j, :, c] = 1.0
    return x


def pair_bias_forms(lengths, ts, pt, tt, time_bucket, pos_bucket):
    """For every causal pair of the batch: (b, i, j, h, bias), with the bucket
    functions passed in (so that a test can pass deliberately slipped ones)."""
    off = offsets_from_lengths(lengths)
    rows = []
    for b in range(len(lengths)):
        n = int(lengths[b])
        for i in range(n):
            j = np.arange(i + 1)
            dt = ts[off[b] + i] - ts[off[b] + j]
            pb = pos_bucket(i - j, pt.shape[1])
            tb = time_bucket(dt, tt.shape[1])
            for h in range(H):
                rows.append((b, i, j, h, pt[h][pb].astype(np.float64) + tt[h][tb].astype(np.float64)))
    return rows


# (Bp, Bt, table scale) of the runs: the clamp of the position bucket inside
# the first off-diagonal block (Bp 3) or in the middle of it (Bp 40); every
# reachable time bucket its own entry (Bt 64) or the clamp at 19 (Bt 20); the
# polynomial SiLU range (scale 1) and beyond it (scale 3).
CONFIGS = [(3, 64, 1.0), (40, 20, 1.0), (3, 64, 3.0), (40, 64, 3.0)]


def cand_edge_batch(seed: int = 1):
    """Histories (at most 127 tokens, so that v_c = e_127 does not collide with
    a history column) and candidates whose timestamps sit on bucket edges
    relative to history tokens: per sequence the history lengths, the history
    timestamps, the candidate counts and the candidate timestamps."""
    rng = np.random.default_rng(seed)
    lengths, ts = edge_batch(seed)
    off = offsets_from_lengths(lengths)
    hist = [ts[off[b]:off[b + 1]][:127] for b in range(len(lengths))]
    hist.append(np.zeros(0, np.int64))                      # an empty history
    cands = []
    for b, t in enumerate(hist):
        m = 40 if b % 3 else 7
        if t.size == 0:
            cands.append(np.full(m, T0, np.int64))
        elif b == 4:                                        # every candidate at one far time
            cands.append(np.full(m, t.max() + (1 << 40), np.int64))
        else:
            j = rng.integers(0, t.size, size=m)
            k = rng.integers(0, 36, size=m)
            sub = rng.integers(1, 3, size=m)
            cands.append((t[j] + np.left_shift(np.int64(1), k.astype(np.int64)) - sub).astype(np.int64))
    hl = np.array([t.size for t in hist], np.int64)
    cm = np.array([c.size for c in cands], np.int64)
    return hl, np.concatenate(hist).astype(np.int64), cm, np.concatenate(cands).astype(np.int64)
