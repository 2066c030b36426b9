"""Seeded input recipes for the five HSTU workloads and their reduced variants.

Every array is drawn from ``numpy.random.default_rng(seed)`` in a fixed order,
so the same name and seed always give the same bytes. Floating-point inputs
are drawn in float32; for the bfloat16 workloads they are rounded to the
nearest bfloat16 (ties to even) and kept as float32 arrays holding exactly
representable values, so the oracle (which widens them to float64) and the
GPU path (which narrows them to bfloat16 without further rounding) see the
same numbers.

Shapes follow the pages' workloads: 1024-token interleaved histories with a
512-wide embedding over a 200000-item vocabulary and four 4-head blocks of
width 128 (neurarch "HSTU (Generative Recommender)" model card, Structure
table and exported ``HSTUBlock``), 8k-long sequences (briansu.co HSTU
explainer, section 3), and timestamped actions (the same explainer, section 1;
kongchang HSTU knowledge page). No public dataset is read: all values are
synthetic stand-ins with those shapes and the distributions listed below.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

VOCAB = 200000
T0_SECONDS = 1_700_000_000  # first timestamp of every sequence (int64 seconds)


# ----------------------------------------------------------------------------
# bfloat16 conversion of inputs (input preparation, not method arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array of the nearest bfloat16 values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# elementary recipes
# ----------------------------------------------------------------------------
def log_uniform_lengths(rng: np.random.Generator, count: int, lo: int, hi: int) -> np.ndarray:
    """n = clip(floor(exp(U(ln lo, ln hi))), lo, hi), int64."""
    u = rng.uniform(np.log(lo), np.log(hi), size=count)
    return np.clip(np.floor(np.exp(u)).astype(np.int64), lo, hi)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def exponential_timestamps(rng: np.random.Generator, lengths, mean_s: float = 3600.0,
                           t0: int = T0_SECONDS) -> np.ndarray:
    """Per sequence: t = t0 + floor(cumsum(increments)), increments ~ Exp(mean_s).

    The first token of each sequence sits at t0 (its increment is not drawn),
    so timestamps are int64 seconds, non-decreasing inside each sequence.
    """
    out = []
    for n in np.asarray(lengths, dtype=np.int64):
        n = int(n)
        if n == 0:
            continue
        inc = rng.exponential(mean_s, size=n - 1)
        t = np.empty(n, dtype=np.int64)
        t[0] = t0
        t[1:] = t0 + np.floor(np.cumsum(inc)).astype(np.int64)
        out.append(t)
    if not out:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(out)


def embedding_rows(ids: np.ndarray, dim: int = 512, std: float = 0.02) -> np.ndarray:
    """Rows of a virtual [VOCAB, dim] N(0, std) table; row ``i`` comes from
    ``default_rng([1, i])`` so the 200000x512 table is never materialised."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    rows = np.empty((ids.size, dim), dtype=np.float32)
    cache: Dict[int, np.ndarray] = {}
    for t, i in enumerate(ids):
        i = int(i)
        r = cache.get(i)
        if r is None:
            r = (std * np.random.default_rng([1, i]).standard_normal(dim)).astype(np.float32)
            cache[i] = r
        rows[t] = r
    return rows


def xavier_uniform(rng: np.random.Generator, out_features: int, in_features: int) -> np.ndarray:
    """[out, in] (nn.Linear layout) ~ U(-a, a), a = sqrt(6 / (fan_in + fan_out))."""
    a = np.sqrt(6.0 / (in_features + out_features))
    return rng.uniform(-a, a, size=(out_features, in_features)).astype(np.float32)


def normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (std * rng.standard_normal(size=shape)).astype(np.float32)


# ----------------------------------------------------------------------------
# workload container
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    kind: str                   # "attn" | "attn_bwd" | "layer" | "stack"
    dtype: str                  # "f32" | "bf16"
    num_heads: int
    dqk: int
    dv: int
    seq_offsets: np.ndarray     # int64 [B+1]
    timestamps: Optional[np.ndarray] = None   # int64 [T] or None
    pos_table: Optional[np.ndarray] = None    # float32 [H, Bp] (attention workloads)
    time_table: Optional[np.ndarray] = None   # float32 [H, Bt] (attention workloads)
    q: Optional[np.ndarray] = None            # float32 [T, H, dqk]
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None            # float32 [T, H, dv]
    d_o: Optional[np.ndarray] = None          # float32 [T, H, dv] (backward)
    x: Optional[np.ndarray] = None            # float32 [T, D] (layer / stack)
    embed_dim: int = 0
    layers: List[dict] = dataclasses.field(default_factory=list)
    alpha: float = 1.0
    divisor: float = 0.0        # <= 0: per-sequence length n; > 0: fixed constant
    ln_eps: float = 1e-6
    note: str = ""
    cand: Optional[dict] = None               # candidate scoring: offsets, q, k, v, timestamps
    head: Optional[dict] = None               # retrieval head: table [V, D], gamma [D] or None, eps
    sl: Optional[dict] = None                 # Stochastic Length: keys uint32 [T], max_len

    @property
    def num_seqs(self) -> int:
        return int(self.seq_offsets.size - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.seq_offsets[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.seq_offsets)

    @property
    def max_seq_len(self) -> int:
        return int(self.lengths.max()) if self.num_seqs else 0

    def causal_pairs(self) -> int:
        n = self.lengths.astype(np.int64)
        return int((n * (n + 1) // 2).sum())

    def attn_fwd_flops(self) -> float:
        """Causal-effective forward flops: sum_b H n_b(n_b+1)/2 * 2(dqk+dv)."""
        return float(self.causal_pairs()) * self.num_heads * 2.0 * (self.dqk + self.dv)

    def attn_bwd_flops(self) -> float:
        """Causal-effective backward flops: sum_b H n_b(n_b+1)/2 * (6 dqk + 4 dv)."""
        return float(self.causal_pairs()) * self.num_heads * (6.0 * self.dqk + 4.0 * self.dv)

    def layer_gemm_flops(self) -> float:
        T, D, H = self.total_tokens, self.embed_dim, self.num_heads
        return 2.0 * T * D * H * (2 * self.dv + 2 * self.dqk) + 2.0 * T * H * self.dv * D


def _maybe_bf16(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    if a is None or dtype != "bf16":
        return a
    return round_to_bf16(a)


# ----------------------------------------------------------------------------
# recipes (draw order is part of the definition)
# ----------------------------------------------------------------------------
def _attn_recipe(name, seed, lengths, H, d, *, dtype="bf16", qkv_std=None, time=True,
                 pos=True, Bp=128, Bt=128, table_std=0.02, backward=False,
                 divisor=0.0, draw_lengths=None, note=""):
    """Attention-only inputs.

    Draw order: [lengths], q, k, v, [dO], [timestamps], [pos table], [time table].
    """
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        lo, hi, count = draw_lengths
        lengths = log_uniform_lengths(rng, count, lo, hi)
    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    std = (1.0 / np.sqrt(d)) if qkv_std is None else qkv_std
    q = normal(rng, (T, H, d), std)
    k = normal(rng, (T, H, d), std)
    v = normal(rng, (T, H, d), std)
    d_o = normal(rng, (T, H, d), 1.0) if backward else None
    ts = exponential_timestamps(rng, lengths) if time else None
    pt = normal(rng, (H, Bp), table_std) if pos else None
    tt = normal(rng, (H, Bt), table_std) if time else None
    return Workload(
        name=name, kind="attn_bwd" if backward else "attn", dtype=dtype,
        num_heads=H, dqk=d, dv=d, seq_offsets=off, timestamps=ts,
        pos_table=pt, time_table=tt,
        q=_maybe_bf16(q, dtype), k=_maybe_bf16(k, dtype), v=_maybe_bf16(v, dtype),
        d_o=_maybe_bf16(d_o, dtype), divisor=divisor, note=note)


def _layer_params(rng, D, H, dqk, dv, Bp, Bt, time):
    """One layer: W_uvqk [H(2dv+2dqk), D], W_out [D, H dv] (Xavier-U, bf16),
    position table [H, Bp] ~ 0.02 N, [time table [H, Bt] ~ 0.02 N];
    linear biases 0, LayerNorm gamma 1 / beta 0 (configs give weights only)."""
    n_uvqk = H * (2 * dv + 2 * dqk)
    w_uvqk = round_to_bf16(xavier_uniform(rng, n_uvqk, D))
    w_out = round_to_bf16(xavier_uniform(rng, D, H * dv))
    pt = normal(rng, (H, Bp), 0.02)
    tt = normal(rng, (H, Bt), 0.02) if time else None
    return dict(
        w_uvqk=w_uvqk, b_uvqk=np.zeros(n_uvqk, np.float32),
        w_out=w_out, b_out=np.zeros(D, np.float32),
        ln_in_gamma=np.ones(D, np.float32), ln_in_beta=np.zeros(D, np.float32),
        ln_out_gamma=np.ones(H * dv, np.float32), ln_out_beta=np.zeros(H * dv, np.float32),
        pos_table=pt, time_table=tt)


def _layer_recipe(name, seed, *, lengths=None, draw_lengths=None, num_layers=1, D=512,
                  H=4, d=128, Bp=128, Bt=128, time=False, backward=False, note=""):
    """Layer / stack inputs.

    Draw order: [lengths], token ids U[0, VOCAB), [timestamps], then per layer
    W_uvqk, W_out, position table, [time table], then [dOut ~ N(0, 1) [T, D]
    for a backward]. X = embedding rows of the ids.
    """
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        lo, hi, count = draw_lengths
        lengths = log_uniform_lengths(rng, count, lo, hi)
    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    ids = rng.integers(0, VOCAB, size=T)
    ts = exponential_timestamps(rng, lengths) if time else None
    layers = [_layer_params(rng, D, H, d, d, Bp, Bt, time) for _ in range(num_layers)]
    d_out = round_to_bf16(normal(rng, (T, D), 1.0)) if backward else None
    x = round_to_bf16(embedding_rows(ids, D))
    return Workload(
        name=name, kind="layer_bwd" if backward else ("stack" if num_layers > 1 else "layer"),
        dtype="bf16", num_heads=H, dqk=d, dv=d, seq_offsets=off, timestamps=ts, x=x, embed_dim=D,
        layers=layers, d_o=d_out, note=note)


def _cand_recipe(name, seed, *, lengths=None, draw_lengths=None, cands=1024, H=4, d=128,
                 Bp=128, Bt=128, table_std=0.02, note=""):
    """Candidate-scoring inputs: histories with cached k, v and a micro-batch
    of candidates per history.

    Draw order: [history lengths], history k, v, candidate q, k, v, history
    timestamps, candidate gaps ~ Exponential(mean 3600 s) after each history's
    last timestamp (one per sequence: the request time), position table, time
    table. q, k, v ~ N(0, 1/d) rounded to bf16. The history's q (not read by
    candidate scoring) is all zeros.
    """
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        lo, hi, count = draw_lengths
        lengths = log_uniform_lengths(rng, count, lo, hi)
    lengths = np.asarray(lengths, dtype=np.int64)
    m = np.full(lengths.size, cands, np.int64) if np.isscalar(cands) else np.asarray(cands, np.int64)
    hoff, coff = offsets_from_lengths(lengths), offsets_from_lengths(m)
    Th, Tc = int(hoff[-1]), int(coff[-1])
    std = 1.0 / np.sqrt(d)
    kh, vh = (round_to_bf16(normal(rng, (Th, H, d), std)) for _ in range(2))
    qc, kc, vc = (round_to_bf16(normal(rng, (Tc, H, d), std)) for _ in range(3))
    ts = exponential_timestamps(rng, np.maximum(lengths, 1))
    # per sequence the history's timestamps; an empty history keeps its one drawn value as a base
    base = offsets_from_lengths(np.maximum(lengths, 1))
    ts_h = np.concatenate([ts[base[b]:base[b] + lengths[b]] for b in range(lengths.size)]).astype(np.int64)
    last = np.array([ts[base[b + 1] - 1] for b in range(lengths.size)], np.int64)
    gaps = np.floor(rng.exponential(3600.0, size=lengths.size)).astype(np.int64)
    ts_c = np.repeat(last + gaps, m).astype(np.int64)
    pt = normal(rng, (H, Bp), table_std)
    tt = normal(rng, (H, Bt), table_std)
    return Workload(name=name, kind="cand", dtype="bf16", num_heads=H, dqk=d, dv=d, seq_offsets=hoff,
                    timestamps=ts_h, pos_table=pt, time_table=tt, q=np.zeros_like(kh), k=kh, v=vh,
                    note=note, cand=dict(offsets=coff, q=qc, k=kc, v=vc, timestamps=ts_c))


def _head_recipe(name, seed, *, rows, D=512, vocab=VOCAB, gamma=False, eps=1e-6, note=""):
    """Final RMSNorm + tied retrieval head inputs.

    Draw order: per-row scales log-uniform in [0.01, 10], token rows x =
    scale * N(0, 1) (the last block's output, whose scale the norm removes),
    the item table ~ N(0, 0.02) (the token-embedding table's recipe; with
    tied weights it is that table), [gamma ~ 1 + N(0, 0.1)]. x and the
    table are rounded to bf16. Without gamma the norm keeps its initial
    weight (ones).
    """
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.uniform(np.log(0.01), np.log(10.0), size=(rows, 1))).astype(np.float32)
    x = round_to_bf16(scale * rng.standard_normal((rows, D), dtype=np.float32))
    table = round_to_bf16(np.float32(0.02) * rng.standard_normal((vocab, D), dtype=np.float32))
    g = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32) if gamma else None
    return Workload(name=name, kind="head", dtype="bf16", num_heads=0, dqk=0, dv=0,
                    seq_offsets=np.array([0, rows], np.int64), x=x, embed_dim=D, ln_eps=eps,
                    note=note, head=dict(table=table, gamma=g, eps=eps))


def _sl_recipe(name, seed, *, lengths=None, draw_lengths=None, D=512, max_len=2048, ties=False, note=""):
    """Stochastic Length inputs: a jagged training batch and one random key per token.

    Draw order: [lengths], token rows x ~ N(0, 0.02) (bf16; the embedding
    table's scale), timestamps, keys ~ U[0, 2^32). With ties, the first
    sequence's keys keep only their top 4 bits (16 distinct values) and the
    last sequence's are all 0xFFFFFFFF, so selection has to break ties.
    """
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        lo, hi, count = draw_lengths
        lengths = log_uniform_lengths(rng, count, lo, hi)
    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    x = round_to_bf16(np.float32(0.02) * rng.standard_normal((T, D), dtype=np.float32))
    ts = exponential_timestamps(rng, lengths)
    keys = rng.integers(0, 1 << 32, size=T, dtype=np.uint64).astype(np.uint32)
    if ties and lengths.size:
        keys[off[0]:off[1]] >>= 28
        keys[off[-2]:off[-1]] = 0xFFFFFFFF
    return Workload(name=name, kind="sl", dtype="bf16", num_heads=0, dqk=0, dv=0, seq_offsets=off,
                    timestamps=ts, x=x, embed_dim=D, note=note, sl=dict(keys=keys, max_len=int(max_len)))


def _c0(seed=0):
    """fp32 attention, one sequence n=256, H=2, d=32, q,k,v ~ N(0,1),
    64-bucket position table ~ N(0, 0.02), no time bias."""
    rng = np.random.default_rng(seed)
    T, H, d = 256, 2, 32
    q = normal(rng, (T, H, d))
    k = normal(rng, (T, H, d))
    v = normal(rng, (T, H, d))
    pt = normal(rng, (H, 64), 0.02)
    return Workload(name="c0", kind="attn", dtype="f32", num_heads=H, dqk=d, dv=d,
                    seq_offsets=np.array([0, T], np.int64), pos_table=pt, q=q, k=k, v=v,
                    note="fp32 attention, n=256, H=2, d=32")


WORKLOADS = {
    # --- the five workloads at full size ---
    "c0": lambda seed=0: _c0(seed),
    "c1": lambda seed=1: _layer_recipe(
        "c1", seed, lengths=[1024] * 8, num_layers=4,
        note="4-layer stack, 8 x 1024 tokens, D 512, H 4, d 128"),
    "c2": lambda seed=2: _layer_recipe(
        "c2", seed, draw_lengths=(32, 4096, 64), num_layers=1, time=True,
        note="one layer, 64 sequences log-uniform in [32, 4096], pos + time bias"),
    "c3": lambda seed=3: _attn_recipe(
        "c3", seed, [8192] * 4, 8, 128, divisor=0.0,
        note="attention forward, 4 x 8192, H 8, d 128, pos + time bias"),
    "c4": lambda seed=4: _attn_recipe(
        "c4", seed, None, 4, 128, draw_lengths=(64, 2048, 32), backward=True,
        note="attention forward + backward, 32 sequences log-uniform in [64, 2048]"),
    # --- reduced variants: same recipes, sizes the oracle finishes in seconds,
    #     several tiles and a ragged tail ---
    "c1_small": lambda seed=11: _layer_recipe(
        "c1_small", seed, lengths=[200, 333], num_layers=2,
        note="2-layer stack, ragged lengths"),
    "c2_small": lambda seed=12: _layer_recipe(
        "c2_small", seed, draw_lengths=(1, 700, 9), num_layers=1, time=True,
        note="one layer, 9 ragged sequences, pos + time bias"),
    "c3_small": lambda seed=13: _attn_recipe(
        "c3_small", seed, [517, 1, 0, 300, 129], 3, 128,
        note="attention, ragged lengths incl. empty and single-token sequences"),
    "c4_small": lambda seed=14: _attn_recipe(
        "c4_small", seed, None, 2, 128, draw_lengths=(1, 400, 6), backward=True,
        note="attention fwd+bwd, 6 ragged sequences"),
    # --- one layer forward + backward (a training step's layer): the jagged
    #     fwd+bwd workload's length recipe with the jagged layer's shape ---
    "c5": lambda seed=5: _layer_recipe(
        "c5", seed, draw_lengths=(64, 2048, 32), num_layers=1, time=True, backward=True,
        note="one layer forward + backward, 32 sequences log-uniform in [64, 2048], D 512, H 4, "
             "d 128, pos + time bias"),
    # --- candidate scoring against cached histories (M-FALCON reading) ---
    "c6": lambda seed=6: _cand_recipe(
        "c6", seed, draw_lengths=(1024, 8192, 16), cands=1024, H=4, d=128,
        note="candidate scoring: 16 histories log-uniform in [1024, 8192], 1024 candidates each, "
             "H 4, d 128, pos + time bias"),
    "c6_small": lambda seed=16: _cand_recipe(
        "c6_small", seed, lengths=[300, 0, 77, 1, 140], cands=[5, 3, 0, 130, 64], H=2, d=128,
        note="candidate scoring, ragged histories incl. empty and one-token, 0 to 130 candidates"),
    # --- final RMSNorm + tied retrieval head over the stack's output rows ---
    "c7": lambda seed=7: _head_recipe(
        "c7", seed, rows=8192, D=512, vocab=VOCAB,
        note="final RMSNorm + retrieval head: 8 x 1024 token rows, D 512, 200000 items"),
    "c7_small": lambda seed=17: _head_recipe(
        "c7_small", seed, rows=300, D=512, vocab=1000, gamma=True,
        note="final RMSNorm + retrieval head, ragged against the tiles: 300 rows, 1000 items"),
    # --- Stochastic Length over a long-history training batch ---
    "c8": lambda seed=8: _sl_recipe(
        "c8", seed, draw_lengths=(64, 16384, 64), D=512, max_len=2048,
        note="Stochastic Length: 64 sequences log-uniform in [64, 16384], D 512, cap 2048"),
    "c8_small": lambda seed=18: _sl_recipe(
        "c8_small", seed, lengths=[5000, 0, 1, 300, 299, 301, 77, 2049], D=512, max_len=300, ties=True,
        note="Stochastic Length, cap 300: lengths around the cap, empty, one-token, tied keys"),
    "c5_small": lambda seed=15: _layer_recipe(
        "c5_small", seed, draw_lengths=(1, 500, 7), num_layers=1, time=True, backward=True,
        note="one layer forward + backward, 7 ragged sequences"),
}


def make_workload(name: str, seed: Optional[int] = None) -> Workload:
    fn = WORKLOADS[name]
    return fn() if seed is None else fn(seed)
