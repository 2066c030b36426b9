"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/hstu.h declares, and
reject bad arguments with the documented status before enqueuing anything.
Every call below carries at least one invalid argument, so it returns from the
host validation; fake device addresses are never dereferenced.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from hstu_pointwise_attention_causal_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from hstu_pointwise_attention_causal_amd import build
        build.build()
    return _lib


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "hstu.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(lib.EXPORTED) == declared
    cdll = lib.load()
    for name in declared:
        assert hasattr(cdll, name), name
    assert cdll.hstu_version() >= 100
    for s in range(9):
        assert cdll.hstu_status_string(s)


def _desc(lib, H=2, d=64, dtype=1):
    x = lib.AttnDesc()
    x.num_heads, x.dqk, x.dv, x.dtype, x.qk_scale, x.divisor = H, d, d, dtype, 1.0, 0.0
    return x


def _jag(lib, B=1, T=100, ts=False):
    j = lib.Jagged()
    j.num_seqs, j.total_tokens = B, T
    j.seq_offsets = 0x10000
    j.timestamps = 0x20000 if ts else None
    return j


FAKE_Q, FAKE_K, FAKE_V, FAKE_O, FAKE_W = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def _fwd(lib, desc, jag, bias=None, q=FAKE_Q, ldq=128, k=FAKE_K, ldk=128, v=FAKE_V, ldv=128,
         o=FAKE_O, ldo=128, ws=FAKE_W, wsb=0):
    c = lib.load()
    b = bias if bias is not None else lib.Bias()
    return c.hstu_attn_fwd(ctypes.byref(desc), ctypes.byref(jag), ctypes.byref(b),
                           q, ldq, k, ldk, v, ldv, o, ldo, ws, wsb, None)


def test_rejections(lib):
    c = lib.load()
    d, j = _desc(lib), _jag(lib)
    assert c.hstu_attn_fwd(None, ctypes.byref(j), None, FAKE_Q, 128, FAKE_K, 128, FAKE_V, 128,
                           FAKE_O, 128, FAKE_W, 0, None) == 1          # NULL descriptor
    assert _fwd(lib, d, j, q=None) == 1                              # NULL q
    assert _fwd(lib, _desc(lib, d=48), j) == 5                       # head dim not built
    assert _fwd(lib, _desc(lib, dtype=7), j) == 3                    # unknown dtype
    assert _fwd(lib, d, j, q=FAKE_Q + 2) == 4                        # misaligned base
    assert _fwd(lib, d, j, ldk=130) == 4                             # stride not a multiple of 8
    assert _fwd(lib, d, j, ldv=100) == 2                             # stride < H*d
    assert _fwd(lib, d, j, o=FAKE_Q + 64 * 2) == 7                   # o overlaps q
    assert _fwd(lib, d, j) == 6                                      # workspace too small
    b = lib.Bias()
    b.time_table, b.time_buckets = 0x600000, 16
    assert _fwd(lib, d, j, bias=b) == 1                              # time bias w/o timestamps
    b.time_buckets = 0
    assert _fwd(lib, d, _jag(lib, ts=True), bias=b) == 2             # zero buckets
    assert _fwd(lib, _desc(lib, H=0), j) == 2                        # no heads
    assert b"workspace" in c.hstu_last_error() or c.hstu_last_error()


def test_workspace_size_is_a_host_function(lib):
    c = lib.load()
    d = _desc(lib, H=8, d=128)
    j = _jag(lib, B=4, T=32768)
    out = ctypes.c_size_t(0)
    assert c.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), None, 0, ctypes.byref(out)) == 0
    # 4 sequences x 8192 tokens, 128-row tiles: at most 8 * (32768 + 4*127)/128 + 8 items
    assert 8 * 260 * 8 <= out.value < 1 << 20
    assert c.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), None, 0, None) == 1


FAKE_DO, FAKE_DQ, FAKE_DK, FAKE_DV = 0x700000, 0x800000, 0x900000, 0xA00000


def _bwd(lib, desc, jag, bias=None, d_o=FAKE_DO, dq=FAKE_DQ, dk=FAKE_DK, dv=FAKE_DV, dpos=None, dtime=None,
         wsb=0):
    c = lib.load()
    b = bias if bias is not None else lib.Bias()
    return c.hstu_attn_bwd(ctypes.byref(desc), ctypes.byref(jag), ctypes.byref(b),
                           FAKE_Q, 128, FAKE_K, 128, FAKE_V, 128, d_o, 128, dq, 128, dk, 128, dv, 128,
                           dpos, dtime, FAKE_W, wsb, None)


def test_backward_rejections(lib):
    d, j = _desc(lib), _jag(lib)
    assert _bwd(lib, _desc(lib, dtype=lib.HSTU_F32), j) == 5          # fp32 backward not built
    assert _bwd(lib, d, j, d_o=None) == 1                            # NULL upstream gradient
    assert _bwd(lib, d, j, dq=FAKE_Q) == 7                           # dq overlaps q
    assert _bwd(lib, d, j, dk=FAKE_DQ + 64) == 7                     # dk overlaps dq
    assert _bwd(lib, d, j) == 6                                      # workspace too small
    b = lib.Bias()
    b.pos_table, b.pos_buckets = 0x600000, 128
    assert _bwd(lib, d, j, bias=b) == 1                              # table without its gradient
    assert _bwd(lib, d, j, dpos=0xB00000) == 1                       # gradient without its table
    b.pos_buckets = 1025
    assert _bwd(lib, d, j, bias=b, dpos=0xB00000) == 5               # position table too large


def test_backward_workspace_adds_bias_partials(lib):
    c = lib.load()
    d = _desc(lib, H=4, d=128)
    j = _jag(lib, B=32, T=24321, ts=True)
    fwd, bwd, nob = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    b = lib.Bias()
    b.pos_table, b.pos_buckets, b.time_table, b.time_buckets = 0x600000, 128, 0x610000, 128
    assert c.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b), 0, ctypes.byref(fwd)) == 0
    assert c.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b), 1, ctypes.byref(bwd)) == 0
    assert c.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), None, 1, ctypes.byref(nob)) == 0
    assert nob.value == fwd.value
    # one row of 128 position + 64 time slots per (head, key tile)
    tiles = (24321 + 32 * 127) // 128
    assert bwd.value >= fwd.value + 4 * 4 * tiles * (128 + 64)


FAKE_X, FAKE_TABLE, FAKE_LOGITS, FAKE_HWS = 0x1000000, 0x2000000, 0x10000000, 0x3000000


def _head(lib, rows=300, dim=512, vocab=1000, eps=1e-6, x=FAKE_X, ldx=512, gamma=None, table=FAKE_TABLE,
          ldt=512, logits=FAKE_LOGITS, ldl=1000, ws=FAKE_HWS, wsb=0):
    return lib.load().hstu_head_fwd(rows, dim, vocab, eps, x, ldx, gamma, table, ldt, logits, ldl, ws, wsb, None)


def test_head_rejections(lib):
    assert _head(lib, dim=256) == 5                                  # width not built
    assert _head(lib, vocab=1004, ldl=1008) == 5                              # vocab not a multiple of 8
    assert _head(lib, x=None) == 1                                   # NULL x
    assert _head(lib, ldx=500) == 2                                  # stride below the width
    assert _head(lib, ldl=999) == 2                                  # logits stride below vocab
    assert _head(lib, eps=-1.0) == 2                                 # negative eps
    assert _head(lib, table=FAKE_TABLE + 8) == 4                     # misaligned table
    assert _head(lib, ldt=520 + 4) == 4                              # stride not a multiple of 8
    assert _head(lib, logits=FAKE_X + 1024) == 7                     # logits overlap x
    assert _head(lib) == 6                                           # workspace too small
    need = ctypes.c_size_t(0)
    assert lib.load().hstu_head_workspace_size(300, 512, ctypes.byref(need)) == 0
    assert need.value == 300 * 512 * 2
    assert _head(lib, ws=FAKE_LOGITS + 64, wsb=need.value) == 7      # workspace overlaps logits
    assert _head(lib, rows=0) == 0 and _head(lib, vocab=0) == 0      # nothing to do, nothing launched


def test_stochastic_length_and_gather_rejections(lib):
    c = lib.load()
    OFF, KEYS, NOFF, IDX = 0x100000, 0x200000, 0x300000, 0x400000
    sl = c.hstu_stochastic_length
    assert sl(-1, OFF, 10, 4, KEYS, NOFF, IDX, None) == 2            # negative num_seqs
    assert sl(2, OFF, 10, -1, KEYS, NOFF, IDX, None) == 2            # negative cap
    assert sl(2, OFF, 1 << 31, 4, KEYS, NOFF, IDX, None) == 5        # too many tokens
    assert sl(2, None, 10, 4, KEYS, NOFF, IDX, None) == 1            # NULL offsets
    assert sl(2, OFF, 10, 4, KEYS, None, IDX, None) == 1             # NULL new_offsets
    assert sl(2, OFF, 10, 4, KEYS + 2, NOFF, IDX, None) == 4         # misaligned keys
    assert sl(2, OFF, 10, 4, KEYS, NOFF, IDX + 4, None) == 4         # misaligned index
    assert sl(2, OFF, 10, 4, KEYS, OFF + 8, IDX, None) == 7          # new_offsets overlaps offsets
    assert sl(2, OFF, 10, 4, KEYS, NOFF, NOFF + 8, None) == 7        # the two outputs overlap
    g = c.hstu_gather_rows
    SRC, DST, CNT = 0x500000, 0x600000, 0x700000
    assert g(IDX, CNT, -1, SRC, 10, 1024, DST, 1024, 1024, None) == 2  # negative rows
    assert g(None, CNT, 4, SRC, 10, 1024, DST, 1024, 1024, None) == 1  # NULL index
    assert g(IDX, CNT, 4, SRC, 10, 512, DST, 1024, 1024, None) == 2    # stride below row bytes
    assert g(IDX, CNT, 4, SRC + 2, 10, 1024, DST, 1024, 1024, None) == 4  # misaligned src
    assert g(IDX, CNT, 4, SRC, 10, 1024, SRC + 4096, 1024, 1024, None) == 7  # dst overlaps src
    assert g(IDX, CNT, 0, SRC, 10, 1024, DST, 1024, 1024, None) == 0   # nothing to copy


def test_candidate_workspace_is_checked(lib):
    c = lib.load()
    d = _desc(lib, H=4, d=128)
    hist = _jag(lib, B=2, T=5000)
    cand = _jag(lib, B=2, T=300)
    cand.seq_offsets = 0x30000
    need = ctypes.c_size_t(0)
    assert c.hstu_attn_cand_workspace_size(ctypes.byref(d), ctypes.byref(hist), 200, ctypes.byref(need)) == 0
    # chunks: ceil(5000 / 2048) + 2 sequences = 5; 5 x 200 candidates x 4 heads x 128 x 4 bytes + offsets
    assert need.value >= 5 * 200 * 4 * 128 * 4
    b = lib.Bias()
    G = 1 << 28   # fake device buffers 256 MB apart, never dereferenced
    o = 6 * G
    args = (ctypes.byref(d), ctypes.byref(hist), ctypes.byref(cand), 200, ctypes.byref(b),
            1 * G, 512, 2 * G, 512, 3 * G, 512, 4 * G, 512, 5 * G, 512, o, 512)
    assert c.hstu_attn_fwd_candidates(*args, 7 * G, need.value - 1, None) == 6      # workspace too small
    assert c.hstu_attn_fwd_candidates(*args, 7 * G + 8, need.value, None) == 4      # misaligned workspace
    assert c.hstu_attn_fwd_candidates(*args, o, need.value, None) == 7              # workspace overlaps o
