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
