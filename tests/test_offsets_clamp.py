"""Host test of the offsets clamp that every attention kernel reads through
(csrc/offsets.h): the caller's seq_offsets are copied on the device into
c(b) = min(max(off[b], c(b-1)), T), c(-1) = 0, so that a malformed array
(offsets past T, negative or decreasing) cannot move a read or a write out of
bounds. The header's __host__ __device__ helper is compiled with g++ and
driven in both of its forms: the sequential recurrence, and the chunked
prefix maximum the work-list builder and the candidate chunk scan use
(inclusive maximum inside a chunk of threads, running maximum of the earlier
chunks as the floor)."""

import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hstu_pointwise_attention_causal_amd", "csrc")

_SRC = r"""
#include <stdint.h>
#include "offsets.h"
extern "C" void clamp_recurrence(const int64_t* in, int n, int64_t T, int64_t* out) {
  int64_t prev = 0;
  for (int b = 0; b < n; ++b) prev = out[b] = hstu::clamp_offset(in[b], prev, T);
}
extern "C" void clamp_chunked(const int64_t* in, int n, int64_t T, int64_t* out, int chunk) {
  int64_t run = 0;
  for (int c0 = 0; c0 < n; c0 += chunk) {
    int64_t m = INT64_MIN, chunk_max = INT64_MIN;
    for (int b = c0; b < n && b < c0 + chunk; ++b) chunk_max = in[b] > chunk_max ? in[b] : chunk_max;
    for (int b = c0; b < n && b < c0 + chunk; ++b) {
      m = in[b] > m ? in[b] : m;                 // inclusive maximum inside the chunk
      out[b] = hstu::clamp_offset(m, run, T);
    }
    run = chunk_max > run ? chunk_max : run;
  }
}
"""


@pytest.fixture(scope="module")
def lib():
    d = tempfile.mkdtemp(prefix="hstu_offsets_")
    src, so = os.path.join(d, "o.cpp"), os.path.join(d, "o.so")
    with open(src, "w") as f:
        f.write(_SRC)
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", f"-I{CSRC}", src, "-o", so], check=True)
    L = ctypes.CDLL(so)
    P = ctypes.POINTER(ctypes.c_int64)
    L.clamp_recurrence.argtypes = [P, ctypes.c_int, ctypes.c_int64, P]
    L.clamp_chunked.argtypes = [P, ctypes.c_int, ctypes.c_int64, P, ctypes.c_int]
    return L


def _run(lib, off, T, chunk=None):
    off = np.ascontiguousarray(off, dtype=np.int64)
    out = np.empty_like(off)
    P = ctypes.POINTER(ctypes.c_int64)
    if chunk is None:
        lib.clamp_recurrence(off.ctypes.data_as(P), off.size, T, out.ctypes.data_as(P))
    else:
        lib.clamp_chunked(off.ctypes.data_as(P), off.size, T, out.ctypes.data_as(P), chunk)
    return out


def _expected(off, T):
    """The documented result: prefix maximum (from 0) of the offsets, capped at T."""
    return np.minimum(np.maximum.accumulate(np.maximum(np.asarray(off, np.int64), 0)), T)


@pytest.mark.parametrize("off,T,want", [
    ([0, 3, 7, 10], 10, [0, 3, 7, 10]),            # well formed: unchanged
    ([0, 3, 7, 12], 10, [0, 3, 7, 10]),            # last offset past T
    ([0, 8, 4, 10], 10, [0, 8, 8, 10]),            # decreasing step: empty sequence
    ([-5, 2, -1, 3], 10, [0, 2, 2, 3]),            # negative offsets
    ([5, 6, 7], 4, [4, 4, 4]),                     # everything past T
    ([0, 2 ** 62, 1, 2 ** 63 - 1], 100, [0, 100, 100, 100]),
    ([0], 0, [0]),
    ([-(2 ** 63), 0], 0, [0, 0]),
])
def test_clamp_cases(lib, off, T, want):
    assert _run(lib, off, T).tolist() == want
    for chunk in (1, 2, 3, 1024):
        assert _run(lib, off, T, chunk).tolist() == want


def test_clamp_random_against_definition(lib):
    rng = np.random.default_rng(7)
    for trial in range(300):
        n = int(rng.integers(1, 3000))
        T = int(rng.integers(0, 5000))
        off = rng.integers(-100, 6000, size=n)
        if trial % 3 == 0:   # mostly well formed with a few bad entries
            off = np.sort(rng.integers(0, T + 1, size=n))
            bad = rng.integers(0, n, size=3)
            off[bad] = rng.integers(-50, 2 * T + 50, size=3)
        want = _expected(off, T)
        assert np.array_equal(_run(lib, off, T), want)
        assert np.array_equal(_run(lib, off, T, 1024), want)
        assert np.array_equal(_run(lib, off, T, int(rng.integers(1, 70))), want)
        lengths = np.diff(want)
        assert np.all(lengths >= 0) and lengths.sum() <= T and want.min() >= 0 and want.max() <= T
