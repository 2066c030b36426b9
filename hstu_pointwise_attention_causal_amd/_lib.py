"""ctypes mirror of include/hstu.h and the loader of libhstu.so.

Argument marshalling only: no arithmetic of the method happens here. The
library must have been built (``python -m hstu_pointwise_attention_causal_amd.build``);
loading fails loudly otherwise, there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhstu.so")

HSTU_F32 = 0
HSTU_BF16 = 1

STATUS_NAMES = {
    0: "HSTU_OK", 1: "HSTU_E_NULL", 2: "HSTU_E_SHAPE", 3: "HSTU_E_DTYPE", 4: "HSTU_E_ALIGN",
    5: "HSTU_E_UNSUPPORTED", 6: "HSTU_E_WORKSPACE", 7: "HSTU_E_ALIAS", 8: "HSTU_E_HIP",
}

# Every function the header declares (checked against include/hstu.h by the CPU tests).
EXPORTED = (
    "hstu_attn_workspace_size", "hstu_attn_fwd", "hstu_attn_fwd_noalloc", "hstu_attn_bwd", "hstu_attn_fwd_candidates", "hstu_attn_cand_workspace_size",
    "hstu_layer_workspace_size", "hstu_layer_fwd",
    "hstu_layer_bwd_workspace_size", "hstu_layer_bwd",
    "hstu_head_workspace_size", "hstu_head_fwd",
    "hstu_stochastic_length", "hstu_gather_rows",
    "hstu_timing_enable", "hstu_timing_read",
    "hstu_status_string", "hstu_last_error", "hstu_version",
)


class Jagged(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("seq_offsets", ctypes.c_void_p),
        ("timestamps", ctypes.c_void_p),
    ]


class Bias(ctypes.Structure):
    _fields_ = [
        ("pos_table", ctypes.c_void_p),
        ("pos_buckets", ctypes.c_int32),
        ("time_table", ctypes.c_void_p),
        ("time_buckets", ctypes.c_int32),
    ]


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("dqk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("qk_scale", ctypes.c_float),
        ("divisor", ctypes.c_float),
    ]


class LayerParams(ctypes.Structure):
    _fields_ = [
        ("embed_dim", ctypes.c_int32),
        ("attn", AttnDesc),
        ("ln_eps", ctypes.c_float),
        ("ln_in_gamma", ctypes.c_void_p),
        ("ln_in_beta", ctypes.c_void_p),
        ("w_uvqk", ctypes.c_void_p),
        ("b_uvqk", ctypes.c_void_p),
        ("ln_out_gamma", ctypes.c_void_p),
        ("ln_out_beta", ctypes.c_void_p),
        ("w_out", ctypes.c_void_p),
        ("b_out", ctypes.c_void_p),
        ("bias", Bias),
    ]


class LayerGrads(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "d_ln_in_gamma", "d_ln_in_beta", "d_w_uvqk", "d_b_uvqk", "d_ln_out_gamma",
        "d_ln_out_beta", "d_w_out", "d_b_out", "d_pos_table", "d_time_table")]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_lib = None


def load() -> ctypes.CDLL:
    """Load libhstu.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m hstu_pointwise_attention_causal_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    c = ctypes.c_int32
    lib.hstu_attn_workspace_size.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.POINTER(_SZ)]
    lib.hstu_attn_workspace_size.restype = c
    lib.hstu_attn_fwd.argtypes = [_P, _P, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _SZ, _P]
    lib.hstu_attn_fwd.restype = c
    lib.hstu_attn_fwd_noalloc.argtypes = [_P, _P, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P]
    lib.hstu_attn_fwd_noalloc.restype = c
    lib.hstu_attn_bwd.argtypes = [_P, _P, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                  _P, _I64, _P, _I64, _P, _I64, _P, _P, _P, _SZ, _P]
    lib.hstu_attn_bwd.restype = c
    lib.hstu_attn_fwd_candidates.argtypes = [_P, _P, _P, c, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                             _P, _I64, _P, _I64, _P, _SZ, _P]
    lib.hstu_attn_cand_workspace_size.argtypes = [_P, _P, c, ctypes.POINTER(_SZ)]
    lib.hstu_attn_cand_workspace_size.restype = c
    lib.hstu_attn_fwd_candidates.restype = c
    lib.hstu_layer_workspace_size.argtypes = [_P, _P, ctypes.POINTER(_SZ)]
    lib.hstu_layer_workspace_size.restype = c
    lib.hstu_layer_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.hstu_layer_fwd.restype = c
    lib.hstu_layer_bwd_workspace_size.argtypes = [_P, _P, ctypes.POINTER(_SZ)]
    lib.hstu_layer_bwd_workspace_size.restype = c
    lib.hstu_layer_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.hstu_layer_bwd.restype = c
    lib.hstu_head_workspace_size.argtypes = [_I64, c, ctypes.POINTER(_SZ)]
    lib.hstu_head_workspace_size.restype = c
    lib.hstu_head_fwd.argtypes = [_I64, c, _I64, ctypes.c_float, _P, _I64, _P, _P, _I64, _P, _I64, _P, _SZ, _P]
    lib.hstu_head_fwd.restype = c
    lib.hstu_stochastic_length.argtypes = [c, _P, _I64, _I64, _P, _P, _P, _P]
    lib.hstu_stochastic_length.restype = c
    lib.hstu_gather_rows.argtypes = [_P, _P, _I64, _P, _I64, _I64, _P, _I64, _I64, _P]
    lib.hstu_gather_rows.restype = c
    lib.hstu_timing_enable.argtypes = [c]
    lib.hstu_timing_enable.restype = c
    lib.hstu_timing_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double)]
    lib.hstu_timing_read.restype = c
    lib.hstu_status_string.argtypes = [c]
    lib.hstu_status_string.restype = ctypes.c_char_p
    lib.hstu_last_error.argtypes = []
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_version.argtypes = []
    lib.hstu_version.restype = c
    _lib = lib
    return lib


class HstuError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


def check(status: int) -> None:
    if status != 0:
        lib = load()
        raise HstuError(status, lib.hstu_last_error().decode(errors="replace"))
