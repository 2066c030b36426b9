"""Thin PyTorch binding over the C ABI (argument marshalling only).

PyTorch provides device memory and the current stream; every step of the
computation runs in the HIP kernels of libhstu.so. Functions keep the names
of the C entry points without the ``hstu_`` prefix.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.HSTU_BF16, torch.float32: _lib.HSTU_F32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _token_view(name: str, t: torch.Tensor, H: int):
    """Check a [T, H, d] view whose head/feature axes are contiguous; return (d, ld)."""
    if t.dim() != 3 or t.shape[1] != H:
        raise ValueError(f"{name} must be [T, {H}, d], got {tuple(t.shape)}")
    d = t.shape[2]
    if t.shape[0] == 0:
        return d, H * d
    if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != d):
        raise ValueError(f"{name}: heads and features must be contiguous inside a token row")
    return d, t.stride(0)


def _same_as(ref_name: str, ref: torch.Tensor, **named):
    """Every named tensor (None skipped) matches `ref` in dtype and device:
    the C ABI takes raw pointers and sizes, so a mismatch it cannot see would
    make a kernel read past a buffer or misread its elements."""
    for name, t in named.items():
        if t is None:
            continue
        if t.dtype != ref.dtype:
            raise ValueError(f"{name} is {t.dtype}, {ref_name} is {ref.dtype}")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, {ref_name} on {ref.device}")


def _tokens_heads(name: str, t: torch.Tensor, T: int, H: int, d: Optional[int] = None):
    if t.dim() != 3 or t.shape[0] != T or t.shape[1] != H or (d is not None and t.shape[2] != d):
        want = f"[{T}, {H}, {'d' if d is None else d}]"
        raise ValueError(f"{name} must be {want}, got {tuple(t.shape)}")


def _same_device(ref_name: str, ref: torch.Tensor, **named):
    for name, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, {ref_name} on {ref.device}")


def _on_gpu(**named):
    """Every tensor argument is device memory (the library dereferences the
    pointers on the GPU)."""
    for name, t in named.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")


def _check_bias_tables(H: int, ref: torch.Tensor, pos_table, time_table, timestamps, T: int):
    for name, t in (("pos_table", pos_table), ("time_table", time_table)):
        if t is not None:
            if t.dim() != 2 or t.shape[0] != H:
                raise ValueError(f"{name} must be [{H}, buckets], got {tuple(t.shape)}")
            if t.device != ref.device:
                raise ValueError(f"{name} is on {t.device}, q on {ref.device}")
    if timestamps is not None:
        if timestamps.dim() != 1 or timestamps.numel() != T:
            raise ValueError(f"timestamps must hold one entry per token ({T}), got {tuple(timestamps.shape)}")
        if timestamps.device != ref.device:
            raise ValueError(f"timestamps are on {timestamps.device}, q on {ref.device}")
    if time_table is not None and timestamps is None and T > 0:
        raise ValueError("a time table needs timestamps")


def _check_offsets(name: str, off: torch.Tensor):
    if off.dtype != torch.int64 or off.dim() != 1 or not off.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D int64 tensor")
    if off.numel() < 1:
        raise ValueError(f"{name} needs B + 1 >= 1 entries")


def _jagged(seq_offsets: torch.Tensor, total_tokens: int, timestamps: Optional[torch.Tensor]):
    _check_offsets("seq_offsets", seq_offsets)
    if timestamps is not None and (timestamps.dtype != torch.int64 or not timestamps.is_contiguous()):
        raise ValueError("timestamps must be a contiguous int64 tensor")
    j = _lib.Jagged()
    j.num_seqs = seq_offsets.numel() - 1
    j.total_tokens = total_tokens
    j.seq_offsets = seq_offsets.data_ptr() if seq_offsets.numel() else None
    j.timestamps = timestamps.data_ptr() if timestamps is not None else None
    return j


def _bias(pos_table: Optional[torch.Tensor], time_table: Optional[torch.Tensor]):
    b = _lib.Bias()
    for t, name in ((pos_table, "pos_table"), (time_table, "time_table")):
        if t is not None and (t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [H, buckets] tensor")
    if pos_table is not None:
        b.pos_table = pos_table.data_ptr()
        b.pos_buckets = pos_table.shape[1]
    if time_table is not None:
        b.time_table = time_table.data_ptr()
        b.time_buckets = time_table.shape[1]
    return b


def _desc(H, dqk, dv, dtype, alpha, divisor):
    d = _lib.AttnDesc()
    d.num_heads, d.dqk, d.dv = H, dqk, dv
    d.dtype = _DT[dtype]
    d.qk_scale = float(alpha)
    d.divisor = float(divisor)
    return d


def attn_workspace_size(num_heads: int, dqk: int, dv: int, dtype: torch.dtype, num_seqs: int,
                        total_tokens: int, is_bwd: bool = False, pos_buckets: int = 0,
                        time_buckets: int = 0) -> int:
    lib = _lib.load()
    d = _desc(num_heads, dqk, dv, dtype, 1.0, 0.0)
    j = _lib.Jagged()
    j.num_seqs, j.total_tokens = num_seqs, total_tokens
    j.seq_offsets = 16 if num_seqs else None   # only non-NULL-ness is read
    b = _lib.Bias()
    if pos_buckets:
        b.pos_table, b.pos_buckets = 16, pos_buckets
    if time_buckets:
        b.time_table, b.time_buckets = 16, time_buckets
        j.timestamps = 16
    out = ctypes.c_size_t(0)
    _lib.check(lib.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b),
                                            int(is_bwd), ctypes.byref(out)))
    return out.value


def _attn_fwd_args(q, k, v, seq_offsets, timestamps, pos_table, time_table, alpha, divisor, out, workspace):
    """Checks and marshals the arguments shared by attn_fwd and attn_fwd_noalloc."""
    if q.dtype not in _DT:
        raise ValueError(f"q must be bf16 or fp32, got {q.dtype}")
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, d], got {tuple(q.shape)}")
    T, H = q.shape[0], q.shape[1]
    _tokens_heads("k", k, T, H, q.shape[2])
    _tokens_heads("v", v, T, H)
    _same_as("q", q, k=k, v=v, out=out)
    _check_offsets("seq_offsets", seq_offsets)
    _same_device("q", q, seq_offsets=seq_offsets, workspace=workspace)
    if out is not None:
        _tokens_heads("out", out, T, H, v.shape[2])
    _check_bias_tables(H, q, pos_table, time_table, timestamps, T)
    _on_gpu(q=q, k=k, v=v, out=out, seq_offsets=seq_offsets, timestamps=timestamps, pos_table=pos_table,
            time_table=time_table, workspace=workspace)
    lib = _lib.load()
    dqk, ldq = _token_view("q", q, H)
    _, ldk = _token_view("k", k, H)
    dv, ldv = _token_view("v", v, H)
    if out is None:
        out = torch.empty((T, H, dv), dtype=v.dtype, device=v.device)
    _, ldo = _token_view("o", out, H)
    d = _desc(H, dqk, dv, q.dtype, alpha, divisor)
    j = _jagged(seq_offsets, T, timestamps)
    b = _bias(pos_table, time_table)
    return lib, T, H, ldq, ldk, ldv, out, ldo, d, j, b


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_offsets: torch.Tensor, *,
             timestamps: Optional[torch.Tensor] = None, pos_table: Optional[torch.Tensor] = None,
             time_table: Optional[torch.Tensor] = None, alpha: float = 1.0, divisor: float = 0.0,
             out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_attn_fwd on [T, H, d] tensors (bf16 or fp32) of one jagged batch."""
    lib, T, H, ldq, ldk, ldv, out, ldo, d, j, b = _attn_fwd_args(
        q, k, v, seq_offsets, timestamps, pos_table, time_table, alpha, divisor, out, workspace)
    need = ctypes.c_size_t(0)
    _lib.check(lib.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b), 0,
                                            ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.hstu_attn_fwd(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b),
                                 _ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv, _ptr(out), ldo,
                                 _ptr(workspace), workspace.numel(), _stream_handle(q.device)))
    return out


def attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_offsets: torch.Tensor, *,
                     timestamps: Optional[torch.Tensor] = None, pos_table: Optional[torch.Tensor] = None,
                     time_table: Optional[torch.Tensor] = None, alpha: float = 1.0, divisor: float = 0.0,
                     out: torch.Tensor) -> torch.Tensor:
    """hstu_attn_fwd_noalloc: attn_fwd without a workspace (the library's own
    fixed device array holds it). `out` must be passed: the call allocates
    nothing, and calls that overlap in time on one GPU race on the array."""
    lib, T, H, ldq, ldk, ldv, out, ldo, d, j, b = _attn_fwd_args(
        q, k, v, seq_offsets, timestamps, pos_table, time_table, alpha, divisor, out, None)
    _lib.check(lib.hstu_attn_fwd_noalloc(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b),
                                         _ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv, _ptr(out), ldo,
                                         _stream_handle(q.device)))
    return out


def attn_cand_workspace_size(num_heads: int, d: int, num_seqs: int, hist_tokens: int, max_candidates: int) -> int:
    """hstu_attn_cand_workspace_size: workspace bytes of attn_fwd_candidates."""
    desc = _desc(num_heads, d, d, torch.bfloat16, 1.0, 0.0)
    j = _lib.Jagged()
    j.num_seqs, j.total_tokens = int(num_seqs), int(hist_tokens)
    need = _lib._SZ(0)
    _lib.check(_lib.load().hstu_attn_cand_workspace_size(ctypes.byref(desc), ctypes.byref(j), int(max_candidates),
                                                         ctypes.byref(need)))
    return int(need.value)


def attn_fwd_candidates(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cand_offsets: torch.Tensor,
                        k_hist: torch.Tensor, v_hist: torch.Tensor, hist_offsets: torch.Tensor, *,
                        timestamps: Optional[torch.Tensor] = None,
                        cand_timestamps: Optional[torch.Tensor] = None,
                        pos_table: Optional[torch.Tensor] = None, time_table: Optional[torch.Tensor] = None,
                        alpha: float = 1.0, divisor: float = 0.0, max_candidates: Optional[int] = None,
                        out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_attn_fwd_candidates: candidates q, k, v [T_c, H, d] (offsets
    cand_offsets) scored against a history with cached k_hist, v_hist
    [T_h, H, d] (offsets hist_offsets). max_candidates defaults to the largest
    per-sequence candidate count (read from cand_offsets on the host)."""
    if q.dim() != 3:
        raise ValueError(f"q must be [T_c, H, d], got {tuple(q.shape)}")
    Tc, H, dd = q.shape
    for name, t in (("k", k), ("v", v)):
        _tokens_heads(name, t, Tc, H, dd)
    Th = k_hist.shape[0] if k_hist.dim() == 3 else -1
    for name, t in (("k_hist", k_hist), ("v_hist", v_hist)):
        _tokens_heads(name, t, Th, H, dd)
    if out is not None:
        _tokens_heads("out", out, Tc, H, dd)
    _same_as("q", q, k=k, v=v, k_hist=k_hist, v_hist=v_hist, out=out)
    _same_device("q", q, cand_offsets=cand_offsets, hist_offsets=hist_offsets, cand_timestamps=cand_timestamps,
                 workspace=workspace)
    _check_bias_tables(H, q, pos_table, time_table, timestamps, Th)
    if cand_timestamps is not None and (cand_timestamps.dim() != 1 or cand_timestamps.numel() != Tc):
        raise ValueError(f"cand_timestamps must hold one entry per candidate ({Tc})")
    if time_table is not None and cand_timestamps is None and Tc > 0:
        raise ValueError("a time table needs candidate timestamps")
    _check_offsets("hist_offsets", hist_offsets)
    _check_offsets("cand_offsets", cand_offsets)
    if hist_offsets.numel() != cand_offsets.numel():
        raise ValueError("hist_offsets and cand_offsets must describe the same number of sequences")
    _on_gpu(q=q, k=k, v=v, k_hist=k_hist, v_hist=v_hist, out=out, cand_offsets=cand_offsets,
            hist_offsets=hist_offsets, timestamps=timestamps, cand_timestamps=cand_timestamps,
            pos_table=pos_table, time_table=time_table, workspace=workspace)
    lib = _lib.load()
    d, ldq = _token_view("q", q, H)
    _, ldk = _token_view("k", k, H)
    _, ldv = _token_view("v", v, H)
    _, ldkh = _token_view("k_hist", k_hist, H)
    _, ldvh = _token_view("v_hist", v_hist, H)
    if out is None:
        out = torch.empty((Tc, H, d), dtype=v.dtype, device=v.device)
    _, ldo = _token_view("o", out, H)
    if max_candidates is None:
        c = cand_offsets.cpu()
        max_candidates = int((c[1:] - c[:-1]).max()) if c.numel() > 1 else 0
    desc = _desc(H, d, d, q.dtype, alpha, divisor)
    jh = _jagged(hist_offsets, k_hist.shape[0], timestamps)
    jc = _jagged(cand_offsets, Tc, cand_timestamps)
    b = _bias(pos_table, time_table)
    need = _lib._SZ(0)
    _lib.check(lib.hstu_attn_cand_workspace_size(ctypes.byref(desc), ctypes.byref(jh), int(max_candidates),
                                                 ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.hstu_attn_fwd_candidates(ctypes.byref(desc), ctypes.byref(jh), ctypes.byref(jc),
                                            int(max_candidates), ctypes.byref(b), _ptr(k_hist), ldkh,
                                            _ptr(v_hist), ldvh, _ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv,
                                            _ptr(out), ldo, _ptr(workspace), workspace.numel(),
                                            _stream_handle(q.device)))
    return out


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, d_o: torch.Tensor,
             seq_offsets: torch.Tensor, *, timestamps: Optional[torch.Tensor] = None,
             pos_table: Optional[torch.Tensor] = None, time_table: Optional[torch.Tensor] = None,
             alpha: float = 1.0, divisor: float = 0.0, workspace: Optional[torch.Tensor] = None,
             out: Optional[tuple] = None):
    """hstu_attn_bwd: returns (dq, dk, dv, d_pos_table or None, d_time_table or None).
    ``out`` may pass preallocated tensors in that order (the same shapes)."""
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, d], got {tuple(q.shape)}")
    T, H = q.shape[0], q.shape[1]
    _tokens_heads("k", k, T, H, q.shape[2])
    _tokens_heads("v", v, T, H)
    _tokens_heads("d_o", d_o, T, H, v.shape[2])
    _same_as("q", q, k=k, v=v, d_o=d_o)
    _check_offsets("seq_offsets", seq_offsets)
    _same_device("q", q, seq_offsets=seq_offsets, workspace=workspace)
    _check_bias_tables(H, q, pos_table, time_table, timestamps, T)
    if out is not None:
        dq, dk, dvv, dP, dTt = out
        _tokens_heads("dq", dq, T, H, q.shape[2])
        _tokens_heads("dk", dk, T, H, q.shape[2])
        _tokens_heads("dv", dvv, T, H, v.shape[2])
        _same_as("q", q, dq=dq, dk=dk, dv=dvv)
        for name, g, t in (("d_pos_table", dP, pos_table), ("d_time_table", dTt, time_table)):
            if (g is None) != (t is None):
                raise ValueError(f"{name} must be given exactly when its table is")
            if g is not None and (g.dtype != torch.float32 or tuple(g.shape) != tuple(t.shape)
                                  or not g.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {tuple(t.shape)}")
        _on_gpu(dq=dq, dk=dk, dv=dvv, d_pos_table=dP, d_time_table=dTt)
    _on_gpu(q=q, k=k, v=v, d_o=d_o, seq_offsets=seq_offsets, timestamps=timestamps, pos_table=pos_table,
            time_table=time_table, workspace=workspace)
    lib = _lib.load()
    dqk, ldq = _token_view("q", q, H)
    _, ldk = _token_view("k", k, H)
    dv_, ldv = _token_view("v", v, H)
    _, lddo = _token_view("d_o", d_o, H)
    if out is None:
        dq = torch.empty((T, H, dqk), dtype=q.dtype, device=q.device)
        dk = torch.empty((T, H, dqk), dtype=q.dtype, device=q.device)
        dvv = torch.empty((T, H, dv_), dtype=q.dtype, device=q.device)
        dP = torch.empty_like(pos_table) if pos_table is not None else None
        dTt = torch.empty_like(time_table) if time_table is not None else None
    d = _desc(H, dqk, dv_, q.dtype, alpha, divisor)
    j = _jagged(seq_offsets, T, timestamps)
    b = _bias(pos_table, time_table)
    need = ctypes.c_size_t(0)
    _lib.check(lib.hstu_attn_workspace_size(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b), 1,
                                            ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.hstu_attn_bwd(ctypes.byref(d), ctypes.byref(j), ctypes.byref(b),
                                 _ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv, _ptr(d_o), lddo,
                                 _ptr(dq), _token_view("dq", dq, H)[1], _ptr(dk), _token_view("dk", dk, H)[1],
                                 _ptr(dvv), _token_view("dv", dvv, H)[1],
                                 _ptr(dP), _ptr(dTt), _ptr(workspace), workspace.numel(),
                                 _stream_handle(q.device)))
    return dq, dk, dvv, dP, dTt


def make_layer_params(embed_dim: int, num_heads: int, dqk: int, dv: int, *, w_uvqk, w_out,
                      ln_in_gamma, ln_in_beta, ln_out_gamma, ln_out_beta, b_uvqk=None, b_out=None,
                      pos_table=None, time_table=None, ln_eps: float = 1e-6, alpha: float = 1.0,
                      divisor: float = 0.0):
    """Build the hstu_layer_params_t for device tensors (kept alive by the caller)."""
    D, H = int(embed_dim), int(num_heads)
    n1, hv = H * (2 * dv + 2 * dqk), H * dv
    want = {"ln_in_gamma": ((D,), torch.float32), "ln_in_beta": ((D,), torch.float32),
            "w_uvqk": ((n1, D), torch.bfloat16), "b_uvqk": ((n1,), torch.float32),
            "ln_out_gamma": ((hv,), torch.float32), "ln_out_beta": ((hv,), torch.float32),
            "w_out": ((D, hv), torch.bfloat16), "b_out": ((D,), torch.float32)}
    given = {"ln_in_gamma": ln_in_gamma, "ln_in_beta": ln_in_beta, "w_uvqk": w_uvqk, "b_uvqk": b_uvqk,
             "ln_out_gamma": ln_out_gamma, "ln_out_beta": ln_out_beta, "w_out": w_out, "b_out": b_out}
    device = None
    for name, t in given.items():
        if t is None:
            if name in ("b_uvqk", "b_out"):
                continue
            raise ValueError(f"{name} is required")
        shape, dtype = want[name]
        if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} "
                             f"(nn.Linear layout [out, in] for weights), got {t.dtype} {tuple(t.shape)}")
        device = t.device if device is None else device
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other parameters on {device}")
    for name, t in (("pos_table", pos_table), ("time_table", time_table)):
        if t is not None and (t.dim() != 2 or t.shape[0] != H or t.device != device):
            raise ValueError(f"{name} must be [{H}, buckets] on {device}, got {tuple(t.shape)} on {t.device}")
    _on_gpu(pos_table=pos_table, time_table=time_table, **given)
    p = _lib.LayerParams()
    p.embed_dim = embed_dim
    p.attn = _desc(num_heads, dqk, dv, torch.bfloat16, alpha, divisor)
    p.ln_eps = float(ln_eps)
    for name, t in given.items():
        setattr(p, name, None if t is None else t.data_ptr())
    p.bias = _bias(pos_table, time_table)
    return p


def layer_fwd(x: torch.Tensor, seq_offsets: torch.Tensor, params: "_lib.LayerParams", *,
              timestamps: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              uvqk_out: Optional[torch.Tensor] = None, o_out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_layer_fwd on a bf16 [T, D] input; returns X'."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [T, D] tensor")
    T, D = x.shape
    _check_layer_io(x, params, timestamps)
    H, dqk, dv = params.attn.num_heads, params.attn.dqk, params.attn.dv
    n1, hv = H * (2 * dv + 2 * dqk), H * dv
    for name, t, w in (("out", out, D), ("uvqk_out", uvqk_out, n1), ("o_out", o_out, hv)):
        if t is not None and (t.dtype != torch.bfloat16 or tuple(t.shape) != (T, w) or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bf16 [{T}, {w}] tensor")
    _on_gpu(x=x, seq_offsets=seq_offsets, timestamps=timestamps, out=out, uvqk_out=uvqk_out, o_out=o_out,
            workspace=workspace)
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(x)
    j = _jagged(seq_offsets, T, timestamps)
    need = ctypes.c_size_t(0)
    _lib.check(lib.hstu_layer_workspace_size(ctypes.byref(params), ctypes.byref(j), ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=x.device)
    _lib.check(lib.hstu_layer_fwd(ctypes.byref(params), ctypes.byref(j), _ptr(x), _ptr(out),
                                  _ptr(uvqk_out), _ptr(o_out), _ptr(workspace), workspace.numel(),
                                  _stream_handle(x.device)))
    return out


def _check_layer_io(x: torch.Tensor, params: "_lib.LayerParams", timestamps: Optional[torch.Tensor]):
    """x agrees with the layer's width; timestamps cover every token when the
    layer has a time table."""
    T, D = x.shape
    if D != params.embed_dim:
        raise ValueError(f"x has {D} features, the layer's embed_dim is {params.embed_dim}")
    if timestamps is not None and (timestamps.dim() != 1 or timestamps.numel() != T):
        raise ValueError(f"timestamps must hold one entry per token ({T})")
    if params.bias.time_table and timestamps is None and T > 0:
        raise ValueError("the layer has a time table: timestamps are required")


LAYER_GRAD_NAMES = ("d_ln_in_gamma", "d_ln_in_beta", "d_w_uvqk", "d_b_uvqk", "d_ln_out_gamma",
                    "d_ln_out_beta", "d_w_out", "d_b_out", "d_pos_table", "d_time_table")


def layer_bwd(x: torch.Tensor, d_out: torch.Tensor, seq_offsets: torch.Tensor,
              params: "_lib.LayerParams", *, timestamps: Optional[torch.Tensor] = None,
              dx: Optional[torch.Tensor] = None, grads: Optional[dict] = None,
              workspace: Optional[torch.Tensor] = None):
    """hstu_layer_bwd: gradients of sum(X' * d_out) for the layer with these
    parameters at input x (bf16 [T, D]). Returns (dx, dict of fp32 parameter
    gradients keyed as LAYER_GRAD_NAMES; the table entries are present when the
    layer has that table). `grads` may supply the output tensors."""
    for name, t in (("x", x), ("d_out", d_out)):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 [T, D] tensor")
    if d_out.shape != x.shape:
        raise ValueError("d_out must have the shape of x")
    T, D = x.shape
    _check_layer_io(x, params, timestamps)
    if dx is not None and (dx.dtype != torch.bfloat16 or dx.shape != x.shape or not dx.is_contiguous()):
        raise ValueError("dx must be a contiguous bf16 tensor of the shape of x")
    _on_gpu(x=x, d_out=d_out, dx=dx, seq_offsets=seq_offsets, timestamps=timestamps, workspace=workspace)
    lib = _lib.load()
    H, dqk, dv = params.attn.num_heads, params.attn.dqk, params.attn.dv
    n1, hv = H * (2 * dv + 2 * dqk), H * dv
    if dx is None:
        dx = torch.empty_like(x)
    shapes = {"d_ln_in_gamma": (D,), "d_ln_in_beta": (D,), "d_w_uvqk": (n1, D), "d_b_uvqk": (n1,),
              "d_ln_out_gamma": (hv,), "d_ln_out_beta": (hv,), "d_w_out": (D, hv), "d_b_out": (D,)}
    if params.bias.pos_table:
        shapes["d_pos_table"] = (H, params.bias.pos_buckets)
    if params.bias.time_table:
        shapes["d_time_table"] = (H, params.bias.time_buckets)
    grads = dict(grads or {})
    for name, shp in shapes.items():
        if name not in grads:
            grads[name] = torch.empty(shp, dtype=torch.float32, device=x.device)
    g = _lib.LayerGrads()
    for name in LAYER_GRAD_NAMES:
        t = grads.get(name) if name in shapes else None
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shapes[name]):
            raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {shapes[name]}")
        setattr(g, name, None if t is None else t.data_ptr())
    j = _jagged(seq_offsets, T, timestamps)
    need = ctypes.c_size_t(0)
    _lib.check(lib.hstu_layer_bwd_workspace_size(ctypes.byref(params), ctypes.byref(j), ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=x.device)
    _lib.check(lib.hstu_layer_bwd(ctypes.byref(params), ctypes.byref(j), _ptr(x), _ptr(d_out), _ptr(dx),
                                  ctypes.byref(g), _ptr(workspace), workspace.numel(), _stream_handle(x.device)))
    return dx, {k: grads[k] for k in shapes}


def head_workspace_size(rows: int, dim: int) -> int:
    """hstu_head_workspace_size: workspace bytes of head_fwd."""
    need = _lib._SZ(0)
    _lib.check(_lib.load().hstu_head_workspace_size(int(rows), int(dim), ctypes.byref(need)))
    return int(need.value)


def head_fwd(x: torch.Tensor, table: torch.Tensor, *, gamma: Optional[torch.Tensor] = None,
             eps: float = 1e-6, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_head_fwd: bf16 logits [rows, vocab] = RMSNorm(x; gamma, eps)
    table^T for token rows x [rows, dim] and an item table [vocab, dim] (the
    token-embedding table when the head's weights are tied)."""
    if x.dim() != 2 or table.dim() != 2 or x.shape[1] != table.shape[1]:
        raise ValueError("x [rows, dim] and table [vocab, dim] must share dim")
    if x.dtype != torch.bfloat16 or table.dtype != torch.bfloat16:
        raise ValueError("x and table must be bf16")
    if gamma is not None and (gamma.dtype != torch.float32 or tuple(gamma.shape) != (x.shape[1],)
                              or not gamma.is_contiguous()):
        raise ValueError(f"gamma must be a contiguous fp32 [{x.shape[1]}] tensor")
    if out is not None and out.dtype != torch.bfloat16:
        raise ValueError("out must be bf16")
    _same_device("x", x, table=table, gamma=gamma, out=out, workspace=workspace)
    _on_gpu(x=x, table=table, gamma=gamma, out=out, workspace=workspace)
    lib = _lib.load()
    if x.stride(1) != 1 or table.stride(1) != 1:
        raise ValueError("x and table rows must be contiguous")
    rows, dim = x.shape
    vocab = table.shape[0]
    if out is None:
        out = torch.empty((rows, vocab), dtype=torch.bfloat16, device=x.device)
    if out.dim() != 2 or out.shape[0] != rows or out.shape[1] != vocab or out.stride(1) != 1:
        raise ValueError("out must be [rows, vocab] with contiguous rows")
    need = head_workspace_size(rows, dim)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _lib.check(lib.hstu_head_fwd(rows, dim, vocab, float(eps), _ptr(x), x.stride(0), _ptr(gamma),
                                 _ptr(table), table.stride(0), _ptr(out), out.stride(0),
                                 _ptr(workspace), workspace.numel(), _stream_handle(x.device)))
    return out


def stochastic_length(seq_offsets: torch.Tensor, keys: torch.Tensor, max_len: int, *,
                      new_offsets: Optional[torch.Tensor] = None,
                      gather_index: Optional[torch.Tensor] = None):
    """hstu_stochastic_length: (new_offsets int64 [B+1], gather_index int64
    [T]) for int64 offsets [B+1] and one uint32 key per token (held in an
    int32 tensor, bit for bit). Only the first new_offsets[-1] entries of
    gather_index are written; nothing here waits for the device."""
    if seq_offsets.dtype != torch.int64 or keys.dtype not in (torch.int32, torch.uint32):
        raise ValueError("seq_offsets must be int64 and keys 32-bit")
    if seq_offsets.dim() != 1 or not seq_offsets.is_contiguous() or not keys.is_contiguous():
        raise ValueError("seq_offsets and keys must be contiguous, seq_offsets 1-D")
    for name, t in (("new_offsets", new_offsets), ("gather_index", gather_index)):
        if t is not None and (t.dtype != torch.int64 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int64 tensor")
    _same_device("keys", keys, seq_offsets=seq_offsets, new_offsets=new_offsets, gather_index=gather_index)
    _on_gpu(keys=keys, seq_offsets=seq_offsets, new_offsets=new_offsets, gather_index=gather_index)
    lib = _lib.load()
    B, T = seq_offsets.numel() - 1, keys.numel()
    if new_offsets is None:
        new_offsets = torch.empty(B + 1, dtype=torch.int64, device=keys.device)
    if gather_index is None:
        gather_index = torch.empty(max(T, 1), dtype=torch.int64, device=keys.device)
    if new_offsets.numel() < B + 1 or gather_index.numel() < T:
        raise ValueError("new_offsets needs B+1 entries and gather_index T")
    _lib.check(lib.hstu_stochastic_length(B, _ptr(seq_offsets), T, int(max_len), _ptr(keys), _ptr(new_offsets),
                                          _ptr(gather_index), _stream_handle(keys.device)))
    return new_offsets, gather_index


def gather_rows(src: torch.Tensor, index: torch.Tensor, count: torch.Tensor, max_rows: int, *,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_gather_rows: out[r] = src[index[r]] for r < min(count, max_rows),
    count a one-element int64 device tensor (e.g. new_offsets[-1:]). Rows are
    src's first axis; each row must be contiguous."""
    if count.dtype != torch.int64 or index.dtype != torch.int64:
        raise ValueError("index and count must be int64")
    if out is not None and (out.dtype != src.dtype or tuple(out.shape[1:]) != tuple(src.shape[1:])
                            or out.shape[0] < max_rows):
        raise ValueError("out must have src's dtype and row shape and at least max_rows rows")
    if index.numel() < max_rows or count.numel() < 1:
        raise ValueError("index needs max_rows entries (the kernel may read that many) and count one")
    _same_device("src", src, index=index, count=count, out=out)
    _on_gpu(src=src, index=index, count=count, out=out)
    lib = _lib.load()
    row_shape = tuple(src.shape[1:])
    if out is None:
        out = torch.empty((max_rows,) + row_shape, dtype=src.dtype, device=src.device)
    row_bytes = src[0:1].numel() * src.element_size() if src.shape[0] else \
        int(torch.tensor(row_shape).prod()) * src.element_size()
    if src.dim() > 1 and not src[0:1].is_contiguous() or out.dim() > 1 and not out[0:1].is_contiguous():
        raise ValueError("rows must be contiguous")
    _lib.check(lib.hstu_gather_rows(_ptr(index), _ptr(count), int(max_rows), _ptr(src), src.shape[0],
                                    src.stride(0) * src.element_size(), _ptr(out),
                                    out.stride(0) * out.element_size(), row_bytes, _stream_handle(src.device)))
    return out


def timing_enable(enable: bool = True) -> None:
    """hstu_timing_enable: bracket every timed kernel launch with HIP events."""
    _lib.check(_lib.load().hstu_timing_enable(int(bool(enable))))


def timing_read(kernel: str):
    """hstu_timing_read: (launches, total milliseconds) of `kernel` since its
    last read; waits for the recorded events."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _lib.check(_lib.load().hstu_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)
