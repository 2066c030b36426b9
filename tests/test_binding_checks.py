"""Host checks of the Python binding: every operand must agree with q (dtype,
device, token count, heads, head dim), tables must have one row per head,
timestamps one entry per token, layer weights their [out, in] shapes and
dtypes, and every tensor must be GPU memory. The C ABI receives raw pointers
and cannot see any of this, so each mismatch must raise ValueError before a
call is made. CPU tensors only: no kernel is launched."""

import pytest
import torch

from hstu_pointwise_attention_causal_amd import ops

T, H, D = 40, 2, 64


def _attn(**over):
    bf = torch.bfloat16
    a = dict(q=torch.zeros(T, H, D, dtype=bf), k=torch.zeros(T, H, D, dtype=bf), v=torch.zeros(T, H, D, dtype=bf),
             seq_offsets=torch.tensor([0, 10, T], dtype=torch.int64),
             timestamps=torch.zeros(T, dtype=torch.int64),
             pos_table=torch.zeros(H, 16), time_table=torch.zeros(H, 8))
    a.update(over)
    return a


def _fwd(a):
    ops.attn_fwd(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("seq_offsets"), **a)


@pytest.mark.parametrize("over,msg", [
    (dict(k=torch.zeros(T, H, D, dtype=torch.float32)), "k is torch.float32"),
    (dict(v=torch.zeros(T - 1, H, D, dtype=torch.bfloat16)), "v must be"),
    (dict(k=torch.zeros(T, H, 32, dtype=torch.bfloat16)), "k must be"),
    (dict(k=torch.zeros(T, H + 1, D, dtype=torch.bfloat16)), "k must be"),
    (dict(pos_table=torch.zeros(H + 1, 16)), "pos_table must be"),
    (dict(time_table=torch.zeros(1, H, 8)), "time_table must be"),
    (dict(timestamps=torch.zeros(T - 3, dtype=torch.int64)), "timestamps must hold"),
    (dict(timestamps=None), "needs timestamps"),
    (dict(out=torch.zeros(T, H, D, dtype=torch.float32)), "out is torch.float32"),
    (dict(out=torch.zeros(T, H, 2 * D, dtype=torch.bfloat16)), "out must be"),
    (dict(q=torch.zeros(T, H, D, dtype=torch.float16), k=torch.zeros(T, H, D, dtype=torch.float16),
          v=torch.zeros(T, H, D, dtype=torch.float16)), "bf16 or fp32"),
    (dict(seq_offsets=torch.zeros(2, 2, dtype=torch.int64)), "seq_offsets"),
    (dict(), "must be a GPU tensor"),
])
def test_attn_fwd_mismatches_raise(over, msg):
    with pytest.raises(ValueError, match=msg):
        _fwd(_attn(**over))


@pytest.mark.parametrize("over,msg", [
    (dict(d_o=torch.zeros(T, H, D, dtype=torch.float32)), "d_o is torch.float32"),
    (dict(d_o=torch.zeros(T, H, D + 8, dtype=torch.bfloat16)), "d_o must be"),
    (dict(k=torch.zeros(T + 1, H, D, dtype=torch.bfloat16)), "k must be"),
    (dict(time_table=torch.zeros(H + 2, 8)), "time_table must be"),
    (dict(), "must be a GPU tensor"),
])
def test_attn_bwd_mismatches_raise(over, msg):
    a = _attn(d_o=torch.zeros(T, H, D, dtype=torch.bfloat16))
    a.update(over)
    with pytest.raises(ValueError, match=msg):
        ops.attn_bwd(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("d_o"), a.pop("seq_offsets"), **a)


def test_attn_bwd_gradient_outputs_checked():
    a = _attn(d_o=torch.zeros(T, H, D, dtype=torch.bfloat16))
    bf = torch.bfloat16
    good = [torch.zeros(T, H, D, dtype=bf) for _ in range(3)] + [torch.zeros(H, 16), torch.zeros(H, 8)]
    for i, bad in ((0, torch.zeros(T, H, D, dtype=torch.float32)), (3, torch.zeros(H, 17)), (4, None)):
        out = list(good)
        out[i] = bad
        b = dict(a)
        with pytest.raises(ValueError):
            ops.attn_bwd(b.pop("q"), b.pop("k"), b.pop("v"), b.pop("d_o"), b.pop("seq_offsets"),
                         out=tuple(out), **b)


def _cand(**over):
    bf = torch.bfloat16
    Tc, Th = 12, 30
    a = dict(q=torch.zeros(Tc, H, D, dtype=bf), k=torch.zeros(Tc, H, D, dtype=bf), v=torch.zeros(Tc, H, D, dtype=bf),
             cand_offsets=torch.tensor([0, 5, Tc]), k_hist=torch.zeros(Th, H, D, dtype=bf),
             v_hist=torch.zeros(Th, H, D, dtype=bf), hist_offsets=torch.tensor([0, 10, Th]),
             timestamps=torch.zeros(Th, dtype=torch.int64), cand_timestamps=torch.zeros(Tc, dtype=torch.int64),
             pos_table=torch.zeros(H, 16), time_table=torch.zeros(H, 8), max_candidates=7)
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(v_hist=torch.zeros(29, H, D, dtype=torch.bfloat16)), "v_hist must be"),
    (dict(k=torch.zeros(12, H, D, dtype=torch.float32)), "k must be|k is"),
    (dict(cand_timestamps=torch.zeros(11, dtype=torch.int64)), "cand_timestamps"),
    (dict(timestamps=torch.zeros(31, dtype=torch.int64)), "timestamps must hold"),
    (dict(hist_offsets=torch.tensor([0, 30])), "same number of sequences"),
    (dict(), "must be a GPU tensor"),
])
def test_candidates_mismatches_raise(over, msg):
    a = _cand(**over)
    with pytest.raises(ValueError, match=msg):
        ops.attn_fwd_candidates(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("cand_offsets"), a.pop("k_hist"),
                                a.pop("v_hist"), a.pop("hist_offsets"), **a)


def _layer_kw(D_=512, H_=4, d=128, **over):
    n1, hv = H_ * 4 * d, H_ * d
    kw = dict(w_uvqk=torch.zeros(n1, D_, dtype=torch.bfloat16), w_out=torch.zeros(D_, hv, dtype=torch.bfloat16),
              ln_in_gamma=torch.ones(D_), ln_in_beta=torch.zeros(D_), ln_out_gamma=torch.ones(hv),
              ln_out_beta=torch.zeros(hv), pos_table=torch.zeros(H_, 128))
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,msg", [
    (dict(w_uvqk=torch.zeros(512, 2048, dtype=torch.bfloat16)), "w_uvqk must be"),   # [in, out] by mistake
    (dict(w_out=torch.zeros(512, 512, dtype=torch.float32)), "w_out must be"),
    (dict(ln_out_gamma=torch.ones(511)), "ln_out_gamma must be"),
    (dict(b_out=torch.zeros(512, dtype=torch.bfloat16)), "b_out must be"),
    (dict(pos_table=torch.zeros(3, 128)), "pos_table must be"),
    (dict(ln_in_beta=None), "ln_in_beta is required"),
    (dict(), "must be a GPU tensor"),
])
def test_layer_params_checked(over, msg):
    with pytest.raises(ValueError, match=msg):
        ops.make_layer_params(512, 4, 128, 128, **_layer_kw(**over))


def test_head_and_stochastic_length_checked():
    x = torch.zeros(8, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="bf16"):
        ops.head_fwd(x, torch.zeros(16, 512))
    with pytest.raises(ValueError, match="gamma"):
        ops.head_fwd(x, torch.zeros(16, 512, dtype=torch.bfloat16), gamma=torch.ones(256))
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.head_fwd(x, torch.zeros(16, 512, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.stochastic_length(torch.tensor([0, 4]), torch.zeros(4, dtype=torch.int32), 2)
    with pytest.raises(ValueError, match="index needs"):
        ops.gather_rows(torch.zeros(10, 4), torch.zeros(3, dtype=torch.int64), torch.zeros(1, dtype=torch.int64), 5)
