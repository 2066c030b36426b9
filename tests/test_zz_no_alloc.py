"""hstu_attn_fwd_noalloc (the attention forward whose workspace is the
library's own fixed device array) against hstu_attn_fwd with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
batch, each bitwise equal to the workspace entry point's output (the same
kernels on the same work list) and within the bf16 tolerance of the oracle;
and a batch beyond the array's size is rejected with HSTU_E_UNSUPPORTED."""

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import TOL_BF16, attn_inputs_on_device, rel_err
from workloads import make_workload
from workloads.generators import _attn_recipe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hstu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import hstu_pointwise_attention_causal_amd as pkg
    pkg.load()
    return pkg


def _both(hstu, wl):
    import torch
    d = attn_inputs_on_device(wl)
    kw = dict(timestamps=d["timestamps"], pos_table=d["pos_table"], time_table=d["time_table"], alpha=wl.alpha,
              divisor=wl.divisor)
    ref_gpu = hstu.attn_fwd(d["q"], d["k"], d["v"], d["seq_offsets"], **kw)
    out = torch.full_like(ref_gpu, float("nan"))
    hstu.attn_fwd_noalloc(d["q"], d["k"], d["v"], d["seq_offsets"], out=out, **kw)
    torch.cuda.synchronize()
    return out, ref_gpu


def test_two_calls_in_a_row_match_the_workspace_entry_point(hstu):
    import torch
    big = make_workload("c3_small")                                   # 5 ragged sequences up to 517 tokens, H 3
    small = _attn_recipe("noalloc_small", 61, [130, 0, 77], 2, 64)     # then a smaller batch
    for wl in (big, small):
        got, want = _both(hstu, wl)
        assert torch.equal(got, want), wl.name
        ref = orc.attn_fwd(wl.q, wl.k, wl.v, wl.seq_offsets, alpha=wl.alpha, divisor=wl.divisor,
                           pos_table=wl.pos_table, time_table=wl.time_table, timestamps=wl.timestamps)
        err = rel_err(got.float().cpu().numpy(), ref)
        print(f"{wl.name}: noalloc == workspace entry point bitwise; oracle err {err:.2e}")
        assert err <= TOL_BF16


def test_batch_beyond_the_array_is_rejected(hstu):
    """T x H far beyond what 16 MiB holds: refused before anything runs (the
    tensors are views of a small buffer, never read)."""
    import torch
    from hstu_pointwise_attention_causal_amd import _lib
    T, H = 1 << 24, 4
    base = torch.zeros(H * 32, dtype=torch.bfloat16, device="cuda:0")
    q = base.as_strided((T, H, 32), (0, 32, 1))      # every token row aliases one H x 32 row
    off = torch.tensor([0, T], dtype=torch.int64, device="cuda:0")
    out = torch.zeros(H * 32, dtype=torch.bfloat16, device="cuda:0").as_strided((T, H, 32), (0, 32, 1))
    with pytest.raises(_lib.HstuError) as e:
        hstu.attn_fwd_noalloc(q, q, q, off, out=out)
    assert e.value.status == 5, e.value
