"""MI355X (gfx950) HSTU hot path: causal pointwise aggregated attention over
jagged sequences and its backward, one HSTU layer forward and backward,
candidate scoring against cached history keys and values, Stochastic Length,
and the final RMSNorm with the tied retrieval head, behind the C ABI of
``libhstu.so`` (declared in ``include/hstu.h``).

The Python functions below only marshal torch tensors into that ABI. The
library is loaded on first use and its absence is an error: there is no CPU
or PyTorch fallback.
"""

from ._lib import HstuError, load  # noqa: F401
from .ops import (  # noqa: F401
    attn_bwd,
    attn_cand_workspace_size,
    attn_fwd,
    attn_fwd_candidates,
    attn_fwd_noalloc,
    attn_workspace_size,
    head_fwd,
    gather_rows,
    head_workspace_size,
    layer_bwd,
    layer_fwd,
    make_layer_params,
    stochastic_length,
    timing_enable,
    timing_read,
)

__all__ = [
    "HstuError", "load",
    "attn_fwd", "attn_fwd_noalloc", "attn_bwd", "attn_workspace_size",
    "attn_fwd_candidates", "attn_cand_workspace_size",
    "layer_fwd", "layer_bwd", "make_layer_params",
    "head_fwd", "head_workspace_size",
    "stochastic_length", "gather_rows",
    "timing_enable", "timing_read",
]
