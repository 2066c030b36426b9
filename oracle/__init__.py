"""fp64 CPU oracle for HSTU causal pointwise aggregated attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it. It shares no code with the HIP path (no
kernels, headers, helpers or tables), and the HIP path never falls back to it.

``oracle.oracle`` is the plain NumPy float64 definition of what the path
computes; ``oracle.brute`` restates the same operations as pure-Python loops
for tiny inputs. The pins that check both against the mathematics live in
``tests/test_oracle_*.py``.
"""

from .oracle import (  # noqa: F401
    attn_bwd,
    attn_fwd,
    attn_fwd_rows,
    layer_fwd,
    layer_fwd_rows,
    layer_norm,
    pos_bucket,
    silu,
    stack_fwd,
    time_bucket,
)
