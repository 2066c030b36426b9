"""Seeded synthetic inputs for the HSTU attention / layer workloads.

This package holds only input generation: random draws, shapes, offsets,
timestamps and the round-to-nearest-even conversion of the drawn values to
bfloat16. It holds none of the method's arithmetic (no bias bucketing, no
SiLU, no attention, no norm). Both the fp64 oracle and the HIP path consume
exactly the arrays produced here.
"""

from .generators import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_workload,
    round_to_bf16,
    log_uniform_lengths,
    exponential_timestamps,
    embedding_rows,
    xavier_uniform,
)
