"""Seeded synthetic inputs shared by the GPU path, the CPU oracle and the bench.

This package only draws random numbers and converts storage formats
(bf16 bit patterns <-> float64).  It contains none of the attention method's
arithmetic: no distances, no assignment, no aggregation, no softmax.
"""

from .generators import (  # noqa: F401
    WORKLOADS,
    WORKLOAD_ORDER,
    EXTRA_WORKLOADS,
    Inputs,
    generate,
    generate_dyadic,
    generate_dyadic3,
    generate_one_key_per_leaf,
    f64_to_bf16_bits,
    bf16_bits_to_f64,
    to_storage,
    storage_to_f64,
)
