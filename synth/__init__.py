"""Seeded synthetic inputs for the SnapKV compression path.

This package only draws random numbers and arranges them into the shapes the
compression path consumes. It contains none of the method's arithmetic (no
attention, pooling or selection), so both the CPU oracle and the GPU path can
take their inputs from it without sharing any of the computation.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    LayerInputs,
    bf16_round_bits,
    make_layer,
    make_custom,
    workload,
)
