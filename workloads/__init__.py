"""Seeded synthetic inputs for XAttention block-sparse prefill.

This package only draws numbers and lays them out (token-major Q/K/V,
cu_seqlens, paged block tables, pinned-history splits).  It holds none of the
method's arithmetic, so both the float64 oracle and the HIP path can consume
the same tensors without sharing any code that computes a result.
"""

from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_layer_pair,
    make_workload,
    make_random,
    make_well_separated,
    to_paged,
)
