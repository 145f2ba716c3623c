"""Seeded synthetic inputs for the CompactAttention chunked-prefill path.

This package only draws random numbers and lays them out; it holds none of
the method's arithmetic (no union, no attention).  Both the CPU oracle's tests
and the GPU parity tests / benchmark take their inputs from here, so that the
two sides see exactly the same bytes.
"""
from .workloads import (  # noqa: F401
    BLOCK,
    WORKLOADS,
    VSLASH_DENSITIES,
    VSLASH_HEAD_MODES,
    Workload,
    bf16_bits_to_f32,
    make_custom,
    make_workload,
    tensor_to_f32,
)
from .prefill import PREFILL_STREAMS, PrefillStream, make_prefill_stream  # noqa: F401
