"""Seeded synthetic inputs for the MoE grouped GEMM.

This package is shared by the GPU path's tests and bench and by the oracle's
tests.  It produces input bit patterns and offset arrays only: it contains no
part of the grouped GEMM's arithmetic (no products, no sums over a reduction
axis, no output rounding).
"""
from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    make_workload,
    normal_bf16_bits,
    offsets_from_sizes,
    router_offsets,
    zipf_sizes,
    random_offsets,
)
