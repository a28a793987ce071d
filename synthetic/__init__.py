"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

Nothing in this package computes any part of the paged-attention method:
it draws sequence lengths, a pool free order, an allocation trace, queries
and per-token key/value vectors, and hands them to whichever side asks.
"""
from .workloads import (  # noqa: F401
    Op,
    Workload,
    WORKLOADS,
    make_workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    MemoryTrace,
    memory_trace,
    multi_query,
)
