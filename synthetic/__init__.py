"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package draws random numbers, rounds them to the storage dtype and builds
the row bookkeeping (labels, masks, aligned target-row maps) of each workload.
It holds none of the loss arithmetic, so both sides can read the same bits
without sharing any of the method.
"""
from .gen import (  # noqa: F401
    Problem,
    WORKLOADS,
    make_problem,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
)
