"""Seeded synthetic inputs for the KDA forward workloads.

This package is shared by the tests, the benchmark and the CPU oracle's
callers.  It draws random numbers and shapes them into the input
distributions of the five workloads; it performs none of the KDA
computation itself (no recurrence, no chunk algebra, no layer maths).
"""
from .gen import (  # noqa: F401
    DECODE,
    WORKLOADS,
    Workload,
    bf16_bits,
    bf16_round,
    core_inputs,
    core_inputs_block,
    decode_inputs,
    layer_inputs,
    window_start,
)
