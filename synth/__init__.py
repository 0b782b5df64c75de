"""Seeded synthetic inputs (masks in column-sparse form, Q/K/V/dO, workloads).

Shared by the tests, the benchmark and the oracle checks; holds no attention
arithmetic.
"""
from . import masks, tensors, configs  # noqa: F401
