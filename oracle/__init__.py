"""CPU oracle (float64 / exact integer) for masked tiled attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP kernels or their host library.
"""
from . import attention, masks  # noqa: F401
from .attention import SKIP, PARTIAL, FULL  # noqa: F401
