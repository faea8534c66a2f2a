"""Float64 CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library.
"""
from . import attention, brute  # noqa: F401
