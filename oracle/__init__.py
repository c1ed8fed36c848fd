"""fp64 CPU oracle for R-SWA.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path.
"""
from . import rswa_oracle  # noqa: F401
