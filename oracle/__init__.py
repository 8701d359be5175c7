"""fp64 CPU oracle of the block-indexed sparse attention step.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg, never by the library's product path.
"""
from . import sa_oracle  # noqa: F401
