"""CPU oracle for sparse index attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and by
the benchmark's CPU-baseline leg.  The HIP product path never imports it.
"""
from .sia_oracle import *  # noqa: F401,F403
from .sia_oracle import __all__  # noqa: F401
