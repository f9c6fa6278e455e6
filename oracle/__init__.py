"""CPU oracle for Sparse-Linear Attention (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The HIP library never does.
"""
from .sla_oracle import *  # noqa: F401,F403
