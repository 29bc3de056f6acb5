"""fp64 CPU oracle for the LaplacianFormer attention block.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the benchmark's CPU-baseline leg,
never by the GPU library.
"""
from .lf_oracle import *  # noqa: F401,F403
