"""CPU oracle for the Groth16 H-polynomial pipeline (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The product path (the HIP library and its binding) never
calls it.  See oracle.c for what is computed and which passage each part follows;
the G1 multi-scalar multiplication's oracle is the submodule `msm` (msm_oracle.c).
"""
from .oracle import *  # noqa: F401,F403
