"""fp64 CPU oracle for the TTT scan — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library neither links nor loads it.  See
ttt_oracle.h for the definition it computes and the readings it takes.
"""
from .oracle import build, linear, linear_bwd, linear_ln, linear_momentum, mlp, gelu, gelu_prime, lib_path  # noqa: F401
