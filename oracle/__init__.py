"""fp64 CPU oracle of the p4 group-circulant linear layer (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never does.
"""
from .eqlin_oracle import *  # noqa: F401,F403
from .eqlin_oracle import __all__  # noqa: F401
