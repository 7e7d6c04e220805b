"""fp64 CPU oracle of the p4 group-circulant linear layer and of the p4 group
convolution (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never does.
"""
from .eqlin_oracle import *  # noqa: F401,F403
from .eqlin_oracle import __all__ as _lin_all
from .eqconv_oracle import *  # noqa: F401,F403
from .eqconv_oracle import __all__ as _conv_all

__all__ = list(_lin_all) + list(_conv_all)
