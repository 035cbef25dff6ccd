"""fp64 CPU oracle of Native Sparse Attention (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the GPU library.
"""
from .nsa_oracle import *  # noqa: F401,F403
from .nsa_oracle import __all__  # noqa: F401
