"""CPU oracle for the W8A8 ConvRot expert-choice MoE layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg are the only
callers.  The product path never imports this package.  The arithmetic lives in ``convrot_oracle.c`` (plain
loops, IEEE fp32, no contraction); this package builds it with gcc and wraps it for numpy.
"""
from .binding import *  # noqa: F401,F403
from .binding import __all__  # noqa: F401
