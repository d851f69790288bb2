"""fp64 CPU oracle for batched Lloyd k-means.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU package.
"""
from .lloyd import *  # noqa: F401,F403
from .lloyd import __all__  # noqa: F401
from . import similarity  # noqa: F401  (dot-product and cosine k-means)
