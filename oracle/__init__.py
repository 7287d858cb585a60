"""Plain fp64 CPU oracle of the Kamera reuse operator.

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg of
the benchmark import this package.  The GPU product path never does.
"""
from .oracle import *  # noqa: F401,F403
