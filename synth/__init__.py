"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This package only draws random numbers and places them at the byte positions of
each block format. It holds none of the decoding or matmul arithmetic, so both
the HIP path and the CPU oracle can consume its output without sharing code.
"""

from .gen import *  # noqa: F401,F403
