"""CPU oracle for block-quantized weight products (test infrastructure only).

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path never does.
"""

from .oracle import *  # noqa: F401,F403
