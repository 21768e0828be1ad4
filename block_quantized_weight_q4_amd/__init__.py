"""Block-quantized weight products (Q4_K, Q8_0, TQ1_G128) on MI355X.

The compute path is libkq.so (hand-written HIP for gfx950) behind the C ABI
in include/kq.h; ``kq`` is its thin Python binding.
"""

from .kq import *  # noqa: F401,F403
