"""Build the CPU oracle shared library (test infrastructure only).

``python -m oracle.build`` or ``build_oracle()`` compiles kq_oracle.c with gcc
into oracle/liboracle.so.  Plain C, IEEE double arithmetic (no fast-math, no
contraction into fused multiply-adds), OpenMP over independent output rows.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(force: bool = False) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas",
        SRC, "-o", tmp, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(force="--force" in sys.argv))
