"""Compile libkq.so (all HIP kernels + the C ABI) for gfx950, in-tree.

Each .hip source is compiled to an object in ``_build/`` in parallel, then
linked into ``block_quantized_weight_q4_amd/libkq.so``.  The streaming-read
measuring stick (``csrc/hbm_read.hip``) goes into its own
``libkq_hbmread.so``, which only the benchmark loads.  Always recompiles
(the caller asked for a build); ``build_if_missing`` only builds when the
library is absent.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkq.so")
READ_LIB = os.path.join(PKG, "libkq_hbmread.so")
READ_SOURCES = ["hbm_read.hip"]
SOURCES = ["api.hip", "dequant.hip", "skinny.hip", "mmv2.hip", "mmv3.hip", "gemm.hip", "moe.hip", "moe_dec.hip", "moe_mm.hip", "tq1mv.hip", "quantize.hip", "cmv.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=fast",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + READ_SOURCES
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], READ_LIB)
    if verbose:
        print(f"built {LIB} and {READ_LIB}")
    return LIB


def build_if_missing() -> str:
    if not (os.path.exists(LIB) and os.path.exists(READ_LIB)):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
