"""Build libmxfp4.so (HIP, gfx950) in-tree with hipcc.

Usage: python microscaling_fp4_quantized_block_amd/build.py
(run as a file: importing the package loads the library this builds)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxfp4.so")
SOURCES = ["quantize.hip", "gemm.hip", "noise.hip", "mse.hip", "noalloc.hip", "mxfp4_abi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # IEEE binary32 everywhere: the quantizer's code decisions must match the
    # specification bit for bit (no contraction into FMA, no fast math)
    "-ffp-contract=off", "-fno-fast-math",
    # no packed-FP32 VALU instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The benchmark's shader-clock stamps: a separate library, not part of libmxfp4.
CLOCK_LIB = os.path.join(HERE, "libmxclock.so")
CLOCK_SOURCES = ["clock_stamp.hip"]


def _hipcc(sources, out, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    _hipcc(SOURCES, LIB, verbose)
    _hipcc(CLOCK_SOURCES, CLOCK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
