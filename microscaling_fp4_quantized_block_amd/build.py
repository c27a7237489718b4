"""Build libmxfp4.so (HIP, gfx950) in-tree with hipcc.

Usage: python microscaling_fp4_quantized_block_amd/build.py
(run as a file: importing the package loads the library this builds)
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys
import tempfile

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

# Identity of the kernels whose hardware counters are kept with the
# benchmark: the SHA-256 of each one's gfx950 assembly (function body,
# comments and label numbering left out), so a counter summary stays valid
# exactly as long as the code it was taken on, whatever else changes in the
# file.  Recorded next to the library by build(); the sources it was made
# from are fingerprinted too, so a stale record is noticed.
DIGEST_FILE = os.path.join(HERE, "kernel_digests.json")
DIGEST_SOURCE = "gemm.hip"
DIGEST_KERNELS = {"gemm_mx_kernel_f32": "_ZN5mxfp414gemm_mx_kernelILi0EEEvNS_8GemmArgsE"}


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


def _sources_fingerprint() -> str:
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _function_body(asm: str, symbol: str) -> str:
    lines, inside = [], False
    for ln in asm.splitlines():
        if ln.startswith(symbol + ":"):
            inside = True
            continue
        if inside:
            if ln.startswith(".Lfunc_end"):
                break
            code = ln.split(";", 1)[0].rstrip()
            if code:
                lines.append(re.sub(r"\.LBB\d+_", ".LBB_", code))
    if not lines:
        raise RuntimeError(f"{symbol} not found in the assembly")
    return "\n".join(lines)


def kernel_digests(compile_if_stale: bool = True) -> dict:
    """{kernel name: SHA-256 (16 hex digits) of its assembly}; from
    DIGEST_FILE when it matches the current sources, else compiled (or {}
    when compile_if_stale is False)."""
    fp = _sources_fingerprint()
    try:
        with open(DIGEST_FILE) as f:
            d = json.load(f)
        if d.get("sources") == fp:
            return d
    except (OSError, ValueError):
        pass
    if not compile_if_stale:
        return {}
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
        cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(CSRC, DIGEST_SOURCE), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed emitting the kernel assembly")
        with open(out) as f:
            asm = f.read()
    d = {"sources": fp}
    for name, sym in DIGEST_KERNELS.items():
        d[name] = hashlib.sha256(_function_body(asm, sym).encode()).hexdigest()[:16]
    with open(DIGEST_FILE + ".tmp", "w") as f:
        json.dump(d, f, indent=1)
    os.replace(DIGEST_FILE + ".tmp", DIGEST_FILE)
    return d


def build(verbose: bool = False) -> str:
    _hipcc(SOURCES, LIB, verbose)
    _hipcc(CLOCK_SOURCES, CLOCK_LIB, verbose)
    kernel_digests(compile_if_stale=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
