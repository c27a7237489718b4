"""Host AddressSanitizer / UndefinedBehaviorSanitizer run of the C ABI layer
and the CPU oracle: libmxfp4 is rebuilt with the sanitizers on its host code
only (device code is compiled as usual; nothing is launched), the oracle is
built with them, and tests/sanitize/host_driver.cpp exercises the argument
checks, the size queries and every oracle entry point.  A sanitizer report
makes the driver exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "microscaling_fp4_quantized_block_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang"      # the host compiler hipcc drives: one sanitizer runtime for all parts


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANG), reason="needs hipcc and ROCm clang")
def test_abi_and_oracle_clean_under_host_sanitizers(tmp_path):
    srcs = [os.path.join(CSRC, s) for s in ("quantize.hip", "gemm.hip", "noise.hip", "mse.hip", "noalloc.hip", "mxfp4_abi.cpp")]
    lib = str(tmp_path / "libmxfp4_san.so")
    # sanitizers on the host code only: each -fsanitize= right after -Xarch_host
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    obj = str(tmp_path / "oracle.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
                        "-fno-omit-frame-pointer", "-c", os.path.join(ROOT, "oracle", "mxfp4_oracle.c"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "host_driver")
    r = subprocess.run([CLANG + "++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-fopenmp", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), obj, lib, "-L/opt/rocm/lib",
                        "-lamdhip64", "-Wl,-rpath," + str(tmp_path) + ":/opt/rocm/lib:/opt/rocm/lib/llvm/lib", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-5000:])
    assert "all checks passed" in r.stdout
