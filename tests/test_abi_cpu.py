"""C-ABI contract of libmxfp4, checked on the CPU: every symbol declared in
include/mxfp4.h is exported, size queries return the closed-form byte counts,
and invalid arguments are rejected with the documented status before anything
is launched (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")

OK, INVALID, SHAPE, MISMATCH, WORKSPACE = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def mx():
    import microscaling_fp4_quantized_block_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mxfp4_status|const char\s*\*)\s*(mxfp4_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mxfp4_quantize", "mxfp4_dequantize", "mxfp4_gemm", "mxfp4_tensor_bytes",
              "mxfp4_quantize_workspace_bytes", "mxfp4_gemm_workspace_bytes", "mxfp4_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(mx):
    for n in declared_functions():
        assert hasattr(mx.lib, n), n


def test_status_strings(mx):
    for code in (OK, INVALID, SHAPE, MISMATCH, WORKSPACE, -5):
        assert mx.mxfp4_status_string(code).startswith(mx.STATUS[code])
    assert "unknown" in mx.mxfp4_status_string(42)


def test_tensor_bytes(mx):
    assert mx.mxfp4_tensor_bytes("mx", 4096, 8192) == (4096 * 4096, 4096 * 256)
    assert mx.mxfp4_tensor_bytes("nv", 10, 48) == (240, 30)
    assert mx.mxfp4_tensor_bytes("mx", 0, 0) == (0, 0)
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert mx.lib.mxfp4_tensor_bytes(0, 4, 48, ctypes.byref(cb), ctypes.byref(sb)) == SHAPE
    assert mx.lib.mxfp4_tensor_bytes(2, 4, 64, ctypes.byref(cb), ctypes.byref(sb)) == INVALID
    assert mx.lib.mxfp4_tensor_bytes(0, -1, 64, ctypes.byref(cb), ctypes.byref(sb)) == INVALID
    assert mx.lib.mxfp4_tensor_bytes(0, 4, 64, None, ctypes.byref(sb)) == INVALID


def test_quantize_workspace_bytes(mx):
    assert mx.mxfp4_quantize_workspace_bytes("mx", 100, 64) == 0
    assert mx.mxfp4_quantize_workspace_bytes("nv", 100, 64) == 4096
    # NVFP4: one 32-bit partial per 2048 16-byte chunks of the tensor-amax scan,
    # at least 1024 (the rotated pass), ranges of whole rows below 2^30 chunks
    assert mx.mxfp4_quantize_workspace_bytes("nv", 14336, 8192) == 4 * (14336 * 1024 // 2048)
    assert mx.mxfp4_quantize_workspace_bytes("nv", 2 ** 20 + 1, 2 ** 13) == 4 * (2 ** 30 // 2048 + 1)
    assert mx.mxfp4_quantize_workspace_bytes("nv", 3, 2 ** 33) == 4 * 3 * (2 ** 30 // 2048)
    assert mx.mxfp4_quantize_workspace_bytes("nv", 3, 2 ** 33 + 16) == 4 * 3 * (2 ** 30 // 2048 + 1)
    b = ctypes.c_size_t()
    assert mx.lib.mxfp4_quantize_workspace_bytes(0, 4, 64, 2, ctypes.byref(b)) == INVALID


FAKE = 0x100000   # a 16-byte-aligned non-null address; never dereferenced


def desc(mx, fmt=0, had=0, rows=64, k=256, codes=FAKE, scales=FAKE, ts=FAKE):
    return mx.MxTensorStruct(fmt, had, rows, k, codes, scales, ts)


def quantize(mx, R=64, C=256, ldx=256, fmt=0, rnd=0, had=0, axis=1, out=None, ws=None, ws_bytes=0, x=FAKE):
    if out is None:
        rows, k = (R, C) if axis == 1 else (C, R)
        out = desc(mx, fmt, had, rows, k)
    return mx.lib.mxfp4_quantize(x, R, C, ldx, fmt, rnd, had, axis, 0, ctypes.byref(out) if out != "null" else None,
                                 ws, ws_bytes, None)


def test_quantize_rejects_bad_arguments(mx):
    assert quantize(mx, fmt=3) == INVALID
    assert quantize(mx, rnd=2) == INVALID
    assert quantize(mx, had=2) == INVALID
    assert quantize(mx, axis=2) == INVALID
    assert quantize(mx, out="null") == INVALID
    assert quantize(mx, ldx=100) == INVALID                     # ldx < C
    assert quantize(mx, C=48, ldx=48) == SHAPE                  # k % 32
    assert quantize(mx, fmt=1, C=48, ldx=48, out=desc(mx, 1, 0, 64, 48)) == WORKSPACE  # NV: 16 | 48 ok, no workspace
    assert quantize(mx, fmt=1, had=1, C=48, ldx=48) == SHAPE    # rotation needs k % 32
    assert quantize(mx, R=40, axis=0) == SHAPE                  # axis 0: k = R = 40
    assert quantize(mx, out=desc(mx, rows=63)) == INVALID       # descriptor disagrees with the call
    assert quantize(mx, out=desc(mx, had=1)) == INVALID
    assert quantize(mx, out=desc(mx, fmt=1)) == INVALID
    assert quantize(mx, x=None) == INVALID
    assert quantize(mx, out=desc(mx, codes=FAKE + 4)) == INVALID    # codes must be 16-byte aligned
    assert quantize(mx, fmt=1, out=desc(mx, 1, ts=None)) == INVALID
    assert quantize(mx, fmt=1, out=desc(mx, 1), ws=FAKE, ws_bytes=100) == WORKSPACE
    # empty tensors are valid no-ops
    assert quantize(mx, R=0, out=desc(mx, rows=0)) == OK
    assert quantize(mx, R=64, C=0, ldx=1, out=desc(mx, rows=64, k=0)) == OK


def qnoise(mx, R=64, C=256, ldx=256, fmt=0, rnd=1, had=0, axis=1, out=None, stats=FAKE, ws=FAKE, ws_bytes=1 << 20,
           x=FAKE):
    if out is None:
        rows, k = (R, C) if axis == 1 else (C, R)
        out = desc(mx, fmt, had, rows, k)
    return mx.lib.mxfp4_quantize_noise(x, R, C, ldx, fmt, rnd, had, axis, 0,
                                       ctypes.byref(out) if out != "null" else None, stats, ws, ws_bytes, None)


def qnoise_ws(mx, fmt, had, R, C, axis):
    b = ctypes.c_size_t()
    s = mx.lib.mxfp4_quantize_noise_workspace_bytes(fmt, had, R, C, axis, ctypes.byref(b))
    return s, b.value


def test_quantize_noise_rejects_bad_arguments(mx):
    assert qnoise(mx, fmt=3) == INVALID
    assert qnoise(mx, rnd=2) == INVALID
    assert qnoise(mx, axis=2) == INVALID
    assert qnoise(mx, out="null") == INVALID
    assert qnoise(mx, stats=None) == INVALID
    assert qnoise(mx, stats=FAKE + 4) == INVALID                   # stats: 8-byte aligned doubles
    assert qnoise(mx, ldx=100) == INVALID
    assert qnoise(mx, C=48, ldx=48) == SHAPE
    assert qnoise(mx, out=desc(mx, rows=63)) == INVALID
    assert qnoise(mx, x=None) == INVALID
    assert qnoise(mx, x=FAKE + 1) == INVALID                       # bf16 input: 2-byte aligned
    assert qnoise(mx, out=desc(mx, codes=FAKE + 4)) == INVALID
    assert qnoise(mx, fmt=1, out=desc(mx, 1, ts=None)) == INVALID
    assert qnoise(mx, ws=None) == WORKSPACE
    assert qnoise(mx, ws=FAKE + 8) == WORKSPACE                    # 16-byte aligned workspace
    assert qnoise(mx, ws_bytes=95) == WORKSPACE                     # 4 workgroups x 24 bytes needed


def test_quantize_noise_workspace_bytes(mx):
    assert qnoise_ws(mx, 3, 0, 64, 256, 1)[0] == INVALID
    assert qnoise_ws(mx, 0, 0, 64, 48, 1)[0] == SHAPE
    # MXFP4 rows: one triple of doubles per workgroup of 512 16-byte chunks
    assert qnoise_ws(mx, 0, 0, 50432, 3072, 1) == (OK, 24 * (50432 * 3072 // 8 // 512))
    # transposed: the larger of the tiled kernel's 64 x 256 tiles and the
    # separate noise pass's workgroups (256 units of 32)
    assert qnoise_ws(mx, 0, 0, 50432, 3072, 0) == (OK, 24 * (3072 * 50432 // 32 // 256))
    # NVFP4: the quantizer's amax partials (16-byte padded) come first
    s, b = qnoise_ws(mx, 1, 0, 4096, 4096, 1)
    q = mx.mxfp4_quantize_workspace_bytes("nv", 4096, 4096)
    assert s == OK and b == ((q + 15) // 16 * 16) + 24 * (4096 * 4096 // 8 // 512)
    # empty input: room for one triple
    assert qnoise_ws(mx, 0, 0, 0, 256, 1) == (OK, 24)


def test_dequantize_rejects_bad_arguments(mx):
    d = desc(mx)
    assert mx.lib.mxfp4_dequantize(None, FAKE, 256, None) == INVALID
    assert mx.lib.mxfp4_dequantize(ctypes.byref(d), FAKE, 100, None) == INVALID
    assert mx.lib.mxfp4_dequantize(ctypes.byref(desc(mx, k=48)), FAKE, 48, None) == SHAPE
    assert mx.lib.mxfp4_dequantize(ctypes.byref(d), None, 256, None) == INVALID
    assert mx.lib.mxfp4_dequantize(ctypes.byref(desc(mx, fmt=1, ts=None)), FAKE, 256, None) == INVALID
    assert mx.lib.mxfp4_dequantize(ctypes.byref(desc(mx, rows=0)), None, 256, None) == OK


def test_gemm_rejects_bad_arguments(mx):
    a, b = desc(mx, rows=64, k=256), desc(mx, rows=32, k=256)
    g = lambda A, B, C=FAKE, ldc=32, ws=None, wsb=0: mx.lib.mxfp4_gemm(
        ctypes.byref(A) if A is not None else None, ctypes.byref(B), C, ldc, ws, wsb, None)
    assert g(None, b) == INVALID
    assert g(a, desc(mx, fmt=1, rows=32)) == MISMATCH
    assert g(a, desc(mx, rows=32, k=512)) == MISMATCH
    assert g(a, desc(mx, had=1, rows=32)) == MISMATCH
    assert g(desc(mx, k=96), desc(mx, rows=32, k=96)) == SHAPE     # MX needs k % 128
    assert g(desc(mx, k=(1 << 24) + 128), desc(mx, rows=32, k=(1 << 24) + 128)) == SHAPE   # longest contraction
    assert g(a, b, ldc=16) == INVALID
    assert g(a, b, C=None) == INVALID
    assert g(desc(mx, codes=FAKE + 8), b) == INVALID              # operand codes must be 16-byte aligned
    assert g(desc(mx, fmt=1, ts=None), desc(mx, fmt=1, rows=32)) == INVALID
    assert g(desc(mx, rows=0), b) == OK                            # empty output: no-op


def test_gemm_bf16_rejects_bad_arguments(mx):
    """The bf16-output GEMM checks what mxfp4_gemm checks, and a bf16 C needs
    only 2-byte alignment."""
    a, b = desc(mx, rows=64, k=256), desc(mx, rows=32, k=256)
    g = lambda A, B, C=FAKE, ldc=32, ws=None, wsb=0: mx.lib.mxfp4_gemm_bf16(
        ctypes.byref(A) if A is not None else None, ctypes.byref(B), C, ldc, ws, wsb, None)
    assert g(None, b) == INVALID
    assert g(a, desc(mx, fmt=1, rows=32)) == MISMATCH
    assert g(desc(mx, k=96), desc(mx, rows=32, k=96)) == SHAPE
    assert g(a, b, ldc=16) == INVALID
    assert g(a, b, C=None) == INVALID
    assert g(a, b, C=FAKE + 1) == INVALID                          # bf16 C must be 2-byte aligned
    assert g(desc(mx, codes=FAKE + 8), b) == INVALID
    assert g(desc(mx, rows=0), b) == OK
    # a split plan still needs its FP32 partial-sum workspace (64 rows against
    # 96 over K = 32768: past the decode kernel's bytes per workgroup)
    A, B = desc(mx, rows=64, k=32768), desc(mx, rows=96, k=32768)
    assert mx.lib.mxfp4_gemm_bf16(ctypes.byref(A), ctypes.byref(B), FAKE + 2, 96, None, 0, None) == WORKSPACE


def test_gemm_fp32_output_alignment(mx):
    a, b = desc(mx, rows=64, k=256), desc(mx, rows=32, k=256)
    assert mx.lib.mxfp4_gemm(ctypes.byref(a), ctypes.byref(b), FAKE + 2, 32, None, 0, None) == INVALID


def test_gemm_workspace_query_matches_split_plan(mx):
    b = ctypes.c_size_t()
    # 64 x 96 outputs over a long contraction (80 x 16384 operand bytes per
    # decode workgroup, past its limit): the narrow kernel split along K
    # into 32 ranges, fp32 partials
    A, B = desc(mx, rows=64, k=32768), desc(mx, rows=96, k=32768)
    assert mx.lib.mxfp4_gemm_workspace_bytes(ctypes.byref(A), ctypes.byref(B), ctypes.byref(b)) == OK
    assert b.value == 32 * 64 * 96 * 4
    # the same rows over K = 8192 take the decode kernel: no workspace
    A, B = desc(mx, rows=64, k=8192), desc(mx, rows=96, k=8192)
    assert mx.lib.mxfp4_gemm_workspace_bytes(ctypes.byref(A), ctypes.byref(B), ctypes.byref(b)) == OK
    assert b.value == 0
    # a large output needs no split
    A, B = desc(mx, rows=4096, k=8192), desc(mx, rows=14336, k=8192)
    assert mx.lib.mxfp4_gemm_workspace_bytes(ctypes.byref(A), ctypes.byref(B), ctypes.byref(b)) == OK
    assert b.value == 0
    # the split GEMM rejects a missing workspace before launching
    A, B = desc(mx, rows=64, k=32768), desc(mx, rows=96, k=32768)
    assert mx.lib.mxfp4_gemm(ctypes.byref(A), ctypes.byref(B), FAKE, 96, None, 0, None) == WORKSPACE


def test_nv_gemm_needs_k_multiple_of_128(mx):
    g = lambda A, B: mx.lib.mxfp4_gemm(ctypes.byref(A), ctypes.byref(B), FAKE, 32, None, 0, None)
    assert g(desc(mx, fmt=1, k=192), desc(mx, fmt=1, rows=32, k=192)) == SHAPE


def qgemm(mx, M=16, K=256, ldx=256, had=0, B=None, C=FAKE, ldc=64, ws=None, wsb=0, x=FAKE):
    if B is None:
        B = desc(mx, had=had, rows=64, k=K)
    return mx.lib.mxfp4_quantize_gemm(x, M, K, ldx, had, ctypes.byref(B) if B != "null" else None, C, ldc, ws, wsb,
                                      None)


def qgemm_ws(mx, M, K, had, B):
    b = ctypes.c_size_t()
    s = mx.lib.mxfp4_quantize_gemm_workspace_bytes(M, K, had, ctypes.byref(B), ctypes.byref(b))
    return s, b.value


def test_quantize_gemm_rejects_bad_arguments(mx):
    assert qgemm(mx, B="null") == INVALID
    assert qgemm(mx, had=2, B=desc(mx, rows=64)) == INVALID
    assert qgemm(mx, B=desc(mx, fmt=1, rows=64)) == MISMATCH            # weights must be MXFP4
    assert qgemm(mx, B=desc(mx, rows=64, k=512)) == MISMATCH            # contraction lengths differ
    assert qgemm(mx, had=1, B=desc(mx, had=0, rows=64)) == MISMATCH     # rotation must match the weights'
    assert qgemm(mx, K=96, ldx=96, B=desc(mx, rows=64, k=96)) == SHAPE  # k % 128
    assert qgemm(mx, K=(1 << 24) + 128, ldx=(1 << 24) + 128, B=desc(mx, rows=64, k=(1 << 24) + 128)) == SHAPE
    assert qgemm(mx, ldx=100) == INVALID                                 # ldx < K
    assert qgemm(mx, ldc=63) == INVALID                                  # ldc < N
    assert qgemm(mx, x=None) == INVALID
    assert qgemm(mx, C=None) == INVALID
    assert qgemm(mx, B=desc(mx, rows=64, codes=FAKE + 8)) == INVALID    # weight codes must be 16-byte aligned
    assert qgemm(mx, M=0) == OK                                          # empty output: no-op
    # a decode shape needs its workspace (the quantized activations)
    B = desc(mx, rows=14336, k=4096)
    assert qgemm(mx, M=16, K=4096, ldx=4096, B=B, ldc=14336) == WORKSPACE


def test_quantize_gemm_workspace_bytes(mx):
    # decode 16 x 14336 x 4096 and 16 x 4096 x 14336 (decode plans): quantized
    # into the workspace (codes and scales, 16-byte padded), then the decode
    # GEMM, which needs no workspace
    assert qgemm_ws(mx, 16, 4096, 0, desc(mx, rows=14336, k=4096)) == (OK, 16 * 2048 + 16 * 128)
    assert qgemm_ws(mx, 16, 4096, 1, desc(mx, had=1, rows=14336, k=4096)) == (OK, 16 * 2048 + 16 * 128)
    assert qgemm_ws(mx, 16, 14336, 1, desc(mx, had=1, rows=4096, k=14336)) == (OK, 16 * 7168 + 16 * 448)
    # wide activations: quantized codes and scales (16-byte padded), no split
    assert qgemm_ws(mx, 300, 1024, 0, desc(mx, rows=512, k=1024)) == (OK, 300 * 512 + 300 * 32)
    # 128 rows against 65536 weight rows: the decode GEMM too
    assert qgemm_ws(mx, 128, 8192, 0, desc(mx, rows=65536, k=8192)) == (OK, 128 * 4096 + 128 * 256)
    # 100 rows against 1024 weight rows over K = 16384 (past the decode
    # kernel's bytes per workgroup): the narrow plan with 128-row tiles, 16
    # splits, not fused (the fused kernel takes 32-row tiles): codes, scales
    # and the split partials
    assert qgemm_ws(mx, 100, 16384, 0, desc(mx, rows=1024, k=16384)) == (
        OK, 100 * 8192 + 100 * 512 + 16 * 100 * 1024 * 4)
    # 16 rows against 1024 weight rows over K = 65536 (32 x 32768 operand
    # bytes per decode workgroup, past its limit): fused into the narrow GEMM,
    # 4 column tiles over 128 stage pairs -> 32 splits of 4 pairs; only the
    # split partial sums
    assert qgemm_ws(mx, 16, 65536, 1, desc(mx, had=1, rows=1024, k=65536)) == (OK, 32 * 16 * 1024 * 4)
    # the same against K = 8192: the decode GEMM after quantizing into the workspace
    assert qgemm_ws(mx, 16, 8192, 1, desc(mx, had=1, rows=1024, k=8192)) == (OK, 16 * 4096 + 16 * 256)
    assert qgemm_ws(mx, 16, 4096, 0, desc(mx, fmt=1, rows=64, k=4096))[0] == MISMATCH


def noise(mx, q=None, ldx=256, axis=1, x=FAKE, stats=FAKE, ws=FAKE, wsb=1 << 20):
    if q is None:
        q = desc(mx)
    return mx.lib.mxfp4_quantization_noise(x, ldx, axis, ctypes.byref(q) if q != "null" else None, stats, ws, wsb,
                                           None)


def test_quantization_noise_rejects_bad_arguments(mx):
    assert noise(mx, q="null") == INVALID
    assert noise(mx, axis=2) == INVALID
    assert noise(mx, q=desc(mx, fmt=2)) == INVALID
    assert noise(mx, q=desc(mx, k=48)) == SHAPE                  # MX block of 32
    assert noise(mx, q=desc(mx, fmt=1, had=1, k=48)) == SHAPE    # rotation needs k % 32
    assert noise(mx, ldx=100) == INVALID                         # axis 1: x is [rows, k], ldx >= k
    assert noise(mx, axis=0, ldx=63) == INVALID                  # axis 0: x is [k, rows], ldx >= rows
    assert noise(mx, x=None) == INVALID
    assert noise(mx, stats=None) == INVALID
    assert noise(mx, stats=FAKE + 4) == INVALID                  # stats are doubles
    assert noise(mx, q=desc(mx, fmt=1, ts=None)) == INVALID
    assert noise(mx, q=desc(mx, codes=FAKE + 4)) == INVALID      # codes are read as 8-byte words
    assert noise(mx, ws=None) == WORKSPACE
    assert noise(mx, wsb=8) == WORKSPACE


def test_quantization_noise_workspace_bytes(mx):
    b = ctypes.c_size_t()
    f = lambda q: (mx.lib.mxfp4_quantization_noise_workspace_bytes(ctypes.byref(q), ctypes.byref(b)), b.value)
    # three doubles per workgroup; a workgroup covers 256 units of 32 elements, at most 65536 workgroups
    assert f(desc(mx, rows=64, k=256)) == (OK, 2 * 24)
    assert f(desc(mx, rows=50432, k=3072)) == (OK, 18912 * 24)
    assert f(desc(mx, rows=1 << 20, k=8192)) == (OK, 65536 * 24)
    assert f(desc(mx, fmt=1, rows=10, k=48)) == (OK, 24)        # NVFP4, units of 16: one workgroup
    assert f(desc(mx, rows=0, k=0)) == (OK, 24)
    assert mx.lib.mxfp4_quantization_noise_workspace_bytes(None, ctypes.byref(b)) == INVALID


def qmse(mx, R=64, C=256, ldx=256, fmt=0, had=0, axis=1, iters=2, out=None, ws=FAKE, wsb=1 << 20, x=FAKE):
    if out is None:
        rows, k = (R, C) if axis == 1 else (C, R)
        out = desc(mx, fmt, had, rows, k)
    return mx.lib.mxfp4_quantize_mse(x, R, C, ldx, fmt, had, axis, iters, ctypes.byref(out) if out != "null" else None,
                                     ws, wsb, None)


def test_quantize_mse_rejects_bad_arguments(mx):
    assert qmse(mx, fmt=3) == INVALID
    assert qmse(mx, had=2) == INVALID
    assert qmse(mx, axis=2) == INVALID
    assert qmse(mx, iters=-1) == INVALID
    assert qmse(mx, iters=65) == INVALID
    assert qmse(mx, out="null") == INVALID
    assert qmse(mx, ldx=100) == INVALID
    assert qmse(mx, C=48, ldx=48) == SHAPE                     # MX block of 32
    assert qmse(mx, fmt=1, had=1, C=48, ldx=48) == SHAPE       # rotation needs k % 32
    assert qmse(mx, out=desc(mx, rows=63)) == INVALID          # descriptor disagrees with the call
    assert qmse(mx, x=None) == INVALID
    assert qmse(mx, out=desc(mx, codes=FAKE + 4)) == INVALID   # codes 16-byte aligned
    assert qmse(mx, fmt=1, out=desc(mx, 1, ts=None)) == INVALID
    assert qmse(mx, fmt=1, ws=None, wsb=0) == WORKSPACE
    assert qmse(mx, fmt=1, wsb=100) == WORKSPACE
    assert qmse(mx, R=0, out=desc(mx, rows=0)) == OK             # empty: no-op


def test_quantize_mse_workspace_bytes(mx):
    assert mx.mxfp4_quantize_mse_workspace_bytes("mx", False, 64, 256) == 0
    # NVFP4: amax partials (4096 bytes here), 16 bytes per 32-element unit (64 x 8), 16 per row
    assert mx.mxfp4_quantize_mse_workspace_bytes("nv", False, 64, 256) == 4096 + 64 * 8 * 16 + 64 * 16
    # units of 16 for NVFP4 without rotation on a contraction of 80
    assert mx.mxfp4_quantize_mse_workspace_bytes("nv", False, 10, 80) == 4096 + 10 * 5 * 16 + 10 * 16
    # axis 0: rows = C, k = R
    assert mx.mxfp4_quantize_mse_workspace_bytes("nv", True, 256, 64, 0) == 4096 + 64 * 8 * 16 + 64 * 16


def test_noise_ratio_is_the_sqrt3_test(mx):
    """mxfp4_noise_ratio: sqrt(signal / noise) against sqrt(3) ("FP4 All the
    Way", abstract), host arithmetic only."""
    assert mx.mxfp4_noise_ratio([12.0, 3.0, 0.0]) == (2.0, False)
    r, below = mx.mxfp4_noise_ratio([2.0, 1.0, 0.0])
    assert r == 2.0 ** 0.5 and below
    r, below = mx.mxfp4_noise_ratio([3.0, 1.0, 0.0])      # exactly sqrt(3): not below
    assert not below
    assert mx.mxfp4_noise_ratio([1.0, 0.0, 0.0]) == (float("inf"), False)
    d = ctypes.c_double()
    i = ctypes.c_int()
    bad = (ctypes.c_double * 3)(float("nan"), 1.0, 0.0)
    assert mx.lib.mxfp4_noise_ratio(bad, ctypes.byref(d), ctypes.byref(i)) == INVALID
    neg = (ctypes.c_double * 3)(1.0, -1.0, 0.0)
    assert mx.lib.mxfp4_noise_ratio(neg, ctypes.byref(d), ctypes.byref(i)) == INVALID
    assert mx.lib.mxfp4_noise_ratio(None, ctypes.byref(d), ctypes.byref(i)) == INVALID


def test_binding_rejects_outputs_the_kernels_would_overrun(mx):
    """The library cannot see buffer sizes, so the binding checks every output
    and operand buffer before anything is launched (all raises below happen
    on the host; no GPU is needed)."""
    import torch
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="2-D"):
        mx._check_out(torch.empty(4, 5, dtype=torch.bfloat16), (4, 5), torch.float32, dev)
    with pytest.raises(ValueError, match="shape"):
        mx._check_out(torch.empty(4, 4), (4, 5), torch.float32, dev)
    with pytest.raises(ValueError, match="stride"):
        mx._check_out(torch.empty(5, 4).t(), (4, 5), torch.float32, dev)
    with pytest.raises(ValueError, match="live on"):
        mx._check_out(torch.empty(4, 5), (4, 5), torch.float32, dev)
    qa = mx.empty_qtensor("mx", 64, 256, False, "cpu")
    qb = mx.empty_qtensor("mx", 32, 256, False, "cpu")
    with pytest.raises(ValueError, match="device"):
        mx.mxfp4_gemm(qa, qb)
    with pytest.raises(ValueError, match="device"):
        mx.mxfp4_dequantize(qa)
    short = mx.QTensor("mx", False, 64, 256, torch.empty(64 * 127, dtype=torch.uint8),
                       torch.empty(64 * 8, dtype=torch.uint8), None)
    with pytest.raises(ValueError, match="sizes"):
        mx._check_operands(short)
    nv = mx.QTensor("nv", False, 16, 64, torch.empty(16, 32, dtype=torch.uint8),
                    torch.empty(16, 4, dtype=torch.uint8), None)
    with pytest.raises(ValueError, match="tensor scale"):
        mx._check_operands(nv)
    with pytest.raises(ValueError, match="workspace"):
        mx._nbytes(torch.empty(16, dtype=torch.uint8), dev)


def test_qema_rejects_bad_arguments(mx):
    """mxfp4_qema_quantize: argument errors before any launch."""
    out = mx.MxTensorStruct(0, 0, 64, 256, FAKE, FAKE, None)
    f = mx.lib.mxfp4_qema_quantize
    ok = dict(w=FAKE, R=64, C=256, ldw=256, ema=FAKE, lde=256, beta=0.9, had=0)

    def call(**kw):
        a = dict(ok, **kw)
        o = kw.get("out", out)
        return f(ctypes.c_void_p(a["w"]) if a["w"] else None, a["R"], a["C"], a["ldw"],
                 ctypes.c_void_p(a["ema"]) if a["ema"] else None, a["lde"], a["beta"], a["had"], ctypes.byref(o), None)

    assert call(beta=1.5) == INVALID
    assert call(beta=float("nan")) == INVALID
    assert call(C=250, ldw=256, lde=256) == SHAPE
    assert call(ldw=200) == INVALID
    assert call(w=0) == INVALID
    assert call(ema=FAKE + 4) == INVALID
    assert call(ldw=260) == INVALID                       # not a multiple of 8
    assert call(had=1) == INVALID                          # out->hadamard differs
    assert call(out=mx.MxTensorStruct(1, 0, 64, 256, FAKE, FAKE, FAKE)) == INVALID   # NVFP4 out


def test_gemm_quantize_rejects_bad_arguments_and_sizes_its_workspace(mx):
    a = desc(mx, 0, 0, 512, 1024)
    b = desc(mx, 0, 0, 768, 1024)
    out = desc(mx, 0, 0, 512, 768)
    ws = ctypes.c_size_t()
    f = mx.lib.mxfp4_gemm_quantize
    fw = mx.lib.mxfp4_gemm_quantize_workspace_bytes
    assert fw(ctypes.byref(a), ctypes.byref(b), 0, ctypes.byref(out), ctypes.byref(ws)) == OK and ws.value == 0
    # a split contraction goes through a bf16 C in the workspace
    a2, b2, o2 = desc(mx, 0, 0, 64, 8192), desc(mx, 0, 0, 96, 8192), desc(mx, 0, 0, 64, 96)
    assert fw(ctypes.byref(a2), ctypes.byref(b2), 0, ctypes.byref(o2), ctypes.byref(ws)) == OK
    assert ws.value >= 64 * 96 * 2
    assert f(ctypes.byref(a2), ctypes.byref(b2), 0, ctypes.byref(o2), None, 0, None) == WORKSPACE
    nb = desc(mx, 0, 0, 100, 1024)                       # N not a multiple of 32
    assert f(ctypes.byref(a), ctypes.byref(nb), 0, ctypes.byref(desc(mx, 0, 0, 512, 100)), None, 0, None) == SHAPE
    assert f(ctypes.byref(a), ctypes.byref(b), 1, ctypes.byref(out), None, 0, None) == INVALID   # out->hadamard
    assert f(ctypes.byref(a), ctypes.byref(b), 0, ctypes.byref(desc(mx, 1, 0, 512, 768)), None, 0, None) == INVALID
    assert f(ctypes.byref(a), ctypes.byref(desc(mx, 1, 0, 768, 1024)), 0, ctypes.byref(out), None, 0, None) == MISMATCH


def test_quantize_grid_rejects_bad_arguments(mx):
    out = desc(mx, 0, 1, 64, 256)
    f = mx.lib.mxfp4_quantize_grid
    x = ctypes.c_void_p(FAKE)
    assert f(x, 64, 256, 256, 1, 1, ctypes.c_float(0.0), ctypes.byref(out), None) == INVALID
    assert f(x, 64, 256, 256, 1, 1, ctypes.c_float(float("nan")), ctypes.byref(out), None) == INVALID
    assert f(x, 64, 256, 256, 0, 1, ctypes.c_float(0.75), ctypes.byref(out), None) == INVALID     # hadamard differs
    assert f(x, 64, 240, 240, 1, 1, ctypes.c_float(0.75), ctypes.byref(desc(mx, 0, 1, 64, 240)), None) == SHAPE
    assert f(None, 64, 256, 256, 1, 1, ctypes.c_float(0.75), ctypes.byref(out), None) == INVALID
