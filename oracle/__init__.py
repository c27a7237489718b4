"""CPU oracle for microscaling FP4 quantization and the block-scaled FP4 GEMM.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library never imports,
links or calls it, and it shares no code with the HIP library.

The arithmetic lives in ``mxfp4_oracle.c`` (plain scalar C, binary32 for the
steps that decide codes, binary64 for the GEMM); this module only builds it
and marshals numpy arrays through ctypes.  See the C file's header for the
pages each step follows and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmxfp4_oracle.so")

FMT = {"mx": 0, "nv": 1}
ROUNDING = {"rtn": 0, "sr": 1}
BLOCK = {"mx": 32, "nv": 16}

_lib = None


def build() -> str:
    """Compile the oracle (always; a few seconds)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-std=c11", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, u64, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p
    lib.mxo_e2m1_value.restype = ctypes.c_double
    lib.mxo_e2m1_value.argtypes = [i32]
    lib.mxo_e8m0_value.restype = ctypes.c_double
    lib.mxo_e8m0_value.argtypes = [i32]
    lib.mxo_e4m3_value.restype = ctypes.c_double
    lib.mxo_e4m3_value.argtypes = [i32]
    lib.mxo_e4m3_round_up.restype = i32
    lib.mxo_e4m3_round_up.argtypes = [ctypes.c_float]
    lib.mxo_mx_scale_exponent.restype = i32
    lib.mxo_mx_scale_exponent.argtypes = [ctypes.c_float]
    lib.mxo_rtn_code.restype = i32
    lib.mxo_rtn_code.argtypes = [ctypes.c_double]
    lib.mxo_sr_code.restype = i32
    lib.mxo_sr_code.argtypes = [ctypes.c_double, ctypes.c_uint32]
    lib.mxo_philox4x32_10.restype = None
    lib.mxo_philox4x32_10.argtypes = [vp, vp, vp]
    lib.mxo_rnd16.restype = ctypes.c_uint32
    lib.mxo_rnd16.argtypes = [u64, u64, i32]
    lib.mxo_hadamard_scale.restype = ctypes.c_float
    lib.mxo_hadamard_scale.argtypes = []
    lib.mxo_fwht32.restype = None
    lib.mxo_fwht32.argtypes = [vp]
    lib.mxo_nv_tensor_scale.restype = ctypes.c_float
    lib.mxo_nv_tensor_scale.argtypes = [ctypes.c_float]
    lib.mxo_quantize.restype = i32
    lib.mxo_quantize.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, vp, vp, vp]
    lib.mxo_quantize_rows_at.restype = i32
    lib.mxo_quantize_rows_at.argtypes = [vp, i64, i64, i64, i32, i32, u64, i64, vp, vp]
    lib.mxo_dequantize.restype = i32
    lib.mxo_dequantize.argtypes = [i32, i64, i64, vp, vp, vp, vp, i64]
    lib.mxo_gemm.restype = i32
    lib.mxo_gemm.argtypes = [i32, i64, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64, vp, vp]
    lib.mxo_quantize_mse.restype = i32
    lib.mxo_quantize_mse.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, vp, vp, vp]
    lib.mxo_mse_check.restype = i32
    lib.mxo_mse_check.argtypes = [vp, i64, i64, i64, i32, i32, i32, ctypes.c_float, vp, vp, ctypes.c_double, vp]
    lib.mxo_mse_tensor_step.restype = i32
    lib.mxo_mse_tensor_step.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp, ctypes.c_float, vp]
    lib.mxo_quantize_f32.restype = i32
    lib.mxo_quantize_f32.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, vp, vp, vp]
    lib.mxo_qema_quantize.restype = i32
    lib.mxo_qema_quantize.argtypes = [vp, i64, i64, i64, vp, i64, ctypes.c_float, i32, vp, vp]
    lib.mxo_quantize_grid.restype = i32
    lib.mxo_quantize_grid.argtypes = [vp, i64, i64, i64, i32, i32, ctypes.c_float, vp, vp]
    lib.mxo_noise_stats.restype = i32
    lib.mxo_noise_stats.argtypes = [vp, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---- scalar pieces (exposed for the pins) ----------------------------------
def e2m1_value(code: int) -> float:
    return _load().mxo_e2m1_value(int(code))


def e8m0_value(byte: int) -> float:
    return _load().mxo_e8m0_value(int(byte))


def e4m3_value(byte: int) -> float:
    return _load().mxo_e4m3_value(int(byte))


def e4m3_round_up(r: float) -> int:
    return _load().mxo_e4m3_round_up(float(r))


def mx_scale_exponent(amax: float) -> int:
    return _load().mxo_mx_scale_exponent(float(amax))


def rtn_code(xs: float) -> int:
    return _load().mxo_rtn_code(float(xs))


def sr_code(xs: float, rnd16: int) -> int:
    return _load().mxo_sr_code(float(xs), int(rnd16))


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _load().mxo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def rnd16(seed: int, L: int, axis: int) -> int:
    return _load().mxo_rnd16(int(seed), int(L), int(axis))


def hadamard_scale() -> float:
    return _load().mxo_hadamard_scale()


def fwht32(x) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).copy()
    assert v.shape == (32,)
    _load().mxo_fwht32(_ptr(v))
    return v


def nv_tensor_scale(amax_t: float) -> float:
    return _load().mxo_nv_tensor_scale(float(amax_t))


# ---- tensor-level entry points ---------------------------------------------
def quantize(x_bits: np.ndarray, fmt: str = "mx", rounding: str = "rtn",
             hadamard: bool = False, axis: int = 1, seed: int = 0):
    """Quantize a [R, C] bf16 tensor given as its uint16 bit patterns.

    Returns (codes [rows, K/2] uint8, scales [rows, K/bs] uint8, tensor_scale
    float or None), with (rows, K) = (R, C) for axis 1 and (C, R) for axis 0.
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    rows, K = (R, C) if axis == 1 else (C, R)
    bs = BLOCK[fmt]
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // bs), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32) if fmt == "nv" else None
    rc = _load().mxo_quantize(_ptr(x), R, C, C, FMT[fmt], ROUNDING[rounding], int(bool(hadamard)),
                              int(axis), int(seed), _ptr(codes), _ptr(scales), _ptr(ts))
    if rc != 0:
        raise ValueError("oracle quantize rejected its arguments")
    return codes, scales, (float(ts[0]) if ts is not None else None)


def quantize_rows_at(x_bits: np.ndarray, row0: int, rounding: str = "rtn", hadamard: bool = False, seed: int = 0):
    """MXFP4 along axis 1 for rows row0 .. of a larger tensor (given as those
    rows only): the same codes and scales the whole tensor's quantization
    has there.  Returns (codes, scales)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    codes = np.zeros((R, C // 2), dtype=np.uint8)
    scales = np.zeros((R, C // 32), dtype=np.uint8)
    rc = _load().mxo_quantize_rows_at(_ptr(x), R, C, C, ROUNDING[rounding], int(bool(hadamard)), int(seed),
                                      int(row0), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle quantize_rows_at rejected its arguments")
    return codes, scales


def dequantize(fmt: str, codes: np.ndarray, scales: np.ndarray, tensor_scale=None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    ts = np.array([tensor_scale if tensor_scale is not None else 1.0], dtype=np.float32)
    y = np.zeros((rows, K), dtype=np.float32)
    rc = _load().mxo_dequantize(FMT[fmt], rows, K, _ptr(codes), _ptr(scales), _ptr(ts), _ptr(y), K)
    if rc != 0:
        raise ValueError("oracle dequantize rejected its arguments")
    return y


def gemm(fmt: str, a, b, rows=None, cols=None):
    """C = A B^T in binary64 over the exactly dequantized operands.

    a, b: (codes, scales, tensor_scale) as returned by quantize().  rows / cols
    select a sub-matrix (default: all).  Returns (C, S) float64 arrays of shape
    [len(rows), len(cols)], S = sum_k |a_ik b_jk|.
    """
    ac, asc, ats = a
    bc, bsc, bts = b
    ac = np.ascontiguousarray(ac, dtype=np.uint8)
    bc = np.ascontiguousarray(bc, dtype=np.uint8)
    asc = np.ascontiguousarray(asc, dtype=np.uint8)
    bsc = np.ascontiguousarray(bsc, dtype=np.uint8)
    K = ac.shape[1] * 2
    assert bc.shape[1] * 2 == K
    ri = np.arange(ac.shape[0], dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    cj = np.arange(bc.shape[0], dtype=np.int64) if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    ta = np.array([ats if ats is not None else 1.0], dtype=np.float32)
    tb = np.array([bts if bts is not None else 1.0], dtype=np.float32)
    Cm = np.zeros((len(ri), len(cj)), dtype=np.float64)
    Sm = np.zeros((len(ri), len(cj)), dtype=np.float64)
    rc = _load().mxo_gemm(FMT[fmt], K, _ptr(ac), _ptr(asc), _ptr(ta), _ptr(bc), _ptr(bsc), _ptr(tb),
                          _ptr(ri), len(ri), _ptr(cj), len(cj), _ptr(Cm), _ptr(Sm))
    if rc != 0:
        raise ValueError("oracle gemm rejected its arguments")
    return Cm, Sm


def noise_stats(x_bits: np.ndarray, q, fmt: str = "mx", hadamard: bool = False, axis: int = 1):
    """Signal and quantization noise of a quantized operand (the quantities of
    the sqrt(3) threshold of "FP4 All the Way", abstract).

    x_bits: the [R, C] bf16 input (uint16 patterns); q = (codes, scales,
    tensor_scale) its quantization with this fmt / hadamard / axis.  Returns
    (sum y^2, sum (Q(y) - y)^2, elements left out) in binary64, y = the
    contraction rows (rotated when hadamard), Q(y) the exactly dequantized
    value; blocks with a NaN scale byte are left out.
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    codes = np.ascontiguousarray(q[0], dtype=np.uint8)
    scales = np.ascontiguousarray(q[1], dtype=np.uint8)
    ts = np.array([q[2] if q[2] is not None else 1.0], dtype=np.float32)
    out = np.zeros(3, dtype=np.float64)
    rc = _load().mxo_noise_stats(_ptr(x), R, C, C, FMT[fmt], int(bool(hadamard)), int(axis), _ptr(codes),
                                 _ptr(scales), _ptr(ts), _ptr(out))
    if rc != 0:
        raise ValueError("oracle noise_stats rejected its arguments")
    return float(out[0]), float(out[1]), float(out[2])


def quantize_mse(x_bits: np.ndarray, fmt: str = "nv", hadamard: bool = False, axis: int = 1, iters: int = 2):
    """Round-to-nearest quantization with MSE-fitted scales (the digest of the
    MR-GPTQ paper, step 1): each block keeps the scale at or below its absmax
    scale with the smallest squared error, alternating with the least-squares
    tensor scale (NVFP4) `iters` times.  Same return value as quantize()."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    rows, K = (R, C) if axis == 1 else (C, R)
    bs = BLOCK[fmt]
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // bs), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32) if fmt == "nv" else None
    rc = _load().mxo_quantize_mse(_ptr(x), R, C, C, FMT[fmt], int(bool(hadamard)), int(axis), int(iters),
                                  _ptr(codes), _ptr(scales), _ptr(ts))
    if rc != 0:
        raise ValueError("oracle quantize_mse rejected its arguments")
    return codes, scales, (float(ts[0]) if ts is not None else None)


def mse_check(x_bits: np.ndarray, q, fmt: str, hadamard: bool = False, axis: int = 1, st=None,
              rel_tol: float = 0.0) -> dict:
    """Check that q = (codes, scales, tensor_scale) is a block step of the MSE
    quantizer for x under tensor scale st (default: q's own; ignored for MX):
    every block's byte is a candidate, its codes are the round-to-nearest
    encoding for that byte, and its squared error is within (1 + rel_tol) of
    the smallest over all candidates.  Returns the counts of the C checker."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    codes = np.ascontiguousarray(q[0], dtype=np.uint8)
    scales = np.ascontiguousarray(q[1], dtype=np.uint8)
    if st is None:
        st = q[2] if q[2] is not None else 1.0
    out = np.zeros(5, dtype=np.int64)
    rc = _load().mxo_mse_check(_ptr(x), R, C, C, FMT[fmt], int(bool(hadamard)), int(axis), float(st), _ptr(codes),
                               _ptr(scales), float(rel_tol), _ptr(out))
    if rc != 0:
        raise ValueError("oracle mse_check rejected its arguments")
    return {"blocks": int(out[0]), "bad_encoding": int(out[1]), "bad_error": int(out[2]),
            "differ_from_oracle": int(out[3]), "first_bad": int(out[4])}


def mse_tensor_step(x_bits: np.ndarray, q, hadamard: bool = False, axis: int = 1, st_prev: float = 1.0) -> float:
    """The least-squares NVFP4 tensor scale for the bytes and codes of q (a
    quantization of x), as a binary32 value; st_prev if sum(y p) <= 0."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    codes = np.ascontiguousarray(q[0], dtype=np.uint8)
    scales = np.ascontiguousarray(q[1], dtype=np.uint8)
    out = np.zeros(1, dtype=np.float32)
    rc = _load().mxo_mse_tensor_step(_ptr(x), R, C, C, int(bool(hadamard)), int(axis), _ptr(codes), _ptr(scales),
                                     float(st_prev), _ptr(out))
    if rc != 0:
        raise ValueError("oracle mse_tensor_step rejected its arguments")
    return float(out[0])


def quantize_f32(x: np.ndarray, fmt: str = "mx", rounding: str = "rtn", hadamard: bool = False, axis: int = 1,
                 seed: int = 0):
    """quantize() on a binary32 [R, C] input (values used as they are)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    rows, K = (R, C) if axis == 1 else (C, R)
    bs = BLOCK[fmt]
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // bs), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32) if fmt == "nv" else None
    rc = _load().mxo_quantize_f32(_ptr(x), R, C, C, FMT[fmt], ROUNDING[rounding], int(bool(hadamard)), int(axis),
                                  int(seed), _ptr(codes), _ptr(scales), _ptr(ts))
    if rc != 0:
        raise ValueError("oracle quantize_f32 rejected its arguments")
    return codes, scales, (float(ts[0]) if ts is not None else None)


def qema_quantize(w_bits: np.ndarray, ema: np.ndarray, beta: float, hadamard: bool = False):
    """Q-EMA step (reading, parity unpinned as to the method): ema <- RN(RN(beta
    ema) + RN((1 - beta) w)) in binary32, then MXFP4 round-to-nearest of the
    updated ema along its rows.  Returns (new ema, (codes, scales, None))."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    m = np.ascontiguousarray(ema, dtype=np.float32).copy()
    R, C = w.shape
    assert m.shape == (R, C)
    codes = np.zeros((R, C // 2), dtype=np.uint8)
    scales = np.zeros((R, C // 32), dtype=np.uint8)
    rc = _load().mxo_qema_quantize(_ptr(w), R, C, C, _ptr(m), C, float(beta), int(bool(hadamard)), _ptr(codes),
                                   _ptr(scales))
    if rc != 0:
        raise ValueError("oracle qema_quantize rejected its arguments")
    return m, (codes, scales, None)


def quantize_grid(x_bits: np.ndarray, alpha: float, hadamard: bool = True, axis: int = 1):
    """MXFP4 round-to-nearest with a fixed grid scale alpha: each block's E8M0
    exponent chosen for RN(alpha * absmax) (reading of the digest of the
    MR-GPTQ paper, step 1).  Returns (codes, scales, None)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    rows, K = (R, C) if axis == 1 else (C, R)
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // 32), dtype=np.uint8)
    rc = _load().mxo_quantize_grid(_ptr(x), R, C, C, int(bool(hadamard)), int(axis), float(alpha), _ptr(codes),
                                   _ptr(scales))
    if rc != 0:
        raise ValueError("oracle quantize_grid rejected its arguments")
    return codes, scales, None
