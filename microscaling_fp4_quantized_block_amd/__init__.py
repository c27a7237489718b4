"""Python binding of libmxfp4 -- microscaling FP4 quantization and the
block-scaled FP4 GEMM on AMD Instinct MI355X (gfx950).

This module only marshals arguments: every step of the quantizer and the GEMM
runs in the HIP kernels of ``libmxfp4.so`` (built in-tree by
``microscaling_fp4_quantized_block_amd.build``).  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the library is
missing, importing the binding raises.

Entry points have the names of the C ABI (``include/mxfp4.h``):
``mxfp4_quantize``, ``mxfp4_dequantize``, ``mxfp4_gemm`` and the size and
workspace queries; ``quantize``, ``dequantize`` and ``gemm`` are aliases.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp4.so")

FMT = {"mx": 0, "nv": 1}
ROUNDING = {"rtn": 0, "sr": 1}
BLOCK = {"mx": 32, "nv": 16}

STATUS = {0: "MXFP4_OK", -1: "MXFP4_ERR_INVALID_ARG", -2: "MXFP4_ERR_UNSUPPORTED_SHAPE",
          -3: "MXFP4_ERR_FORMAT_MISMATCH", -4: "MXFP4_ERR_WORKSPACE", -5: "MXFP4_ERR_HIP"}


class MxTensorStruct(ctypes.Structure):
    """Mirror of the C struct mxfp4_tensor."""
    _fields_ = [("fmt", ctypes.c_int32), ("hadamard", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("k", ctypes.c_int64), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


def _load_library() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmxfp4.so not found at {LIB_PATH}; build it with "
            "`python microscaling_fp4_quantized_block_amd/build.py` (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, u64, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    lib.mxfp4_status_string.restype = ctypes.c_char_p
    lib.mxfp4_status_string.argtypes = [i32]
    lib.mxfp4_tensor_bytes.restype = i32
    lib.mxfp4_tensor_bytes.argtypes = [i32, i64, i64, P(sz), P(sz)]
    lib.mxfp4_quantize_workspace_bytes.restype = i32
    lib.mxfp4_quantize_workspace_bytes.argtypes = [i32, i64, i64, i32, P(sz)]
    lib.mxfp4_quantize.restype = i32
    lib.mxfp4_quantize.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, P(MxTensorStruct), vp, sz, vp]
    lib.mxfp4_dequantize.restype = i32
    lib.mxfp4_dequantize.argtypes = [P(MxTensorStruct), vp, i64, vp]
    lib.mxfp4_gemm_workspace_bytes.restype = i32
    lib.mxfp4_gemm_workspace_bytes.argtypes = [P(MxTensorStruct), P(MxTensorStruct), P(sz)]
    lib.mxfp4_gemm.restype = i32
    lib.mxfp4_gemm.argtypes = [P(MxTensorStruct), P(MxTensorStruct), vp, i64, vp, sz, vp]
    lib.mxfp4_gemm_bf16.restype = i32
    lib.mxfp4_gemm_bf16.argtypes = [P(MxTensorStruct), P(MxTensorStruct), vp, i64, vp, sz, vp]
    lib.mxfp4_quantize_gemm_workspace_bytes.restype = i32
    lib.mxfp4_quantize_gemm_workspace_bytes.argtypes = [i64, i64, i32, P(MxTensorStruct), P(sz)]
    lib.mxfp4_quantize_gemm.restype = i32
    lib.mxfp4_quantize_gemm.argtypes = [vp, i64, i64, i64, i32, P(MxTensorStruct), vp, i64, vp, sz, vp]
    lib.mxfp4_quantize_mse_workspace_bytes.restype = i32
    lib.mxfp4_quantize_mse_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, P(sz)]
    lib.mxfp4_quantize_mse.restype = i32
    lib.mxfp4_quantize_mse.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, P(MxTensorStruct), vp, sz, vp]
    lib.mxfp4_quantize_noise_workspace_bytes.restype = i32
    lib.mxfp4_quantize_noise_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, P(sz)]
    lib.mxfp4_quantize_noise.restype = i32
    lib.mxfp4_quantize_noise.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, P(MxTensorStruct), vp, vp, sz,
                                         vp]
    lib.mxfp4_quantization_noise_workspace_bytes.restype = i32
    lib.mxfp4_quantization_noise_workspace_bytes.argtypes = [P(MxTensorStruct), P(sz)]
    lib.mxfp4_quantization_noise.restype = i32
    lib.mxfp4_quantization_noise.argtypes = [vp, i64, i32, P(MxTensorStruct), vp, vp, sz, vp]
    return lib


lib = _load_library()


class MxFp4Error(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(mxfp4_status_string(status))


def mxfp4_status_string(status: int) -> str:
    return lib.mxfp4_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise MxFp4Error(status)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class QTensor:
    """A contraction-major quantized matrix [rows, k] (layout of mxfp4.h)."""
    fmt: str
    hadamard: bool
    rows: int
    k: int
    codes: torch.Tensor                  # uint8 [rows, k/2]
    scales: torch.Tensor                 # uint8 [rows, k/bs]
    tensor_scale: Optional[torch.Tensor]  # float32 [1] (NVFP4) or None

    def as_struct(self) -> MxTensorStruct:
        return MxTensorStruct(FMT[self.fmt], int(self.hadamard), self.rows, self.k,
                              self.codes.data_ptr() if self.codes.numel() else None,
                              self.scales.data_ptr() if self.scales.numel() else None,
                              self.tensor_scale.data_ptr() if self.tensor_scale is not None else None)


def mxfp4_tensor_bytes(fmt: str, rows: int, k: int):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.mxfp4_tensor_bytes(FMT[fmt], rows, k, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def mxfp4_quantize_workspace_bytes(fmt: str, R: int, C: int, axis: int = 1) -> int:
    b = ctypes.c_size_t()
    _check(lib.mxfp4_quantize_workspace_bytes(FMT[fmt], R, C, axis, ctypes.byref(b)))
    return b.value


def empty_qtensor(fmt: str, rows: int, k: int, hadamard: bool, device) -> QTensor:
    cb, sb = mxfp4_tensor_bytes(fmt, rows, k)
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, k // BLOCK[fmt]), dtype=torch.uint8, device=device)
    assert codes.numel() == cb and scales.numel() == sb
    ts = torch.empty(1, dtype=torch.float32, device=device) if fmt == "nv" else None
    return QTensor(fmt, bool(hadamard), rows, k, codes, scales, ts)


def mxfp4_quantize(x: torch.Tensor, fmt: str = "mx", rounding: str = "rtn", hadamard: bool = False,
                   axis: int = 1, seed: int = 0, out: Optional[QTensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> QTensor:
    """Quantize a bf16 [R, C] device tensor (row stride may exceed C).

    axis=1 quantizes along C (result [R, C]); axis=0 along R (result [C, R]).
    """
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 CUDA/HIP tensor")
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its last dimension")
    R, C = x.shape
    rows, k = (R, C) if axis == 1 else (C, R)
    if out is None:
        out = empty_qtensor(fmt, rows, k, hadamard, x.device)
    ws_bytes = mxfp4_quantize_workspace_bytes(fmt, R, C, axis)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = out.as_struct()
    _check(lib.mxfp4_quantize(_ptr(x), R, C, x.stride(0), FMT[fmt], ROUNDING[rounding], int(bool(hadamard)),
                              int(axis), int(seed) & (2 ** 64 - 1), ctypes.byref(st), _ptr(workspace),
                              workspace.numel() if workspace is not None else 0, _stream(x.device)))
    return out


def mxfp4_dequantize(q: QTensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((q.rows, q.k), dtype=torch.float32, device=q.codes.device)
    st = q.as_struct()
    _check(lib.mxfp4_dequantize(ctypes.byref(st), _ptr(out), out.stride(0) if out.dim() == 2 else q.k,
                                _stream(q.codes.device)))
    return out


def mxfp4_gemm_workspace_bytes(qa: QTensor, qb: QTensor) -> int:
    b = ctypes.c_size_t()
    sa, sb = qa.as_struct(), qb.as_struct()
    _check(lib.mxfp4_gemm_workspace_bytes(ctypes.byref(sa), ctypes.byref(sb), ctypes.byref(b)))
    return b.value


def mxfp4_gemm(qa: QTensor, qb: QTensor, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M, N] = A B^T in FP32 over the dequantized operands."""
    if out is None:
        out = torch.empty((qa.rows, qb.rows), dtype=torch.float32, device=qa.codes.device)
    ws_bytes = mxfp4_gemm_workspace_bytes(qa, qb)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=qa.codes.device)
    sa, sb = qa.as_struct(), qb.as_struct()
    _check(lib.mxfp4_gemm(ctypes.byref(sa), ctypes.byref(sb), _ptr(out), out.stride(0), _ptr(workspace),
                          workspace.numel() if workspace is not None else 0, _stream(qa.codes.device)))
    return out


def mxfp4_gemm_bf16(qa: QTensor, qb: QTensor, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M, N] = A B^T as mxfp4_gemm computes it, rounded to bfloat16 (nearest
    even)."""
    if out is None:
        out = torch.empty((qa.rows, qb.rows), dtype=torch.bfloat16, device=qa.codes.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or (out.numel() and out.stride(1) != 1):
        raise ValueError("out must be a 2-D bfloat16 tensor with unit stride along its last dimension")
    ws_bytes = mxfp4_gemm_workspace_bytes(qa, qb)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=qa.codes.device)
    sa, sb = qa.as_struct(), qb.as_struct()
    _check(lib.mxfp4_gemm_bf16(ctypes.byref(sa), ctypes.byref(sb), _ptr(out), out.stride(0), _ptr(workspace),
                               workspace.numel() if workspace is not None else 0, _stream(qa.codes.device)))
    return out


def mxfp4_quantize_gemm_workspace_bytes(M: int, K: int, hadamard: bool, qb: QTensor) -> int:
    b = ctypes.c_size_t()
    sb = qb.as_struct()
    _check(lib.mxfp4_quantize_gemm_workspace_bytes(M, K, int(bool(hadamard)), ctypes.byref(sb), ctypes.byref(b)))
    return b.value


def mxfp4_quantize_gemm(x: torch.Tensor, qb: QTensor, hadamard: bool = False, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M, N] = Q(x) B^T with x [M, K] bf16 quantized on the fly (MXFP4,
    round-to-nearest, optional block Hadamard), the same bits as
    mxfp4_gemm(mxfp4_quantize(x, "mx", "rtn", hadamard), qb)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 CUDA/HIP tensor")
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its last dimension")
    M, K = x.shape
    if out is None:
        out = torch.empty((M, qb.rows), dtype=torch.float32, device=x.device)
    ws_bytes = mxfp4_quantize_gemm_workspace_bytes(M, K, hadamard, qb)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    sb = qb.as_struct()
    _check(lib.mxfp4_quantize_gemm(_ptr(x), M, K, x.stride(0), int(bool(hadamard)), ctypes.byref(sb), _ptr(out),
                                   out.stride(0), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                   _stream(x.device)))
    return out


def mxfp4_quantize_mse_workspace_bytes(fmt: str, hadamard: bool, R: int, C: int, axis: int = 1) -> int:
    b = ctypes.c_size_t()
    _check(lib.mxfp4_quantize_mse_workspace_bytes(FMT[fmt], int(bool(hadamard)), R, C, axis, ctypes.byref(b)))
    return b.value


def mxfp4_quantize_mse(x: torch.Tensor, fmt: str = "nv", hadamard: bool = False, axis: int = 1, iters: int = 2,
                       out: Optional[QTensor] = None, workspace: Optional[torch.Tensor] = None) -> QTensor:
    """Round-to-nearest quantization with MSE-fitted block scales (and, for
    NVFP4, a least-squares tensor scale, alternating iters times)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 CUDA/HIP tensor with unit stride along its last dimension")
    R, C = x.shape
    rows, k = (R, C) if axis == 1 else (C, R)
    if out is None:
        out = empty_qtensor(fmt, rows, k, hadamard, x.device)
    ws_bytes = mxfp4_quantize_mse_workspace_bytes(fmt, hadamard, R, C, axis)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = out.as_struct()
    _check(lib.mxfp4_quantize_mse(_ptr(x), R, C, x.stride(0), FMT[fmt], int(bool(hadamard)), int(axis), int(iters),
                                  ctypes.byref(st), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                  _stream(x.device)))
    return out


def mxfp4_quantization_noise_workspace_bytes(q: QTensor) -> int:
    b = ctypes.c_size_t()
    sq = q.as_struct()
    _check(lib.mxfp4_quantization_noise_workspace_bytes(ctypes.byref(sq), ctypes.byref(b)))
    return b.value


def mxfp4_quantization_noise(x: torch.Tensor, q: QTensor, axis: int = 1, out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device float64 [3]: sum y^2, sum (Q(y) - y)^2 and the number of
    elements left out (NaN blocks), y the elements of q's operand (x's
    contraction rows, rotated when q is), Q(y) their dequantized values."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 CUDA/HIP tensor with unit stride along its last dimension")
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=x.device)
    ws_bytes = mxfp4_quantization_noise_workspace_bytes(q)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    sq = q.as_struct()
    _check(lib.mxfp4_quantization_noise(_ptr(x), x.stride(0), int(axis), ctypes.byref(sq), _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out


def mxfp4_quantize_noise_workspace_bytes(fmt: str, hadamard: bool, R: int, C: int, axis: int = 1) -> int:
    b = ctypes.c_size_t()
    _check(lib.mxfp4_quantize_noise_workspace_bytes(FMT[fmt], int(bool(hadamard)), R, C, axis, ctypes.byref(b)))
    return b.value


def mxfp4_quantize_noise(x: torch.Tensor, fmt: str = "mx", rounding: str = "sr", hadamard: bool = False,
                         axis: int = 1, seed: int = 0, out: Optional[QTensor] = None,
                         stats: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """(q, stats): mxfp4_quantize(x, ...) and, from the same pass, the float64
    [3] sums of mxfp4_quantization_noise (sum y^2, sum (Q(y) - y)^2, elements
    left out)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 CUDA/HIP tensor with unit stride along its last dimension")
    R, C = x.shape
    rows, k = (R, C) if axis == 1 else (C, R)
    if out is None:
        out = empty_qtensor(fmt, rows, k, hadamard, x.device)
    if stats is None:
        stats = torch.empty(3, dtype=torch.float64, device=x.device)
    ws_bytes = mxfp4_quantize_noise_workspace_bytes(fmt, hadamard, R, C, axis)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = out.as_struct()
    _check(lib.mxfp4_quantize_noise(_ptr(x), R, C, x.stride(0), FMT[fmt], ROUNDING[rounding], int(bool(hadamard)),
                                    int(axis), int(seed) & (2 ** 64 - 1), ctypes.byref(st), _ptr(stats),
                                    _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out, stats


def gradient_noise_ratio(x: torch.Tensor, q: QTensor, axis: int = 1):
    """(ratio, below): ratio = ||y|| / ||Q(y) - y|| for the quantized operand,
    and whether it falls below sqrt(3), the threshold under which quantized
    training loses effectiveness ("FP4 All the Way", abstract)."""
    s = mxfp4_quantization_noise(x, q, axis).cpu().tolist()
    ratio = float("inf") if s[1] == 0.0 else (s[0] / s[1]) ** 0.5
    return ratio, ratio < 3.0 ** 0.5


quantize = mxfp4_quantize
dequantize = mxfp4_dequantize
gemm = mxfp4_gemm
quantize_gemm = mxfp4_quantize_gemm

__all__ = ["QTensor", "MxFp4Error", "mxfp4_tensor_bytes", "mxfp4_quantize_workspace_bytes", "mxfp4_quantize",
           "mxfp4_dequantize", "mxfp4_gemm_workspace_bytes", "mxfp4_gemm", "mxfp4_gemm_bf16", "mxfp4_status_string",
           "mxfp4_quantize_gemm_workspace_bytes", "mxfp4_quantize_gemm",
           "mxfp4_quantization_noise_workspace_bytes", "mxfp4_quantization_noise", "gradient_noise_ratio",
           "mxfp4_quantize_noise_workspace_bytes", "mxfp4_quantize_noise",
           "mxfp4_quantize_mse_workspace_bytes", "mxfp4_quantize_mse",
           "quantize", "dequantize", "gemm", "quantize_gemm", "empty_qtensor", "lib", "LIB_PATH"]
