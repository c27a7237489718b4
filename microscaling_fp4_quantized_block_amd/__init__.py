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
    lib.mxfp4_quantize_noalloc.restype = i32
    lib.mxfp4_quantize_noalloc.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, u64, P(MxTensorStruct), vp]
    lib.mxfp4_qema_quantize.restype = i32
    lib.mxfp4_qema_quantize.argtypes = [vp, i64, i64, i64, vp, i64, ctypes.c_float, i32, P(MxTensorStruct), vp]
    lib.mxfp4_quantize_grid.restype = i32
    lib.mxfp4_quantize_grid.argtypes = [vp, i64, i64, i64, i32, i32, ctypes.c_float, P(MxTensorStruct), vp]
    lib.mxfp4_dequantize.restype = i32
    lib.mxfp4_dequantize.argtypes = [P(MxTensorStruct), vp, i64, vp]
    lib.mxfp4_gemm_workspace_bytes.restype = i32
    lib.mxfp4_gemm_workspace_bytes.argtypes = [P(MxTensorStruct), P(MxTensorStruct), P(sz)]
    lib.mxfp4_gemm.restype = i32
    lib.mxfp4_gemm.argtypes = [P(MxTensorStruct), P(MxTensorStruct), vp, i64, vp, sz, vp]
    lib.mxfp4_gemm_bf16.restype = i32
    lib.mxfp4_gemm_bf16.argtypes = [P(MxTensorStruct), P(MxTensorStruct), vp, i64, vp, sz, vp]
    lib.mxfp4_gemm_quantize_workspace_bytes.restype = i32
    lib.mxfp4_gemm_quantize_workspace_bytes.argtypes = [P(MxTensorStruct), P(MxTensorStruct), i32, P(MxTensorStruct),
                                                        P(sz)]
    lib.mxfp4_gemm_quantize.restype = i32
    lib.mxfp4_gemm_quantize.argtypes = [P(MxTensorStruct), P(MxTensorStruct), i32, P(MxTensorStruct), vp, sz, vp]
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
    lib.mxfp4_noise_ratio.restype = i32
    lib.mxfp4_noise_ratio.argtypes = [P(ctypes.c_double), P(ctypes.c_double), P(i32)]
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


def _check_operands(*qs: "QTensor") -> torch.device:
    """Quantized tensors must live on one GPU device, in contiguous buffers of
    exactly the sizes their rows and k call for (the library reads and writes
    that many bytes); returns the device."""
    dev = qs[0].codes.device
    for q in qs:
        if q.fmt not in FMT or q.rows < 0 or q.k < 0 or q.k % BLOCK[q.fmt]:
            raise ValueError("quantized tensor with a bad format or shape")
        if q.codes.dtype != torch.uint8 or q.scales.dtype != torch.uint8:
            raise ValueError("codes and scales must be uint8 tensors")
        if q.codes.numel() != q.rows * (q.k // 2) or q.scales.numel() != q.rows * (q.k // BLOCK[q.fmt]):
            raise ValueError("codes / scales sizes do not match the quantized tensor's rows and k")
        if not q.codes.is_contiguous() or not q.scales.is_contiguous():
            raise ValueError("codes and scales must be contiguous")
        if q.fmt == "nv" and (q.tensor_scale is None or q.tensor_scale.dtype != torch.float32
                              or q.tensor_scale.numel() < 1):
            raise ValueError("an NVFP4 tensor needs a float32 tensor scale")
        for t in (q.codes, q.scales) + ((q.tensor_scale,) if q.tensor_scale is not None else ()):
            if not t.is_cuda or t.device != dev:
                raise ValueError("quantized tensors must live on one CUDA/HIP device")
    return dev


def _nbytes(workspace: Optional[torch.Tensor], device) -> int:
    """Byte size of a caller's workspace (0 for none); it must be contiguous
    and on the call's device."""
    if workspace is None:
        return 0
    if not workspace.is_contiguous() or not workspace.is_cuda or workspace.device != torch.device(device):
        raise ValueError("workspace must be a contiguous tensor on the call's device")
    return workspace.numel() * workspace.element_size()


def _check_out(out: torch.Tensor, shape, dtype, device: torch.device, name: str = "out") -> None:
    """The library cannot see buffer sizes: an output must be a 2-D tensor of
    exactly this shape and dtype on this device, with unit stride along its
    last dimension (any row stride >= its width), or the kernels would write
    past it."""
    if not isinstance(out, torch.Tensor) or out.dtype != dtype or out.dim() != 2:
        raise ValueError(f"{name} must be a 2-D {dtype} tensor")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if out.numel() and out.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    if not out.is_cuda or out.device != device:
        raise ValueError(f"{name} must live on {device}")


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
    if _check_operands(out) != x.device:
        raise ValueError("out must live on x's device")
    ws_bytes = mxfp4_quantize_workspace_bytes(fmt, R, C, axis)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = out.as_struct()
    _check(lib.mxfp4_quantize(_ptr(x), R, C, x.stride(0), FMT[fmt], ROUNDING[rounding], int(bool(hadamard)),
                              int(axis), int(seed) & (2 ** 64 - 1), ctypes.byref(st), _ptr(workspace),
                              _nbytes(workspace, x.device), _stream(x.device)))
    return out


def mxfp4_quantize_noalloc(x: torch.Tensor, out: QTensor, fmt: str = "mx", rounding: str = "rtn",
                           hadamard: bool = False, axis: int = 1, seed: int = 0) -> QTensor:
    """mxfp4_quantize into a caller-allocated out, with no workspace: the
    library's entry point for callers that cannot allocate (the NVFP4 amax
    partials live in a static 1 MiB device array; overlapping calls on one
    device race on it)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 CUDA/HIP tensor with unit stride along its last dimension")
    R, C = x.shape
    rows, k = (R, C) if axis == 1 else (C, R)
    if _check_operands(out) != x.device or (out.rows, out.k, out.fmt) != (rows, k, fmt):
        raise ValueError("out must match the call (rows, k, fmt) and live on x's device")
    st = out.as_struct()
    _check(lib.mxfp4_quantize_noalloc(_ptr(x), R, C, x.stride(0), FMT[fmt], ROUNDING[rounding], int(bool(hadamard)),
                                      int(axis), int(seed) & (2 ** 64 - 1), ctypes.byref(st), _stream(x.device)))
    return out


def mxfp4_qema_quantize(w: torch.Tensor, ema: torch.Tensor, beta: float, hadamard: bool = False,
                        out: Optional[QTensor] = None) -> QTensor:
    """Q-EMA step: ema <- beta ema + (1 - beta) w (binary32, updated in place),
    then the MXFP4 round-to-nearest quantization of the new ema along its rows
    (block Hadamard first if asked), in one pass."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_cuda or w.stride(1) != 1:
        raise ValueError("w must be a 2-D bfloat16 CUDA/HIP tensor with unit stride along its last dimension")
    R, C = w.shape
    if ema.dtype != torch.float32 or tuple(ema.shape) != (R, C) or ema.stride(1) != 1 or ema.device != w.device:
        raise ValueError("ema must be a float32 tensor of w's shape on w's device, unit stride along its last dimension")
    if out is None:
        out = empty_qtensor("mx", R, C, hadamard, w.device)
    if _check_operands(out) != w.device or (out.fmt, out.rows, out.k) != ("mx", R, C):
        raise ValueError("out must be an MXFP4 tensor [R, C] on w's device")
    st = out.as_struct()
    _check(lib.mxfp4_qema_quantize(_ptr(w), R, C, max(w.stride(0), C), _ptr(ema), max(ema.stride(0), C), float(beta),
                                   int(bool(hadamard)), ctypes.byref(st), _stream(w.device)))
    return out


def mxfp4_quantize_grid(x: torch.Tensor, alpha: float, hadamard: bool = True, axis: int = 1,
                        out: Optional[QTensor] = None) -> QTensor:
    """MXFP4 round-to-nearest with a fixed grid scale alpha (each block's
    exponent chosen for RN(alpha * absmax)); alpha = 1 is mxfp4_quantize."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 CUDA/HIP tensor with unit stride along its last dimension")
    R, C = x.shape
    rows, k = (R, C) if axis == 1 else (C, R)
    if out is None:
        out = empty_qtensor("mx", rows, k, hadamard, x.device)
    if _check_operands(out) != x.device or (out.fmt, out.rows, out.k) != ("mx", rows, k):
        raise ValueError("out must be an MXFP4 tensor of the call's shape on x's device")
    st = out.as_struct()
    _check(lib.mxfp4_quantize_grid(_ptr(x), R, C, x.stride(0), int(bool(hadamard)), int(axis), float(alpha),
                                   ctypes.byref(st), _stream(x.device)))
    return out


def mxfp4_dequantize(q: QTensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dev = _check_operands(q)
    if out is None:
        out = torch.empty((q.rows, q.k), dtype=torch.float32, device=dev)
    _check_out(out, (q.rows, q.k), torch.float32, dev)
    st = q.as_struct()
    _check(lib.mxfp4_dequantize(ctypes.byref(st), _ptr(out), max(out.stride(0), q.k), _stream(dev)))
    return out


def mxfp4_gemm_workspace_bytes(qa: QTensor, qb: QTensor) -> int:
    b = ctypes.c_size_t()
    sa, sb = qa.as_struct(), qb.as_struct()
    _check(lib.mxfp4_gemm_workspace_bytes(ctypes.byref(sa), ctypes.byref(sb), ctypes.byref(b)))
    return b.value


def mxfp4_gemm(qa: QTensor, qb: QTensor, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M, N] = A B^T in FP32 over the dequantized operands."""
    dev = _check_operands(qa, qb)
    if out is None:
        out = torch.empty((qa.rows, qb.rows), dtype=torch.float32, device=dev)
    _check_out(out, (qa.rows, qb.rows), torch.float32, dev)
    ws_bytes = mxfp4_gemm_workspace_bytes(qa, qb)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=qa.codes.device)
    sa, sb = qa.as_struct(), qb.as_struct()
    _check(lib.mxfp4_gemm(ctypes.byref(sa), ctypes.byref(sb), _ptr(out), max(out.stride(0), qb.rows), _ptr(workspace),
                          _nbytes(workspace, dev), _stream(dev)))
    return out


def mxfp4_gemm_bf16(qa: QTensor, qb: QTensor, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M, N] = A B^T as mxfp4_gemm computes it, rounded to bfloat16 (nearest
    even)."""
    dev = _check_operands(qa, qb)
    if out is None:
        out = torch.empty((qa.rows, qb.rows), dtype=torch.bfloat16, device=dev)
    _check_out(out, (qa.rows, qb.rows), torch.bfloat16, dev)
    ws_bytes = mxfp4_gemm_workspace_bytes(qa, qb)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=qa.codes.device)
    sa, sb = qa.as_struct(), qb.as_struct()
    _check(lib.mxfp4_gemm_bf16(ctypes.byref(sa), ctypes.byref(sb), _ptr(out), max(out.stride(0), qb.rows),
                               _ptr(workspace),
                               _nbytes(workspace, dev), _stream(dev)))
    return out


def mxfp4_gemm_quantize_workspace_bytes(qa: QTensor, qb: QTensor, hadamard: bool, out: QTensor) -> int:
    b = ctypes.c_size_t()
    sa, sb, so = qa.as_struct(), qb.as_struct(), out.as_struct()
    _check(lib.mxfp4_gemm_quantize_workspace_bytes(ctypes.byref(sa), ctypes.byref(sb), int(bool(hadamard)),
                                                   ctypes.byref(so), ctypes.byref(b)))
    return b.value


def mxfp4_gemm_quantize(qa: QTensor, qb: QTensor, hadamard: bool = False, out: Optional[QTensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> QTensor:
    """Q(bf16(A B^T)): the GEMM with its output quantized to MXFP4 (round to
    nearest, along rows, block Hadamard first if asked) for the next layer --
    the same bits as mxfp4_quantize(mxfp4_gemm_bf16(qa, qb), "mx", "rtn",
    hadamard)."""
    dev = _check_operands(qa, qb)
    if out is None:
        out = empty_qtensor("mx", qa.rows, qb.rows, hadamard, dev)
    if _check_operands(out) != dev:
        raise ValueError("out must live on the operands' device")
    ws_bytes = mxfp4_gemm_quantize_workspace_bytes(qa, qb, hadamard, out)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    sa, sb, so = qa.as_struct(), qb.as_struct(), out.as_struct()
    _check(lib.mxfp4_gemm_quantize(ctypes.byref(sa), ctypes.byref(sb), int(bool(hadamard)), ctypes.byref(so),
                                   _ptr(workspace), _nbytes(workspace, dev), _stream(dev)))
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
    dev = _check_operands(qb)
    if x.device != dev:
        raise ValueError("x and the weights must live on one device")
    if out is None:
        out = torch.empty((M, qb.rows), dtype=torch.float32, device=dev)
    _check_out(out, (M, qb.rows), torch.float32, dev)
    ws_bytes = mxfp4_quantize_gemm_workspace_bytes(M, K, hadamard, qb)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    sb = qb.as_struct()
    _check(lib.mxfp4_quantize_gemm(_ptr(x), M, K, x.stride(0), int(bool(hadamard)), ctypes.byref(sb), _ptr(out),
                                   max(out.stride(0), qb.rows), _ptr(workspace), _nbytes(workspace, x.device),
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
    if _check_operands(out) != x.device:
        raise ValueError("out must live on x's device")
    ws_bytes = mxfp4_quantize_mse_workspace_bytes(fmt, hadamard, R, C, axis)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = out.as_struct()
    _check(lib.mxfp4_quantize_mse(_ptr(x), R, C, x.stride(0), FMT[fmt], int(bool(hadamard)), int(axis), int(iters),
                                  ctypes.byref(st), _ptr(workspace), _nbytes(workspace, x.device),
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
    if _check_operands(q) != x.device:
        raise ValueError("x and q must live on one device")
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=x.device)
    if out.dtype != torch.float64 or out.numel() < 3 or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous float64 tensor of 3 elements on x's device")
    ws_bytes = mxfp4_quantization_noise_workspace_bytes(q)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    sq = q.as_struct()
    _check(lib.mxfp4_quantization_noise(_ptr(x), x.stride(0), int(axis), ctypes.byref(sq), _ptr(out),
                                        _ptr(workspace), _nbytes(workspace, x.device), _stream(x.device)))
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
    if _check_operands(out) != x.device:
        raise ValueError("out must live on x's device")
    if stats is None:
        stats = torch.empty(3, dtype=torch.float64, device=x.device)
    if stats.dtype != torch.float64 or stats.numel() < 3 or not stats.is_contiguous() or stats.device != x.device:
        raise ValueError("stats must be a contiguous float64 tensor of 3 elements on x's device")
    ws_bytes = mxfp4_quantize_noise_workspace_bytes(fmt, hadamard, R, C, axis)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    st = out.as_struct()
    _check(lib.mxfp4_quantize_noise(_ptr(x), R, C, x.stride(0), FMT[fmt], ROUNDING[rounding], int(bool(hadamard)),
                                    int(axis), int(seed) & (2 ** 64 - 1), ctypes.byref(st), _ptr(stats),
                                    _ptr(workspace), _nbytes(workspace, x.device), _stream(x.device)))
    return out, stats


def mxfp4_noise_ratio(stats) -> tuple:
    """(ratio, below) of the sqrt(3) test ("FP4 All the Way", abstract) from
    the three sums of mxfp4_quantization_noise / mxfp4_quantize_noise (a host
    sequence or tensor): computed by the library's mxfp4_noise_ratio."""
    if isinstance(stats, torch.Tensor):
        stats = stats.detach().cpu().tolist()
    arr = (ctypes.c_double * 3)(*[float(v) for v in stats])
    ratio, below = ctypes.c_double(), ctypes.c_int()
    _check(lib.mxfp4_noise_ratio(arr, ctypes.byref(ratio), ctypes.byref(below)))
    return ratio.value, bool(below.value)


def gradient_noise_ratio(x: torch.Tensor, q: QTensor, axis: int = 1):
    """(ratio, below) for the quantized operand q of x: the noise sums on the
    GPU, then the library's sqrt(3) test on them."""
    return mxfp4_noise_ratio(mxfp4_quantization_noise(x, q, axis))


quantize = mxfp4_quantize
dequantize = mxfp4_dequantize
gemm = mxfp4_gemm
quantize_gemm = mxfp4_quantize_gemm

__all__ = ["QTensor", "MxFp4Error", "mxfp4_tensor_bytes", "mxfp4_quantize_workspace_bytes", "mxfp4_quantize",
           "mxfp4_quantize_noalloc", "mxfp4_qema_quantize", "mxfp4_gemm_quantize", "mxfp4_quantize_grid",
           "mxfp4_gemm_quantize_workspace_bytes",
           "mxfp4_dequantize", "mxfp4_gemm_workspace_bytes", "mxfp4_gemm", "mxfp4_gemm_bf16", "mxfp4_status_string",
           "mxfp4_quantize_gemm_workspace_bytes", "mxfp4_quantize_gemm",
           "mxfp4_quantization_noise_workspace_bytes", "mxfp4_quantization_noise", "gradient_noise_ratio",
           "mxfp4_noise_ratio",
           "mxfp4_quantize_noise_workspace_bytes", "mxfp4_quantize_noise",
           "mxfp4_quantize_mse_workspace_bytes", "mxfp4_quantize_mse",
           "quantize", "dequantize", "gemm", "quantize_gemm", "empty_qtensor", "lib", "LIB_PATH"]
