"""Shared helpers for the GPU parity tests (HIP library vs the CPU oracle)."""
import sys

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import microscaling_fp4_quantized_block_amd as mx  # raises if the HIP library is missing
    return mx


def say(*a):
    """Name the case before each GPU step, flushed, so a failing run says where it was."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def to_device_bf16(bits: np.ndarray, pad_cols: int = 0) -> torch.Tensor:
    """uint16 bf16 patterns -> a bf16 device tensor (optionally with a row stride > C)."""
    R, C = bits.shape
    if pad_cols:
        full = np.zeros((R, C + pad_cols), dtype=np.uint16)
        full[:, :C] = bits
        t = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()
        return t[:, :C]
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def q_to_host(q):
    torch.cuda.synchronize()
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    ts = float(q.tensor_scale.cpu()[0]) if q.tensor_scale is not None else None
    return codes, scales, ts


def assert_codes_equal(got, want, what=""):
    gc, gs, gt = got
    wc, ws, wt = want
    if not np.array_equal(gs, ws):
        idx = np.argwhere(gs != ws)
        raise AssertionError(f"{what}: {len(idx)} scale bytes differ, first at {idx[0].tolist()}: "
                             f"gpu {gs[tuple(idx[0])]:#x} oracle {ws[tuple(idx[0])]:#x}")
    if not np.array_equal(gc, wc):
        idx = np.argwhere(gc != wc)
        raise AssertionError(f"{what}: {len(idx)} code bytes differ, first at {idx[0].tolist()}: "
                             f"gpu {gc[tuple(idx[0])]:#04x} oracle {wc[tuple(idx[0])]:#04x}")
    if wt is not None:
        assert np.float32(gt).view(np.uint32) == np.float32(wt).view(np.uint32), (what, gt, wt)


def assert_gemm_within(Cg: np.ndarray, Co: np.ndarray, So: np.ndarray, what="", tol=1e-5):
    # NaN and infinite results must sit where the oracle has them (a bare
    # |difference| comparison would let NaN through)
    Cg = Cg.astype(np.float64)
    ng, no = np.isnan(Cg), np.isnan(Co)
    if not np.array_equal(ng, no):
        i = np.argwhere(ng != no)[0]
        raise AssertionError(f"{what}: NaN positions differ; first {i.tolist()}: gpu {Cg[tuple(i)]!r} "
                             f"oracle {Co[tuple(i)]!r}")
    inf = np.isinf(Cg) | np.isinf(Co)
    if not np.array_equal(Cg[inf], Co[inf]):
        raise AssertionError(f"{what}: infinite results differ from the oracle's")
    special = ng | inf
    Cg, Co, So = np.where(special, 0.0, Cg), np.where(special, 0.0, Co), np.where(special, 0.0, So)
    err = np.abs(Cg - Co)
    bound = tol * So
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements outside 1e-5*sum|ab|; first {i.tolist()}: "
                             f"gpu {Cg[tuple(i)]!r} oracle {Co[tuple(i)]!r} S {So[tuple(i)]!r}")
    return float((err / np.where(So > 0, So, 1)).max())
