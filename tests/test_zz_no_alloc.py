"""mxfp4_quantize_noalloc (the entry point for callers that cannot allocate):
called through the C ABI, it gives exactly mxfp4_quantize's output, on two
calls in a row on one device (the second with a smaller input, so the
static scratch holds the first call's partials when it starts), for NVFP4
(which uses the scratch) and MXFP4 (which does not); inputs whose partials
exceed the scratch are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host

pytestmark = pytest.mark.gpu


def _same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and (
        a[2] is None or np.float32(a[2]).view(np.uint32) == np.float32(b[2]).view(np.uint32))


@pytest.mark.parametrize("fmt,rnd,had,axis", [("nv", "sr", False, 1), ("nv", "rtn", True, 0), ("mx", "sr", False, 0)])
def test_noalloc_matches_quantize_on_two_calls(fmt, rnd, had, axis):
    mx = need_gpu()
    for i, (R, C) in enumerate([(4096, 4096), (768, 512)]):
        X = workloads.small_t_bf16((R, C), 3.0, seed=90 + i, outlier_frac=0.01)
        xt = to_device_bf16(X)
        rows, k = (R, C) if axis == 1 else (C, R)
        say("noalloc", fmt, rnd, had, axis, R, C)
        ref = q_to_host(mx.mxfp4_quantize(xt, fmt, rnd, had, axis, 11))
        out = mx.empty_qtensor(fmt, rows, k, had, xt.device)
        st = out.as_struct()
        status = mx.lib.mxfp4_quantize_noalloc(ctypes.c_void_p(xt.data_ptr()), R, C, xt.stride(0), mx.FMT[fmt],
                                               mx.ROUNDING[rnd], int(had), axis, 11, ctypes.byref(st),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert status == 0, mx.mxfp4_status_string(status)
        got = q_to_host(out)
        assert _same(got, ref), (fmt, rnd, had, axis, R, C)


SCRATCH_BYTES = 1 << 20   # the library's static scratch (262144 partials)


def test_noalloc_refuses_inputs_past_the_scratch():
    mx = need_gpu()
    # 2^20 x 2^13 NVFP4 elements need 2 MiB of partials: refused before any
    # launch.  The pointers are not device memory, so the call is made only
    # once the size query confirms the refusal.
    R, C = 2 ** 20, 2 ** 13
    need = mx.mxfp4_quantize_workspace_bytes("nv", R, C)
    if need <= SCRATCH_BYTES:
        pytest.fail(f"{R}x{C} needs {need} bytes of partials, within the scratch: not a refusal case")
    out = mx.MxTensorStruct(1, 0, R, C, 0x100000, 0x100000, 0x100000)
    status = mx.lib.mxfp4_quantize_noalloc(ctypes.c_void_p(0x100000), R, C, C, 1, 0, 0, 1, 0,
                                           ctypes.byref(out), None)
    assert status == -4
