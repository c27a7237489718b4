"""GPU parity of mxfp4_gemm_quantize (the GEMM whose epilogue quantizes C to
MXFP4 for the next layer): bit for bit the same codes and scale bytes as
mxfp4_gemm_bf16 followed by mxfp4_quantize (round to nearest, along rows,
block Hadamard when asked), and the same as the oracle's quantizer on the
GPU's bf16 C (the GEMM itself is checked against the binary64 oracle by the
GEMM tests).  Covers the fused epilogue (MXFP4 wide tiles, no K split: ragged
tiles, the 256 x 128 half tiles) and the two-step path (the decode kernel's
shapes, split K, NVFP4 operands)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_codes_equal

pytestmark = pytest.mark.gpu


def _check(oracle_mod, mx, qa, qb, had, what):
    ws = mx.mxfp4_gemm_quantize_workspace_bytes(qa, qb, had, mx.empty_qtensor("mx", qa.rows, qb.rows, had, "cuda"))
    say("gemm_quantize", what, qa.rows, qb.rows, qa.k, "had", had, "ws", ws)
    fused = q_to_host(mx.mxfp4_gemm_quantize(qa, qb, had))
    c16 = mx.mxfp4_gemm_bf16(qa, qb)
    two = q_to_host(mx.mxfp4_quantize(c16, "mx", "rtn", had, 1))
    assert_codes_equal(fused, two, f"{what}: fused vs gemm_bf16 + quantize")
    bits = c16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_codes_equal(fused, oracle_mod.quantize(bits, "mx", "rtn", had, 1), f"{what}: vs oracle on the bf16 C")
    return ws


@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("M,N,K", [(256, 256, 1024), (300, 256, 384), (17, 512, 256), (512, 768, 2048),
                                   (4352, 3904, 512), (64, 96, 8192), (128, 160, 640)])
def test_gemm_quantize_matches_two_step(oracle_mod, had, M, N, K):
    mx = need_gpu()
    A = workloads.small_t_bf16((M, K), 3.0, seed=120, outlier_frac=0.02)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=121)
    qa = mx.mxfp4_quantize(to_device_bf16(A), "mx", "rtn", had)
    qb = mx.mxfp4_quantize(to_device_bf16(B), "mx", "rtn", had)
    _check(oracle_mod, mx, qa, qb, had, "mx")


def test_gemm_quantize_nvfp4_operands_two_step(oracle_mod):
    mx = need_gpu()
    A = workloads.small_t_bf16((512, 1024), 3.0, seed=122)
    B = workloads.small_normal_bf16((384, 1024), 0.02, seed=123)
    qa = mx.mxfp4_quantize(to_device_bf16(A), "nv", "rtn")
    qb = mx.mxfp4_quantize(to_device_bf16(B), "nv", "rtn")
    assert _check(oracle_mod, mx, qa, qb, True, "nv") > 0


def test_gemm_quantize_nonfinite_blocks(oracle_mod):
    """A block of C holding infinities (FP32 overflow) gets the NaN scale byte
    and zero codes on both paths."""
    mx = need_gpu()
    va = np.ones((64, 256), dtype=np.float32) * 2.0 ** 100
    vb = np.ones((64, 256), dtype=np.float32) * 2.0 ** 100
    qa = mx.mxfp4_quantize(to_device_bf16(workloads.f32_to_bf16_bits(va)), "mx", "rtn")
    qb = mx.mxfp4_quantize(to_device_bf16(workloads.f32_to_bf16_bits(vb)), "mx", "rtn")
    fused = q_to_host(mx.mxfp4_gemm_quantize(qa, qb, False))
    assert np.all(fused[1] == 0xFF) and np.all(fused[0] == 0)
    _check(oracle_mod, mx, qa, qb, False, "overflow")


def test_gemm_quantize_config3_prefill_up(oracle_mod):
    """Configuration 3 prefill: 4096 x 14336 x 4096 with rotated operands, the
    output quantized (rotated) as the down projection's input."""
    mx = need_gpu()
    X = workloads.make_tensor(3, "x_pre_up")
    W = workloads.make_tensor(3, "W_up")
    qx = mx.mxfp4_quantize(to_device_bf16(X), "mx", "rtn", True)
    qw = mx.mxfp4_quantize(to_device_bf16(W), "mx", "rtn", True)
    assert _check(oracle_mod, mx, qx, qw, True, "config3 prefill up") == 0
