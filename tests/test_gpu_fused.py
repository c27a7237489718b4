"""GPU parity of the online-activation-quantization GEMM (mxfp4_quantize_gemm):
its result must equal mxfp4_quantize followed by mxfp4_gemm bit for bit (same
codes, same scale bytes, same products in the same order), and the oracle
within 1e-5 * sum|ab|.  Covers the two-step path into the decode GEMM (up to
128 rows: with and without the block Hadamard, ragged M and N, contractions
ending mid-stage, unaligned and padded inputs, NaN blocks, configuration 3
decode), the fused narrow path (up to 32 rows on a narrow plan: long
contractions against short weights, split along K) and the other two-step
cases (more rows on narrow tiles, wide activations)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, assert_gemm_within

pytestmark = pytest.mark.gpu


def _bits(C: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return C.cpu().numpy().view(np.uint32)


def _both(mx, x, qw, had):
    """Fused result and quantize-then-GEMM result for the same input."""
    Cf = mx.mxfp4_quantize_gemm(x, qw, had)
    qx = mx.mxfp4_quantize(x, "mx", "rtn", had, 1, 0)
    Cu = mx.mxfp4_gemm(qx, qw)
    return Cf, Cu


@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 300, 256), (16, 256, 1024), (17, 529, 384), (32, 512, 2048),
                                   (5, 96, 8192), (31, 7000, 4096), (33, 640, 1024), (64, 96, 8192),
                                   (100, 256, 640), (128, 160, 512), (129, 200, 256), (300, 272, 384),
                                   (16, 256, 65536), (7, 300, 65536)])
def test_quantize_gemm_matches_two_step_and_oracle(oracle_mod, had, M, N, K):
    """Every element of C: bit-identical to the two-step path, and within the
    oracle's tolerance (128 < M takes the two-step path itself)."""
    mx = need_gpu()
    X = workloads.small_t_bf16((M, K), 4.0, seed=41)
    W = workloads.small_normal_bf16((N, K), 0.02, seed=42)
    say("quantize_gemm", M, N, K, "had", had)
    qw = mx.mxfp4_quantize(to_device_bf16(W), "mx", "rtn", had, 1, 0)
    Cf, Cu = _both(mx, to_device_bf16(X), qw, had)
    assert np.array_equal(_bits(Cf), _bits(Cu)), f"{M}x{N}x{K} had={had}: fused differs from two-step"
    ox = oracle_mod.quantize(X, "mx", "rtn", had)
    ow = oracle_mod.quantize(W, "mx", "rtn", had)
    Co, So = oracle_mod.gemm("mx", ox, ow)
    assert_gemm_within(Cf.cpu().numpy(), Co, So, f"quantize_gemm {M}x{N}x{K}")


@pytest.mark.parametrize("pad,offset", [(3, 0), (0, 1), (5, 1)])
def test_quantize_gemm_unaligned_and_padded_input(oracle_mod, pad, offset):
    """Rows with a stride that is not a multiple of 8 elements, or a start 2
    bytes off a 16-byte boundary, take the element-wise load path."""
    mx = need_gpu()
    M, N, K = 24, 384, 1024
    X = workloads.small_t_bf16((M, K), 4.0, seed=43)
    W = workloads.small_normal_bf16((N, K), 0.02, seed=44)
    full = np.zeros((M, K + pad + offset), dtype=np.uint16)
    full[:, offset:offset + K] = X
    xt = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()[:, offset:offset + K]
    assert xt.stride(0) == K + pad + offset
    say("quantize_gemm unaligned", pad, offset)
    qw = mx.mxfp4_quantize(to_device_bf16(W), "mx", "rtn", True, 1, 0)
    Cf, Cu = _both(mx, xt, qw, True)
    assert np.array_equal(_bits(Cf), _bits(Cu))
    Cc = mx.mxfp4_quantize_gemm(to_device_bf16(X), qw, True)
    assert np.array_equal(_bits(Cf), _bits(Cc))


def test_quantize_gemm_nan_blocks():
    """A block holding NaN or Inf gets the NaN scale byte in both paths, so the
    same output elements come out NaN."""
    mx = need_gpu()
    M, N, K = 8, 256, 512
    X = workloads.small_normal_bf16((M, K), 1.0, seed=45).copy()
    X[2, 70] = 0x7FC0     # NaN
    X[5, 300] = 0xFF80    # -Inf
    W = workloads.small_normal_bf16((N, K), 0.02, seed=46)
    say("quantize_gemm nan blocks")
    qw = mx.mxfp4_quantize(to_device_bf16(W), "mx", "rtn", False, 1, 0)
    Cf, Cu = _both(mx, to_device_bf16(X), qw, False)
    bf, bu = _bits(Cf), _bits(Cu)
    assert np.array_equal(bf, bu)
    C = Cf.cpu().numpy()
    assert np.isnan(C[2]).all() and np.isnan(C[5]).all() and not np.isnan(C[0]).any()


def test_quantize_gemm_config3_decode():
    """Decode-shaped linear layers with rotated weights: 16 x 14336 x 4096 and
    16 x 4096 x 14336, the launch the benchmark sweep times."""
    mx = need_gpu()
    for xname, wname in (("x_dec_up", "W_up"), ("x_dec_down", "W_down")):
        X = workloads.make_tensor(3, xname)
        W = workloads.make_tensor(3, wname)
        say("quantize_gemm config3", xname, X.shape, W.shape)
        qw = mx.mxfp4_quantize(to_device_bf16(W), "mx", "rtn", True, 1, 0)
        # quantized into the workspace, then the decode GEMM
        assert mx.mxfp4_quantize_gemm_workspace_bytes(X.shape[0], X.shape[1], True, qw) == 16 * X.shape[1] * 17 // 32
        Cf, Cu = _both(mx, to_device_bf16(X), qw, True)
        assert np.array_equal(_bits(Cf), _bits(Cu)), xname


def test_quantize_gemm_narrow_plan_not_fused():
    """65 rows against 1024 weight rows over K = 16384 (past the decode
    kernel's bytes per workgroup): a narrow plan with 128-row tiles, which the
    fused kernel (32-row tiles) does not take, so the call quantizes into the
    workspace and runs the split GEMM; the result is still the two-step one."""
    mx = need_gpu()
    M, N, K = 65, 1024, 16384
    g = torch.Generator(device="cuda")
    g.manual_seed(47)
    x = (torch.randn((M, K), generator=g, device="cuda") * 2.0).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    say("quantize_gemm narrow plan, two-step", M, N, K)
    qw = mx.mxfp4_quantize(w, "mx", "rtn", False, 1, 0)
    del w
    need = mx.mxfp4_quantize_gemm_workspace_bytes(M, K, False, qw)
    ws_gemm = mx.mxfp4_gemm_workspace_bytes(mx.empty_qtensor("mx", M, K, False, "cuda"), qw)
    assert ws_gemm > 0 and need == M * K // 2 + ((M * K // 32 + 15) // 16) * 16 + ws_gemm
    Cf, Cu = _both(mx, x, qw, False)
    assert np.array_equal(_bits(Cf), _bits(Cu))
