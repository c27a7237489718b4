"""GPU parity of mxfp4_quantize_mse (MSE-fitted scales) with the oracle: codes,
scale bytes and the NVFP4 tensor scale bit for bit, for both formats, with
and without the rotation, along both axes, for several alternation counts,
on ragged and unaligned inputs, NaN blocks, and full-size weights."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_codes_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("iters", [0, 2])
def test_mse_matches_oracle(oracle_mod, fmt, had, axis, iters):
    mx = need_gpu()
    X = workloads.small_t_bf16((320, 288), 3.0, seed=71, outlier_frac=0.02)
    say("mse", fmt, had, axis, iters)
    q = mx.mxfp4_quantize_mse(to_device_bf16(X), fmt, had, axis, iters)
    assert_codes_equal(q_to_host(q), oracle_mod.quantize_mse(X, fmt, had, axis, iters), f"mse {fmt} {had} {axis} {iters}")


@pytest.mark.parametrize("axis", [1, 0])
def test_mse_nv_units_of_16(oracle_mod, axis):
    mx = need_gpu()
    X = workloads.small_normal_bf16((48, 80), 1.0, seed=72)
    say("mse nv16", axis)
    q = mx.mxfp4_quantize_mse(to_device_bf16(X), "nv", False, axis, 3)
    assert_codes_equal(q_to_host(q), oracle_mod.quantize_mse(X, "nv", False, axis, 3), "mse nv16")


def test_mse_unaligned_input_and_nan_blocks(oracle_mod):
    mx = need_gpu()
    X = workloads.small_t_bf16((64, 256), 4.0, seed=73).copy()
    X[5, 17] = 0x7FC0
    X[60, 250] = 0xFF80
    full = np.zeros((64, 256 + 4), dtype=np.uint16)
    full[:, 1:257] = X
    xt = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()[:, 1:257]
    for fmt in ("mx", "nv"):
        say("mse unaligned nan", fmt)
        q = mx.mxfp4_quantize_mse(xt, fmt, False, 1, 1)
        assert_codes_equal(q_to_host(q), oracle_mod.quantize_mse(X, fmt, False, 1, 1), f"mse unaligned {fmt}")


def test_mse_lowers_the_quantization_error(oracle_mod):
    """The point of the mode: less squared error than the absmax scales
    (measured with the noise pass)."""
    mx = need_gpu()
    X = workloads.small_t_bf16((256, 512), 3.0, seed=74, outlier_frac=0.01)
    xt = to_device_bf16(X)
    for fmt in ("mx", "nv"):
        e_abs = mx.mxfp4_quantization_noise(xt, mx.mxfp4_quantize(xt, fmt, "rtn", False, 1), 1).cpu()[1].item()
        e_mse = mx.mxfp4_quantization_noise(xt, mx.mxfp4_quantize_mse(xt, fmt, False, 1, 2), 1).cpu()[1].item()
        say("mse error", fmt, e_abs, e_mse)
        assert e_mse < e_abs


@pytest.mark.parametrize("cfg,name,fmt,had,axis", [(2, "W", "nv", False, 1), (5, "W_o", "nv", False, 0),
                                                   (3, "W_down", "mx", True, 1)])
def test_mse_full_size_weights(oracle_mod, cfg, name, fmt, had, axis):
    mx = need_gpu()
    X = workloads.make_tensor(cfg, name)
    say("mse full size", cfg, name, X.shape)
    q = mx.mxfp4_quantize_mse(to_device_bf16(X), fmt, had, axis, 2)
    assert_codes_equal(q_to_host(q), oracle_mod.quantize_mse(X, fmt, had, axis, 2), f"mse config {cfg} {name}")
