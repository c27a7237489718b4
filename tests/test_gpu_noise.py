"""GPU parity of the quantization-noise sums (mxfp4_quantization_noise)
against the oracle: sum y^2 and sum (Q(y) - y)^2 within 1e-12 relative (both
sides add the same binary64 terms, in different orders), the left-out count
exactly, and the same bits on a second call."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16

pytestmark = pytest.mark.gpu

COMBOS = [(f, r, h) for f in ("mx", "nv") for r in ("rtn", "sr") for h in (False, True)]


def _check(mx, oracle_mod, X, xt, fmt, rnd, had, axis, seed=9, what=""):
    q = mx.mxfp4_quantize(xt, fmt, rnd, had, axis, seed)
    st = mx.mxfp4_quantization_noise(xt, q, axis)
    st2 = mx.mxfp4_quantization_noise(xt, q, axis)
    torch.cuda.synchronize()
    g = st.cpu().numpy()
    assert np.array_equal(g.view(np.uint64), st2.cpu().numpy().view(np.uint64)), what + ": not deterministic"
    oq = oracle_mod.quantize(X, fmt, rnd, had, axis, seed)
    o = oracle_mod.noise_stats(X, oq, fmt, had, axis)
    for j in (0, 1):
        assert abs(g[j] - o[j]) <= 1e-12 * max(abs(o[j]), 1e-300), (what, j, g[j], o[j])
    assert g[2] == o[2], (what, g[2], o[2])
    return g, o


@pytest.mark.parametrize("fmt,rnd,had", COMBOS)
@pytest.mark.parametrize("axis", [1, 0])
def test_noise_matches_oracle(oracle_mod, fmt, rnd, had, axis):
    mx = need_gpu()
    X = workloads.small_t_bf16((320, 288), 3.0, seed=51, outlier_frac=0.02)
    say("noise", fmt, rnd, had, axis)
    _check(mx, oracle_mod, X, to_device_bf16(X), fmt, rnd, had, axis, what=f"{fmt} {rnd} {had} {axis}")


@pytest.mark.parametrize("axis", [1, 0])
def test_noise_nv_blocks_of_16(oracle_mod, axis):
    """NVFP4 without rotation on a contraction that is not a multiple of 32:
    units of 16 elements."""
    mx = need_gpu()
    X = workloads.small_normal_bf16((48, 80), 1.0, seed=52)
    say("noise nv 16", axis)
    _check(mx, oracle_mod, X, to_device_bf16(X), "nv", "sr", False, axis, what=f"nv16 axis {axis}")


@pytest.mark.parametrize("pad", [0, 3])
def test_noise_unaligned_input(oracle_mod, pad):
    """Inputs 2 bytes off a 16-byte boundary or with an odd row stride take
    the element-wise loads."""
    mx = need_gpu()
    X = workloads.small_normal_bf16((64, 256), 1.0, seed=53)
    full = np.zeros((64, 256 + pad + 1), dtype=np.uint16)
    full[:, 1:257] = X
    xt = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()[:, 1:257]
    say("noise unaligned", pad)
    _check(mx, oracle_mod, X, xt, "mx", "sr", True, 1, what="unaligned")


def test_noise_nan_blocks_left_out(oracle_mod):
    mx = need_gpu()
    X = workloads.small_normal_bf16((64, 128), 1.0, seed=54).copy()
    X[3, 5] = 0x7FC0
    X[40, 100] = 0x7F80
    say("noise nan blocks")
    g, _ = _check(mx, oracle_mod, X, to_device_bf16(X), "nv", "rtn", False, 1, what="nan")
    assert g[2] == 32.0


def test_noise_ratio_helper(oracle_mod):
    """gradient_noise_ratio: ||y|| / ||Q(y) - y|| and the sqrt(3) flag."""
    mx = need_gpu()
    X = workloads.small_normal_bf16((128, 256), 1e-3, seed=55)
    xt = to_device_bf16(X)
    q = mx.mxfp4_quantize(xt, "mx", "sr", False, 1, 2)
    ratio, below = mx.gradient_noise_ratio(xt, q, 1)
    o = oracle_mod.noise_stats(X, oracle_mod.quantize(X, "mx", "sr", False, 1, 2), "mx", False, 1)
    assert abs(ratio - (o[0] / o[1]) ** 0.5) <= 1e-12 * ratio
    assert below == (ratio < 3 ** 0.5)


@pytest.mark.parametrize("cfg,name,fmt,axis", [(4, "dY1", "mx", 1), (4, "dY1", "mx", 0), (5, "dY_o", "nv", 0)])
def test_noise_full_size_gradients(oracle_mod, cfg, name, fmt, axis):
    """The backward operands of the training configurations (stochastic
    rounding), at full size."""
    mx = need_gpu()
    X = workloads.make_tensor(cfg, name)
    say("noise full size", cfg, name, fmt, axis, X.shape)
    _check(mx, oracle_mod, X, to_device_bf16(X), fmt, "sr", False, axis, seed=3, what=f"config {cfg} {name}")
