"""GPU parity of mxfp4_quantize_grid (MXFP4 with a fixed grid scale alpha,
the digest of the MR-GPTQ paper, step 1) with the oracle, bit for bit: several
alpha values, with and without the rotation, both axes, NaN blocks, a
full-size configuration-3 weight; alpha = 1 equals mxfp4_quantize."""
import numpy as np
import pytest

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_codes_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("alpha", [1.0, 0.75, 0.6, 1.5])
@pytest.mark.parametrize("had,axis", [(True, 1), (True, 0), (False, 1)])
def test_grid_matches_oracle(oracle_mod, alpha, had, axis):
    mx = need_gpu()
    X = workloads.small_t_bf16((320, 288), 4.0, seed=140, outlier_frac=0.02).copy()
    X[7, 70] = 0x7FC0
    say("grid", alpha, had, axis)
    q = q_to_host(mx.mxfp4_quantize_grid(to_device_bf16(X), alpha, had, axis))
    assert_codes_equal(q, oracle_mod.quantize_grid(X, alpha, had, axis), f"grid {alpha} {had} {axis}")
    if alpha == 1.0:
        assert_codes_equal(q, q_to_host(mx.mxfp4_quantize(to_device_bf16(X), "mx", "rtn", had, axis)), "grid 1 = rtn")


def test_grid_full_size_weight(oracle_mod):
    mx = need_gpu()
    W = workloads.make_tensor(3, "W_down")
    say("grid full size", W.shape)
    q = q_to_host(mx.mxfp4_quantize_grid(to_device_bf16(W), 0.75, True, 1))
    assert_codes_equal(q, oracle_mod.quantize_grid(W, 0.75, True, 1), "grid config 3 W_down")


@pytest.mark.parametrize("axis", [1, 0])
def test_grid_unaligned_and_overflowing_blocks(oracle_mod, axis):
    """An input view one element off 16-byte alignment (the transposing path
    then takes the block kernel, the row path its element loads), and blocks
    whose alpha * absmax overflows binary32 (scale byte 254)."""
    mx = need_gpu()
    import torch
    X = workloads.small_t_bf16((96, 128), 3.0, seed=141).copy()
    X[3, 0:32] = 0x7F7F            # the largest finite bf16: 1.5 * absmax overflows
    X[40:72, 5] = 0xFF7F           # a column block of the same magnitude (axis 0)
    full = np.zeros((96, 128 + 8), dtype=np.uint16)
    full[:, 1:129] = X
    xt = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()[:, 1:129]
    for alpha in (1.5, 0.75):
        say("grid unaligned", axis, alpha)
        q = q_to_host(mx.mxfp4_quantize_grid(xt, alpha, False, axis))
        assert_codes_equal(q, oracle_mod.quantize_grid(X, alpha, False, axis), f"grid unaligned {axis} {alpha}")
    if axis == 1:
        assert 254 in q_to_host(mx.mxfp4_quantize_grid(xt, 1.5, False, axis))[1]
