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
