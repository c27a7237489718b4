"""GPU validity of mxfp4_quantize_mse (MSE-fitted scales) against the oracle's
definition, round by round.

Several outputs can be correct where two candidate scales give errors that
tie to within the rounding of the kernel's binary64 sums, so the test checks
what is unique and that the rest is valid: for every block the GPU's scale
byte is a candidate (at or below the absmax scale), its codes are exactly the
round-to-nearest encoding for that byte, and its exact squared error is within
REL_TOL of the smallest over all candidates (the oracle's exact search, no
window); for NVFP4 the round-0 tensor scale is bit-exact and each later one is
within one binary32 ulp of the exact least-squares scale for the previous
round's bytes and codes (the GPU's own, so each round is checked on its own
inputs).  Also: ragged and unaligned inputs, NaN blocks, full-size weights,
determinism."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host

pytestmark = pytest.mark.gpu

# The kernel sums at most 32 squared differences (each rounded once) in
# binary64: each computed error is within 33 * 2^-53 (3.7e-15) of the exact
# one, so the chosen block's exact error is within 2 * 3.7e-15 of the minimum.
REL_TOL = 1e-14


def ulp_distance(a, b):
    ia = int(np.float32(a).view(np.int32))
    ib = int(np.float32(b).view(np.int32))
    return abs(ia - ib)


def check_rounds(oracle_mod, mx, xt, X, fmt, had, axis, rounds, what):
    prev = None
    for iters in range(rounds + 1):
        say("mse", what, fmt, had, axis, "iters", iters)
        q = q_to_host(mx.mxfp4_quantize_mse(xt, fmt, had, axis, iters))
        if fmt == "nv":
            if iters == 0:
                want = oracle_mod.quantize(X, "nv", "rtn", had, axis)[2]
                assert np.float32(q[2]).view(np.uint32) == np.float32(want).view(np.uint32), (what, q[2], want)
            else:
                want = oracle_mod.mse_tensor_step(X, prev, had, axis, prev[2])
                assert ulp_distance(q[2], want) <= 1, (what, iters, q[2], want)
        r = oracle_mod.mse_check(X, q, fmt, had, axis, st=q[2], rel_tol=REL_TOL)
        say("   blocks", r["blocks"], "near ties resolved otherwise", r["differ_from_oracle"])
        assert r["bad_encoding"] == 0 and r["bad_error"] == 0, (what, iters, r)
        prev = q
        if fmt == "mx":
            break


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("axis", [1, 0])
def test_mse_valid_round_by_round(oracle_mod, fmt, had, axis):
    mx = need_gpu()
    X = workloads.small_t_bf16((320, 288), 3.0, seed=71, outlier_frac=0.02)
    check_rounds(oracle_mod, mx, to_device_bf16(X), X, fmt, had, axis, 2, "small")


@pytest.mark.parametrize("axis", [1, 0])
def test_mse_nv_units_of_16(oracle_mod, axis):
    mx = need_gpu()
    X = workloads.small_normal_bf16((48, 80), 1.0, seed=72)
    check_rounds(oracle_mod, mx, to_device_bf16(X), X, "nv", False, axis, 3, "nv16")


def test_mse_hand_worked_blocks_where_the_lowest_candidate_wins(oracle_mod):
    """The blocks of the golden fixture: MXFP4 keeps e0 - 1, NVFP4 b0 - 5
    (the lowest scales the kernel's search tries)."""
    mx = need_gpu()
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mse_blocks_worked.json")))
    mxb = np.full((1, 32), 0.25, dtype=np.float32)
    mxb[0, 5] = 3.25
    say("mse golden mx")
    q = q_to_host(mx.mxfp4_quantize_mse(to_device_bf16(workloads.f32_to_bf16_bits(mxb)), "mx", False, 1, 0))
    assert q[1].ravel().tolist() == [g["mx_block"]["expected_scale_byte"]]
    assert q[0].ravel().tolist() == g["mx_block"]["expected_codes"]
    nvb = np.zeros((2, 16), dtype=np.float32)
    nvb[0] = [0.087890625] * 7 + [0.140625] * 6 + [0.15234375] * 2 + [0.1884765625]
    nvb[1, 0] = 2688.0
    say("mse golden nv")
    q = q_to_host(mx.mxfp4_quantize_mse(to_device_bf16(workloads.f32_to_bf16_bits(nvb)), "nv", False, 1, 0))
    assert q[2] == 1.0
    assert q[1].ravel().tolist() == g["nv_block"]["expected_scale_bytes"]
    assert q[0][0].tolist() == g["nv_block"]["expected_codes_row0"]
    assert q[0][1].tolist() == g["nv_block"]["expected_codes_row1"]


def test_mse_unaligned_input_and_nan_blocks(oracle_mod):
    mx = need_gpu()
    X = workloads.small_t_bf16((64, 256), 4.0, seed=73).copy()
    X[5, 17] = 0x7FC0
    X[60, 250] = 0xFF80
    full = np.zeros((64, 256 + 4), dtype=np.uint16)
    full[:, 1:257] = X
    xt = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()[:, 1:257]
    for fmt in ("mx", "nv"):
        check_rounds(oracle_mod, mx, xt, X, fmt, False, 1, 1, "unaligned+nan")


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
    xt = to_device_bf16(X)
    check_rounds(oracle_mod, mx, xt, X, fmt, had, axis, 2, f"config {cfg} {name}")
    say("mse determinism", cfg, name)
    a = q_to_host(mx.mxfp4_quantize_mse(xt, fmt, had, axis, 2))
    b = q_to_host(mx.mxfp4_quantize_mse(xt, fmt, had, axis, 2))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]
