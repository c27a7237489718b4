"""GPU parity of the fused quantize + noise sums (mxfp4_quantize_noise).

The quantized tensor must be exactly what mxfp4_quantize writes for the same
arguments (codes, scale bytes, NVFP4 tensor scale: compared with the oracle's
quantization, bit for bit); the sums are the oracle's noise_stats of that
tensor within 1e-12 relative (the same binary64 terms in another order), the
left-out count exactly, and the same bits on a second call."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_codes_equal

pytestmark = pytest.mark.gpu

COMBOS = [(f, r, h) for f in ("mx", "nv") for r in ("rtn", "sr") for h in (False, True)]


def _check(mx, oracle_mod, X, xt, fmt, rnd, had, axis, seed=9, what=""):
    q, st = mx.mxfp4_quantize_noise(xt, fmt, rnd, had, axis, seed)
    q2, st2 = mx.mxfp4_quantize_noise(xt, fmt, rnd, had, axis, seed)
    torch.cuda.synchronize()
    g = st.cpu().numpy()
    assert np.array_equal(g.view(np.uint64), st2.cpu().numpy().view(np.uint64)), what + ": not deterministic"
    oq = oracle_mod.quantize(X, fmt, rnd, had, axis, seed)
    assert_codes_equal(q_to_host(q), oq, what)
    o = oracle_mod.noise_stats(X, oq, fmt, had, axis)
    for j in (0, 1):
        assert abs(g[j] - o[j]) <= 1e-12 * max(abs(o[j]), 1e-300), (what, j, g[j], o[j])
    assert g[2] == o[2], (what, g[2], o[2])
    return g, o


@pytest.mark.parametrize("fmt,rnd,had", COMBOS)
@pytest.mark.parametrize("axis", [1, 0])
def test_quantize_noise_matches_oracle(oracle_mod, fmt, rnd, had, axis):
    """Several workgroups of the row kernel and of the tiled transposing
    kernel, with a ragged last tile (304 rows: a 16-row NVFP4 tail when
    unrotated) and a column count that is not a multiple of 64."""
    mx = need_gpu()
    shape = (304 if (fmt == "nv" and not had) else 288, 200) if axis == 0 else (320, 288)
    X = workloads.small_t_bf16(shape, 3.0, seed=71, outlier_frac=0.02)
    say("quantize+noise", fmt, rnd, had, axis, shape)
    _check(mx, oracle_mod, X, to_device_bf16(X), fmt, rnd, had, axis, what=f"{fmt} {rnd} {had} {axis}")


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("pad", [3, 8])
def test_quantize_noise_strided_and_unaligned(oracle_mod, axis, pad):
    """Row strides past C; a 2-byte-misaligned view takes the element-wise
    row loads (axis 1) or the small transposing kernel plus the separate
    noise pass (axis 0)."""
    mx = need_gpu()
    X = workloads.small_normal_bf16((96, 256), 1.0, seed=72)
    full = np.zeros((96, 256 + pad + 1), dtype=np.uint16)
    full[:, 1:257] = X
    xt = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).cuda()[:, 1:257]
    say("quantize+noise unaligned", axis, pad)
    _check(mx, oracle_mod, X, xt, "mx", "sr", False, axis, what=f"unaligned axis {axis} pad {pad}")
    full2 = np.zeros((96, 256 + pad), dtype=np.uint16)
    full2[:, :256] = X
    xt2 = torch.from_numpy(full2.view(np.int16)).view(torch.bfloat16).cuda()[:, :256]
    _check(mx, oracle_mod, X, xt2, "nv", "sr", False, axis, what=f"strided axis {axis} pad {pad}")


def test_quantize_noise_nv_blocks_of_16(oracle_mod):
    """NVFP4 without rotation on a contraction that is not a multiple of 32."""
    mx = need_gpu()
    X = workloads.small_normal_bf16((48, 80), 1.0, seed=73)
    say("quantize+noise nv 16")
    _check(mx, oracle_mod, X, to_device_bf16(X), "nv", "sr", False, 1, what="nv16 rows")
    Xt = workloads.small_normal_bf16((80, 64), 1.0, seed=74)
    _check(mx, oracle_mod, Xt, to_device_bf16(Xt), "nv", "sr", False, 0, what="nv16 columns")


@pytest.mark.parametrize("axis", [1, 0])
def test_quantize_noise_nan_blocks_left_out(oracle_mod, axis):
    mx = need_gpu()
    X = workloads.small_normal_bf16((64, 128), 1.0, seed=75).copy()
    X[3, 5] = 0x7FC0
    X[40, 100] = 0x7F80
    say("quantize+noise nan blocks", axis)
    g, _ = _check(mx, oracle_mod, X, to_device_bf16(X), "nv", "rtn", False, axis, what=f"nan axis {axis}")
    assert g[2] == 32.0


def test_quantize_noise_empty():
    mx = need_gpu()
    xt = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, st = mx.mxfp4_quantize_noise(xt, "mx", "sr", False, 1, 1)
    torch.cuda.synchronize()
    assert q.rows == 0 and st.cpu().tolist() == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("cfg,name,fmt,axis", [(4, "dY1", "mx", 1), (4, "dY1", "mx", 0), (5, "dY_o", "nv", 0),
                                               (5, "dY_o", "nv", 1)])
def test_quantize_noise_full_size_gradients(oracle_mod, cfg, name, fmt, axis):
    """The backward operands of the training configurations (stochastic
    rounding), at full size."""
    mx = need_gpu()
    X = workloads.make_tensor(cfg, name)
    say("quantize+noise full size", cfg, name, fmt, axis, X.shape)
    _check(mx, oracle_mod, X, to_device_bf16(X), fmt, "sr", False, axis, seed=3, what=f"config {cfg} {name}")
