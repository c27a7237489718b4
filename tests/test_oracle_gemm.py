"""Pins of the oracle's block-scaled GEMM: C = A B^T in binary64 over the
dequantized operands (the FP4 GEMM of "Bridging the Gap Between Promise and
Performance for Microscaling FP4 Quantization", abstract, and the fully
quantized forward/backward GEMMs of "FP4 All the Way", abstract).

Pinned against numpy's float64 matmul on operands decoded independently
(E2M1 grid list, torch's E8M0/E4M3 decoders), exact integer results on
one-hot operands, and the rotation identity (X H)(W H)^T = X W^T.
"""
import numpy as np
import pytest
import torch

import workloads

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def decode(fmt, codes, scales, ts):
    lo, hi = codes & 0xF, codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    v = np.where(c & 8, -GRID[c & 7], GRID[c & 7])
    bs = 32 if fmt == "mx" else 16
    dt = torch.float8_e8m0fnu if fmt == "mx" else torch.float8_e4m3fn
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(dt).double().numpy()
    out = v * np.repeat(s, bs, axis=1)
    if fmt == "nv":
        out = out * float(ts)
    return out


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_gemm_matches_numpy_float64(oracle_mod, fmt):
    A = workloads.small_t_bf16((48, 256), 3.0, seed=10, outlier_frac=0.05)
    B = workloads.small_normal_bf16((40, 256), 0.02, seed=11)
    qa = oracle_mod.quantize(A, fmt, "rtn")
    qb = oracle_mod.quantize(B, fmt, "rtn")
    C, S = oracle_mod.gemm(fmt, qa, qb)
    Ad, Bd = decode(fmt, *qa), decode(fmt, *qb)
    ref = Ad @ Bd.T
    np.testing.assert_allclose(C, ref, rtol=0, atol=1e-12 * (np.abs(Ad) @ np.abs(Bd).T).max())
    np.testing.assert_allclose(S, np.abs(Ad) @ np.abs(Bd).T, rtol=1e-12)
    assert np.all(S >= np.abs(C))
    # sub-matrix selection is the same computation on the chosen rows/columns
    rows, cols = np.array([3, 0, 47]), np.array([39, 2])
    C2, S2 = oracle_mod.gemm(fmt, qa, qb, rows=rows, cols=cols)
    np.testing.assert_array_equal(C2, C[np.ix_(rows, cols)])
    np.testing.assert_array_equal(S2, S[np.ix_(rows, cols)])


def test_one_hot_operands_give_exact_integers(oracle_mod):
    """Codes of +-1 (0x2/0xA) with unit scales: C counts matching signs."""
    rng = np.random.default_rng(12)
    M, N, K = 8, 8, 128
    sa = rng.integers(0, 2, size=(M, K))
    sb = rng.integers(0, 2, size=(N, K))
    mask = rng.integers(0, 2, size=(M, K))
    ca = np.where(mask == 1, 0x2 | (sa << 3), 0).astype(np.uint8)
    cb = (0x2 | (sb << 3)).astype(np.uint8)
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    ones = np.full((M, K // 32), 127, dtype=np.uint8)
    C, S = oracle_mod.gemm("mx", (pack(ca), ones, None), (pack(cb), np.full((N, K // 32), 127, np.uint8), None))
    va = np.where(mask == 1, 1 - 2 * sa, 0)
    vb = 1 - 2 * sb
    np.testing.assert_array_equal(C, (va @ vb.T).astype(np.float64))
    np.testing.assert_array_equal(S, (np.abs(va) @ np.abs(vb).T).astype(np.float64))


def test_rotation_cancels_in_the_product(oracle_mod):
    """Rotating both operands by the orthonormal block Hadamard leaves the
    product unchanged up to quantization error (rotation fused into the
    weights and applied online to activations; Bridging the Gap ..., abstract)."""
    X = workloads.small_t_bf16((32, 512), 4.0, seed=13)
    W = workloads.small_normal_bf16((24, 512), 0.02, seed=14)
    xf = workloads.bf16_bits_to_f32(X).astype(np.float64)
    wf = workloads.bf16_bits_to_f32(W).astype(np.float64)
    exact = xf @ wf.T
    Ch, _ = oracle_mod.gemm("mx", oracle_mod.quantize(X, "mx", "rtn", True),
                            oracle_mod.quantize(W, "mx", "rtn", True))
    Cp, _ = oracle_mod.gemm("mx", oracle_mod.quantize(X, "mx", "rtn", False),
                            oracle_mod.quantize(W, "mx", "rtn", False))
    scale = np.abs(xf) @ np.abs(wf).T
    # both are FP4 approximations of X W^T; the rotated one is not farther off
    err_h = np.abs(Ch - exact).sum() / scale.sum()
    err_p = np.abs(Cp - exact).sum() / scale.sum()
    assert err_h < 0.1 and err_h <= err_p * 1.05


def test_empty_and_degenerate(oracle_mod):
    q = (np.zeros((0, 16), np.uint8), np.zeros((0, 1), np.uint8), None)
    r = (np.zeros((3, 16), np.uint8), np.zeros((3, 1), np.uint8), None)
    C, S = oracle_mod.gemm("mx", q, r)
    assert C.shape == (0, 3)
    # all-zero codes: exactly zero, with zero error scale
    C, S = oracle_mod.gemm("mx", r, r)
    assert not C.any() and not S.any()
