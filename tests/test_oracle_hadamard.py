"""Pins of the oracle's block-wise Hadamard rotation.

Block-wise (block-diagonal) Hadamard rotations: "Bridging the Gap Between
Promise and Performance for Microscaling FP4 Quantization" (abstract) and its
digest (step 3).  READING: 32 x 32 Sylvester blocks normalised by 1/sqrt(32),
evaluated as a binary32 butterfly.  Pinned against scipy's Hadamard matrix,
exact integer arithmetic, the orthonormality H H^T = 32 I and the binary32
rounding of the normalisation constant.
"""
from decimal import Decimal, getcontext

import numpy as np
import scipy.linalg


def test_normalisation_constant_is_nearest_float(oracle_mod):
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(32).sqrt()
    c = np.float32(oracle_mod.hadamard_scale())
    up = np.nextafter(c, np.float32(1))
    dn = np.nextafter(c, np.float32(0))
    d = abs(Decimal(float(c)) - exact)
    assert d < abs(Decimal(float(up)) - exact) and d < abs(Decimal(float(dn)) - exact)


def test_unit_vectors_give_scipy_hadamard_columns(oracle_mod):
    H = scipy.linalg.hadamard(32)
    c = np.float32(oracle_mod.hadamard_scale())
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=H.dtype))
    for j in range(32):
        e = np.zeros(32, dtype=np.float32)
        e[j] = 1.0
        y = oracle_mod.fwht32(e)
        np.testing.assert_array_equal(y, (H[:, j] * c).astype(np.float32))


def test_integer_inputs_exact_against_matrix_product(oracle_mod):
    """Small integers make every butterfly sum exact; the result is then one
    binary32 rounding of (H x) * c."""
    H = scipy.linalg.hadamard(32).astype(np.int64)
    c = np.float32(oracle_mod.hadamard_scale())
    rng = np.random.default_rng(0)
    for _ in range(200):
        x = rng.integers(-1000, 1000, size=32)
        y = oracle_mod.fwht32(x.astype(np.float32))
        ref = (H @ x).astype(np.float32) * c     # exact sum, one rounding in float32
        np.testing.assert_array_equal(y, ref)


def test_norm_preserved_and_involution(oracle_mod):
    rng = np.random.default_rng(1)
    u = 2.0 ** -24
    for _ in range(300):
        x = (rng.standard_normal(32) * 10 ** rng.uniform(-3, 3)).astype(np.float32)
        y = oracle_mod.fwht32(x)
        nx, ny = np.linalg.norm(x.astype(np.float64)), np.linalg.norm(y.astype(np.float64))
        assert abs(ny - nx) <= 10 * u * nx
        # orthonormal and symmetric: rotating twice returns the input
        z = oracle_mod.fwht32(y)
        np.testing.assert_allclose(z, x, rtol=0, atol=20 * u * np.abs(x).max())
        # matches x H / sqrt(32) in double precision within the butterfly's error
        ref = scipy.linalg.hadamard(32) @ x.astype(np.float64) / np.sqrt(32.0)
        assert np.max(np.abs(y - ref)) <= 10 * u * np.abs(x).sum()


def test_sign_of_zero_follows_butterfly(oracle_mod):
    """x[i] - x[i+h] with equal operands is +0, and the butterfly order is the
    stated one: a vector with x[0] = x[1] = 1 gives +0 (not -0) in slot 1."""
    x = np.zeros(32, dtype=np.float32)
    x[0] = x[1] = 1.0
    y = oracle_mod.fwht32(x)
    assert y[1] == 0.0 and not np.signbit(y[1])


def test_stride_order_on_a_hand_worked_vector(oracle_mod):
    """The butterfly's evaluation order decides binary32 bits: for x = (2^24,
    1, 1, 0, ...) strides 1, 2, 4, 8, 16 and the reverse order give different
    results in slots 1 and 2 (mod 4), worked by hand in the fixture."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fwht_stride_order.json")))
    x = np.zeros(32, dtype=np.float32)
    x[0], x[1], x[2] = 2.0 ** 24, 1.0, 1.0
    y = oracle_mod.fwht32(x)
    c = np.float64(np.float32(oracle_mod.hadamard_scale()))
    # v * c is exact in binary64 (24 + 24 bits), so this is one binary32 rounding
    want = np.array([np.float32(np.float64(g["unscaled_by_i_mod_4"][i % 4]) * c) for i in range(32)])
    other = np.array([np.float32(np.float64(g["other_order_unscaled_by_i_mod_4"][i % 4]) * c) for i in range(32)])
    assert not np.array_equal(want.view(np.uint32), other.view(np.uint32))
    np.testing.assert_array_equal(y.view(np.uint32), want.view(np.uint32))
