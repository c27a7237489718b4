"""Pins of the oracle's Q-EMA weight quantizer.

"Oscillation-Reduced MXFP4 Training for Vision Transformers" (abstract) names
Q-EMA among its methods against weight oscillation but gives no rule: the
method is PARITY UNPINNED.  The reading (an EMA of the latent weights in
binary32, m <- RN(RN(beta m) + RN((1 - beta) w)), quantized MXFP4 RTN along
its rows) is pinned here for its own arithmetic: a hand-worked block, the
special cases beta = 0 (the latent weights themselves) and beta = 1 (the state
unchanged), the exact real EMA within its rounding bound, and the binary32
quantizer against the bf16 one and against brute force."""
import json
import os
from fractions import Fraction as Fr

import numpy as np

import oracle
import workloads

MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def y_of(xb):
    return (xb.astype(np.uint32) << 16).view(np.float32)


def test_hand_worked_block():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "qema_worked.json")))
    m = np.full((1, 32), 0.5, dtype=np.float32)
    w = np.full((1, 32), 0.25, dtype=np.float32)
    m[0, 0], w[0, 0] = 4.0, 8.0
    m[0, 1], w[0, 1] = 1.0, -1.0
    m2, (codes, scales, _) = oracle.qema_quantize(workloads.f32_to_bf16_bits(w), m, g["beta"])
    assert m2[0, 0] == g["expected_ema"]["0"] and m2[0, 1] == g["expected_ema"]["1"]
    assert np.all(m2[0, 2:] == g["expected_ema"]["rest"])
    assert scales.tolist() == [[g["expected_scale_byte"]]]
    assert codes.ravel().tolist() == g["expected_codes"]


def test_beta_zero_quantizes_the_latent_weights_and_one_keeps_the_state():
    w = workloads.small_normal_bf16((64, 256), 0.02, seed=101)
    rng = np.random.default_rng(102)
    m = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    m0, q0 = oracle.qema_quantize(w, m, 0.0)
    assert np.array_equal(m0, y_of(w))
    ref = oracle.quantize(w, "mx", "rtn")
    assert np.array_equal(q0[0], ref[0]) and np.array_equal(q0[1], ref[1])
    m1, q1 = oracle.qema_quantize(w, m, 1.0)
    assert np.array_equal(m1, m)
    ref = oracle.quantize_f32(m, "mx", "rtn")
    assert np.array_equal(q1[0], ref[0]) and np.array_equal(q1[1], ref[1])


def test_ema_within_its_rounding_bound_of_the_exact_average():
    """|m' - (beta m + (1 - beta) w)| <= |beta m| u + |c w| u + |m'| u + |c - (1 - beta)| |w|,
    u = 2^-24 (three binary32 roundings and the rounded coefficient)."""
    w = workloads.small_t_bf16((16, 64), 3.0, seed=103)
    rng = np.random.default_rng(104)
    m = rng.standard_normal((16, 64)).astype(np.float32)
    for beta in (0.9, 0.99, 0.3):
        m2, _ = oracle.qema_quantize(w, m, beta)
        b = Fr(float(np.float32(beta)))
        c = Fr(float(np.float32(1.0) - np.float32(beta)))
        u = Fr(1, 2 ** 24)
        for i in range(16):
            for k in range(64):
                mv, wv = Fr(float(m[i, k])), Fr(float(y_of(w)[i, k]))
                exact = b * mv + (1 - b) * wv
                got = Fr(float(m2[i, k]))
                bound = (abs(b * mv) + abs(c * wv) + abs(got)) * u + abs(c - (1 - b)) * abs(wv)
                assert abs(got - exact) <= bound, (beta, i, k)


def test_f32_quantizer_matches_bf16_and_brute_force():
    xb = workloads.small_t_bf16((32, 128), 3.0, seed=105)
    for had in (False, True):
        a = oracle.quantize(xb, "mx", "rtn", had)
        b = oracle.quantize_f32(y_of(xb), "mx", "rtn", had)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # non-bf16 values: every code is the nearest magnitude (ties to the even code)
    rng = np.random.default_rng(106)
    x = (rng.standard_normal((8, 64)) * 3).astype(np.float32)
    codes, scales, _ = oracle.quantize_f32(x, "mx", "rtn")
    for i in range(8):
        for blk in range(2):
            e = int(scales[i, blk]) - 127
            for j in range(32):
                k = 32 * blk + j
                c = (int(codes[i, k // 2]) >> (4 * (k & 1))) & 0xF
                a = min(abs(float(x[i, k])) / 2.0 ** e, 6.0)
                d = np.abs(MAG - a)
                best = [n for n in range(8) if d[n] == d.min()]
                want = min(best, key=lambda n: n % 2)
                assert (c & 7) == want and ((c >> 3) == int(np.signbit(x[i, k])))
