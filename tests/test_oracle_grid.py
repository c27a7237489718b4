"""Pins of the oracle's MXFP4 quantizer with a fixed grid scale (the digest
of "Bridging the Gap Between Promise and Performance for Microscaling FP4
Quantization", step 1: for MXFP4 with Hadamard rotations one fixed grid
scale serves every model; no value is given, so alpha is an argument).
Reading: each block's exponent is chosen for RN(alpha * absmax)."""
import numpy as np
import pytest

import oracle
import workloads

MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def y_of(xb):
    return (xb.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("had,axis", [(False, 1), (True, 1), (True, 0)])
def test_alpha_one_is_the_absmax_quantizer(had, axis):
    xb = workloads.small_t_bf16((64, 256), 3.0, seed=130)
    a = oracle.quantize(xb, "mx", "rtn", had, axis)
    b = oracle.quantize_grid(xb, 1.0, had, axis)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_hand_worked_block():
    """Block of 32: one 5.0, the rest 0.25; alpha = 0.5.  RN(0.5 * 5) = 2.5:
    e = -1 (6 * 2^-1 = 3 >= 2.5 > 1.5), byte 126.  5 / 0.5 = 10 saturates to 6
    (code 0x7); 0.25 / 0.5 = 0.5 (code 0x1).  With alpha = 1: e = 0 (byte 127),
    5 -> tie 4/6 -> 4 (0x6), 0.25 -> tie 0/0.5 -> 0 (0x0)."""
    v = np.full((1, 32), 0.25, dtype=np.float32)
    v[0, 0] = 5.0
    xb = workloads.f32_to_bf16_bits(v)
    c, s, _ = oracle.quantize_grid(xb, 0.5, False, 1)
    assert s.tolist() == [[126]]
    assert c.ravel().tolist() == [0x17] + [0x11] * 15
    c1, s1, _ = oracle.quantize_grid(xb, 1.0, False, 1)
    assert s1.tolist() == [[127]] and c1.ravel().tolist() == [0x06] + [0x00] * 15


def test_codes_are_nearest_for_the_chosen_scale_and_scale_follows_alpha():
    xb = workloads.small_normal_bf16((32, 128), 1.0, seed=131)
    y = y_of(xb)
    for alpha in (0.6, 0.75, 1.3):
        c, s, _ = oracle.quantize_grid(xb, alpha, False, 1)
        for i in range(32):
            for b in range(4):
                blk = y[i, 32 * b:32 * b + 32]
                a = float(np.float32(np.float32(alpha) * np.float32(np.abs(blk).max())))
                e = next(e for e in range(-127, 128) if 6.0 * 2.0 ** e >= a)
                assert s[i, b] == e + 127
                for j in range(32):
                    k = 32 * b + j
                    code = (int(c[i, k // 2]) >> (4 * (k & 1))) & 0xF
                    t = min(abs(float(blk[j])) / 2.0 ** e, 6.0)
                    d = np.abs(MAG - t)
                    want = min([n for n in range(8) if d[n] == d.min()], key=lambda n: n % 2)
                    assert (code & 7) == want


def test_a_grid_scale_below_one_lowers_the_error_on_rotated_gaussian_weights():
    """The page's claim, observed here (not a pin of a value): on rotated
    Gaussian weights some alpha < 1 gives less squared error than alpha = 1."""
    xb = workloads.small_normal_bf16((256, 512), 0.02, seed=132)
    y = np.stack([np.concatenate([oracle.fwht32(y_of(xb)[i, 32 * b:32 * b + 32]) for b in range(16)])
                  for i in range(256)]).astype(np.float64)

    def err(alpha):
        q = oracle.quantize_grid(xb, alpha, True, 1)
        return float(np.sum((y - oracle.dequantize("mx", *q)) ** 2))
    e1 = err(1.0)
    assert min(err(a) for a in (0.6, 0.7, 0.8, 0.9)) < e1
