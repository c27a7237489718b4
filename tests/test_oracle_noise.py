"""Pins of the oracle's quantization-noise statistics (the quantities of the
sqrt(3) threshold of "FP4 All the Way: Fully Quantized Training of LLMs",
abstract): hand-computed blocks, exact zero noise on grid points, the closed
form of the stochastic-rounding noise in expectation, norm preservation
under the block rotation, and the count of left-out NaN blocks."""
import numpy as np

import oracle
import workloads

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16(vals):
    return workloads.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_mx_hand_block():
    # one MX block: amax 6 -> scale 2^0; 1.25 is a tie between 1 and 1.5 and
    # goes to the even code (1.0): noise -0.25
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0], x[0, 31] = 1.25, 6.0
    xb = bf16(x)
    q = oracle.quantize(xb, "mx", "rtn")
    s0, s1, n = oracle.noise_stats(xb, q, "mx")
    assert (s0, s1, n) == (1.25 ** 2 + 36.0, 0.0625, 0.0)


def test_nv_hand_blocks():
    # amax_t = 2688 -> s_t = 1.  Block 0: 2688 -> s_b = 448, code 6, exact.
    # Block 1: 100 -> r = 100/6 -> smallest E4M3 >= r is 18; 100 * RN(1/18)
    # rounds to the code for 6, so Q = 108 and the noise is 8.
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0], x[0, 16] = 2688.0, 100.0
    xb = bf16(x)
    q = oracle.quantize(xb, "nv", "rtn")
    assert q[2] == 1.0 and q[1][0, 0] == 0x7E and oracle.e4m3_value(int(q[1][0, 1])) == 18.0
    s0, s1, n = oracle.noise_stats(xb, q, "nv")
    assert (s0, s1, n) == (2688.0 ** 2 + 100.0 ** 2, 64.0, 0.0)


def test_grid_points_have_no_noise():
    rng = np.random.default_rng(7)
    vals = GRID[rng.integers(0, 8, size=(8, 128))] * np.where(rng.random((8, 128)) < 0.5, -1.0, 1.0)
    vals[:, ::32] = 6.0                       # every block's amax is 6 -> scale 1
    vals *= 2.0 ** 3                          # then scale 2^3
    xb = bf16(vals)
    for rnd in ("rtn", "sr"):
        q = oracle.quantize(xb, "mx", rnd, seed=3)
        s0, s1, n = oracle.noise_stats(xb, q, "mx")
        assert s1 == 0.0 and n == 0.0
        assert s0 == float(np.sum(vals.astype(np.float64) ** 2))


def _sr_expected_noise(xb):
    """Closed form of E[(Q(y) - y)^2] for MXFP4 SR without rotation: per
    element scale^2 * frac (1 - frac) * delta^2, with lo <= a < hi the grid
    neighbours of a = |y| / scale and frac = (a - lo) / delta.  bf16 inputs
    put a on a 2^-16 lattice of the neighbour interval, so the 16-bit
    comparison realises frac exactly."""
    y = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    R, C = y.shape
    e = np.zeros((R, C // 32))
    for i in range(R):
        for b in range(C // 32):
            amax = np.max(np.abs(y[i, 32 * b:32 * b + 32]))
            k = int(np.ceil(np.log2(amax / 6.0))) if amax > 0 else -127
            while 6.0 * 2.0 ** (k - 1) >= amax and amax > 0:
                k -= 1
            while 6.0 * 2.0 ** k < amax:
                k += 1
            e[i, b] = k
    scale = np.repeat(2.0 ** e, 32, axis=1)
    a = np.minimum(np.abs(y) / scale, 6.0)
    lo = GRID[np.searchsorted(GRID, a, side="right") - 1]
    hi = GRID[np.minimum(np.searchsorted(GRID, a, side="left"), 7)]
    delta = np.where(hi > lo, hi - lo, 1.0)
    frac = np.where(hi > lo, (a - lo) / delta, 0.0)
    return float(np.sum(scale ** 2 * frac * (1.0 - frac) * delta ** 2))


def test_sr_noise_matches_closed_form_in_expectation():
    xb = workloads.small_normal_bf16((8, 256), 1.0, seed=11)
    expect = _sr_expected_noise(xb)
    draws = np.array([oracle.noise_stats(xb, oracle.quantize(xb, "mx", "sr", seed=s), "mx")[1]
                      for s in range(300)])
    se = draws.std(ddof=1) / np.sqrt(len(draws))
    assert abs(draws.mean() - expect) < 5 * se, (draws.mean(), expect, se)
    # and RTN is never noisier than SR's expectation on this input
    assert oracle.noise_stats(xb, oracle.quantize(xb, "mx", "rtn"), "mx")[1] < expect


def test_rotation_preserves_the_signal_norm():
    xb = workloads.small_t_bf16((16, 512), 4.0, seed=12)
    s0 = oracle.noise_stats(xb, oracle.quantize(xb, "mx", "rtn"), "mx")[0]
    s0h = oracle.noise_stats(xb, oracle.quantize(xb, "mx", "rtn", True), "mx", True)[0]
    assert abs(s0h - s0) <= 1e-6 * s0


def test_axis0_is_the_transpose():
    xb = workloads.small_normal_bf16((64, 96), 1.0, seed=13)
    a = oracle.noise_stats(xb, oracle.quantize(xb, "nv", "sr", axis=0, seed=4), "nv", axis=0)
    b = oracle.noise_stats(np.ascontiguousarray(xb.T), oracle.quantize(np.ascontiguousarray(xb.T), "nv", "sr",
                                                                         axis=1, seed=4), "nv", axis=1)
    assert abs(a[0] - b[0]) <= 1e-12 * a[0] and a[2] == b[2] == 0.0


def test_nan_blocks_are_left_out():
    x = workloads.small_normal_bf16((4, 64), 1.0, seed=14).copy()
    x[1, 40] = 0x7FC0
    q = oracle.quantize(x, "mx", "rtn")
    s0, s1, n = oracle.noise_stats(x, q, "mx")
    assert n == 32.0 and np.isfinite(s0) and np.isfinite(s1)
    x2 = x.copy()
    x2[1, 32:64] = 0
    s0b, s1b, _ = oracle.noise_stats(x2, oracle.quantize(x2, "mx", "rtn"), "mx")
    assert (s0, s1) == (s0b, s1b)
