"""Pins of the oracle's element rounding and random stream.

Round-to-nearest (forward pass) and stochastic rounding (backward and update
passes) are the rounding choices of "FP4 All the Way: Fully Quantized Training
of LLMs" (abstract).  The RTN tie rule, the SR resolution (16 random bits) and
the Philox counter layout are readings; see the oracle's header.
"""
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import workloads

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def rtn_reference(xs: np.ndarray) -> np.ndarray:
    """Independent formulation of round-to-nearest-even onto E2M1: on each
    binade the grid is evenly spaced (0.5 on [0, 2), 1 on [2, 4), 2 on
    [4, 6]); numpy's half-to-even rounding of x/step picks the nearest point
    and resolves ties to the even multiple, which is the even-mantissa code."""
    a = np.minimum(np.abs(xs), 6.0)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    v = np.round(a / step) * step            # np.round: half to even
    v = np.minimum(v, 6.0)
    code = np.searchsorted(GRID, v)
    assert np.all(GRID[code] == v)
    return code | np.where(np.signbit(xs), 8, 0)


def test_rtn_exhaustive_bf16_times_scales(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    x32 = bits.view(np.float32)
    x = x32[np.isfinite(x32)].astype(np.float64)
    for e in (-127, -10, -1, 0, 1, 10, 126):
        xs = x * 2.0 ** (-e)
        ours = np.array([oracle_mod.rtn_code(v) for v in xs.tolist()])
        np.testing.assert_array_equal(ours, rtn_reference(xs), err_msg=f"e={e}")


def test_rtn_ties_and_saturation(oracle_mod):
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (6.0, 7), (7.0, 7), (1e30, 7), (0.0, 0), (-0.0, 8), (-0.1, 8), (-5.0, 14), (-5.01, 15)]
    for v, c in cases:
        assert oracle_mod.rtn_code(v) == c, v


def _sr_exact_fraction(a: float):
    a = min(abs(a), 6.0)
    fa = Fraction(a)
    lo = max(g for g in GRID if g <= a)
    hi = min(g for g in GRID if g >= a)
    if lo == hi:
        return lo, hi, Fraction(0)
    return lo, hi, (fa - Fraction(lo)) / (Fraction(hi) - Fraction(lo))


@pytest.mark.parametrize("xs", [0.3, 0.5000152587890625, 0.74, 1.0 + 2 ** -17, 1.3, 1.999,
                                2.2, 3.999, 4.5, 5.9, -2.7, 6.0, 1.5, -0.0, 2 ** -30, 100.0])
def test_sr_enumeration_over_all_random_words(oracle_mod, xs):
    """Over all 2^16 values of the 16 random bits the number that round up
    equals t = floor(frac * 2^16), so P(up) is within 2^-16 of the exact
    fraction (a - lo)/(hi - lo) and never above it."""
    lo, hi, frac = _sr_exact_fraction(xs)
    codes = np.array([oracle_mod.sr_code(xs, r) for r in range(65536)])
    mags = GRID[codes & 7]
    assert set(np.unique(mags)).issubset({lo, hi})
    ups = int(np.sum(mags == hi)) if hi != lo else 0
    t = int(frac * 65536)        # floor for a non-negative Fraction
    assert ups == t
    assert Fraction(ups, 65536) <= frac < Fraction(ups + 1, 65536)
    assert np.all((codes >> 3) == (1 if np.signbit(xs) else 0))


def test_sr_exact_for_bf16_mx_inputs(oracle_mod):
    """Every bf16 input scaled by a power of two has a rounding fraction with
    at most 16 fractional bits when a >= 2^-10: SR is then exactly unbiased."""
    rng = np.random.default_rng(3)
    bits = (rng.integers(0, 0x7F80, size=400).astype(np.uint32) << np.uint32(16))
    for v in bits.view(np.float32).tolist():
        e = oracle_mod.mx_scale_exponent(v * 1.37) if v > 0 else -127
        xs = v / 2.0 ** e
        if abs(xs) < 2 ** -10:
            continue
        lo, hi, frac = _sr_exact_fraction(xs)
        t = int(frac * 65536)
        assert Fraction(t, 65536) == frac


def _rocrand_reference(lines):
    """Philox4x32-10 from rocRAND's engine (host build of its header)."""
    src = os.path.join(os.path.dirname(__file__), "helpers", "philox_rocrand_ref.cpp")
    exe = os.path.join(os.environ.get("TMPDIR", "/tmp"), "mxfp4_philox_rocrand_ref")
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(src):
        subprocess.run([hipcc, "-O1", "-o", exe, src], check=True, capture_output=True)
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         check=True).stdout.split("\n")
    return [list(map(int, o.split())) for o in out if o.strip()]


def test_philox_matches_rocrand(oracle_mod):
    rng = np.random.default_rng(11)
    cases = [(0, 0, 0, 0, 0), (0, 1, 0, 0, 0), (2 ** 64 - 1, 2 ** 32 - 1, 2 ** 30 - 1, 1, 0),
             (12345, 77, 0, 1, 0), (0xDEADBEEFCAFEF00D, 123456789, 5, 0, 0)]
    for _ in range(200):
        # the helper reaches a counter by skipping 4 * block outputs, so the
        # block index (words 0 and 1) stays below 2^62
        cases.append((int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 32)),
                      int(rng.integers(0, 2 ** 30)), int(rng.integers(0, 2)), 0))
    ref = _rocrand_reference(["%d %d %d %d %d" % c for c in cases])
    assert len(ref) == len(cases)
    for (seed, c0, c1, c2, c3), r in zip(cases, ref):
        key = [seed & 0xFFFFFFFF, seed >> 32]
        ours = oracle_mod.philox4x32_10([c0, c1, c2, c3], key)
        assert list(map(int, ours)) == r, (seed, c0, c1, c2, c3)


def test_rnd16_counter_layout(oracle_mod):
    """Element L takes half (L & 1) of word (L & 7) / 2 of the Philox block
    for counter (L >> 3, axis) under key = seed."""
    seed = 0x0123456789ABCDEF
    for axis in (0, 1):
        for L in [0, 1, 2, 7, 8, 9, 1000, 2 ** 33 + 5]:
            g = L >> 3
            w = oracle_mod.philox4x32_10([g & 0xFFFFFFFF, g >> 32, axis, 0],
                                         [seed & 0xFFFFFFFF, seed >> 32])
            expect = (int(w[(L & 7) >> 1]) >> (16 * (L & 1))) & 0xFFFF
            assert oracle_mod.rnd16(seed, L, axis) == expect


def test_rnd16_is_uniform(oracle_mod):
    vals = np.array([oracle_mod.rnd16(7, L, 1) for L in range(40000)])
    # mean of U{0..65535} is 32767.5, sd 18918; 6 sigma of the mean
    assert abs(vals.mean() - 32767.5) < 6 * 18918 / np.sqrt(len(vals))
    # low and high halves of the words are both used
    assert len(np.unique(vals)) > 28000
