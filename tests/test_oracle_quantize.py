"""Tensor-level pins of the oracle's quantizer: hand-worked examples, the
nearest-code property by exhaustive enumeration, scale placement, packing,
axis handling, NVFP4 tensor/block scales, stochastic-rounding unbiasedness,
and the qualitative claims the pages make about the formats.
"""
import json
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16_of(values):
    return workloads.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def code_values(c: np.ndarray) -> np.ndarray:
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


@pytest.mark.parametrize("name", ["mx_block_worked.json", "nv_block_worked.json"])
def test_hand_worked_examples(oracle_mod, name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    x = bf16_of(np.array(g["x"], dtype=np.float64).reshape(g["rows"], g["cols"]))
    # the hand-worked inputs are bf16-exact
    np.testing.assert_array_equal(workloads.bf16_bits_to_f32(x).ravel(), np.float32(g["x"]))
    codes, scales, ts = oracle_mod.quantize(x, g["fmt"], g["rounding"], False, 1, 0)
    assert codes.ravel().tolist() == g["codes"]
    assert scales.ravel().tolist() == g["scales"]
    if g["fmt"] == "nv":
        assert ts == g["tensor_scale"]


def _block_view(v, bs):
    return v.reshape(v.shape[0], -1, bs)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_rtn_picks_the_nearest_code_by_enumeration(oracle_mod, fmt):
    """For every element, no other of the 16 codes lies closer to the scaled
    input than the chosen one (ties broken towards the even code)."""
    x = workloads.small_t_bf16((64, 256), 3.0, seed=1, outlier_frac=0.02)
    codes, scales, ts = oracle_mod.quantize(x, fmt, "rtn")
    bs = 32 if fmt == "mx" else 16
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    c = unpack_codes(codes)
    if fmt == "mx":
        s = np.array([oracle_mod.e8m0_value(b) for b in range(256)])[scales]
        xs = _block_view(xf, bs) / s[..., None]
    else:
        sb = np.array([oracle_mod.e4m3_value(b) for b in range(256)], dtype=np.float32)[scales]
        d = (sb * np.float32(ts)).astype(np.float32)
        with np.errstate(divide="ignore"):
            inv = (np.float32(1.0) / d).astype(np.float32)
        xs = (_block_view(xf.astype(np.float32), bs) * inv[..., None]).astype(np.float32).astype(np.float64)
    xs = np.minimum(np.abs(xs), 6.0) * np.sign(xs)
    xs = xs.reshape(c.shape)
    chosen = np.abs(xs - code_values(c))
    all_codes = code_values(np.arange(16))
    dist = np.abs(xs[..., None] - all_codes[None, None, :])
    assert np.all(chosen <= dist.min(axis=-1) + 0.0)


def test_mx_scale_places_block_absmax_in_range(oracle_mod):
    x = workloads.small_normal_bf16((128, 512), 1.0, seed=2)
    codes, scales, _ = oracle_mod.quantize(x, "mx", "rtn")
    xf = _block_view(workloads.bf16_bits_to_f32(x).astype(np.float64), 32)
    amax = np.abs(xf).max(axis=-1)
    q = amax / 2.0 ** (scales.astype(np.float64) - 127)
    assert np.all((q > 3.0) & (q <= 6.0))


def test_roundtrip_on_grid_values(oracle_mod):
    """Inputs that are grid values times one power of two per block (with the
    block maximum in (3, 6] of that power) come back exactly."""
    rng = np.random.default_rng(4)
    R, C = 16, 128
    e = rng.integers(-20, 20, size=(R, C // 32))
    g = code_values(rng.integers(0, 16, size=(R, C)))
    g = _block_view(g, 32)
    g[..., 0] = rng.choice([4.0, 6.0, -4.0, -6.0], size=(R, C // 32))
    x = (g * 2.0 ** e[..., None]).reshape(R, C)
    xb = bf16_of(x)
    codes, scales, _ = oracle_mod.quantize(xb, "mx", "rtn")
    np.testing.assert_array_equal(oracle_mod.dequantize("mx", codes, scales), x.astype(np.float32))


def test_packing_even_low_nibble(oracle_mod):
    x = np.zeros((2, 64))
    x[0, 5] = 6.0      # odd k -> high nibble of byte 2
    x[1, 8] = -3.0     # even k -> low nibble of byte 4
    codes, scales, _ = oracle_mod.quantize(bf16_of(x), "mx", "rtn")
    assert codes[0, 2] == 0x70 and np.count_nonzero(codes[0]) == 1
    assert scales[0].tolist() == [127, 0]
    # -3 with absmax 3: e = -1, -3 / 0.5 = -6 -> code 0xF
    assert codes[1, 4] == 0x0F and scales[1].tolist() == [126, 0]


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("hadamard", [False, True])
def test_axis0_is_the_transpose_of_axis1(oracle_mod, fmt, hadamard):
    x = workloads.small_t_bf16((96, 64), 4.0, seed=3)
    a0 = oracle_mod.quantize(x, fmt, "rtn", hadamard, 0)
    a1 = oracle_mod.quantize(np.ascontiguousarray(x.T), fmt, "rtn", hadamard, 1)
    for u, v in zip(a0, a1):
        np.testing.assert_array_equal(u, v)


def test_nv_tensor_and_block_scales(oracle_mod):
    x = workloads.small_t_bf16((64, 256), 3.0, seed=5, outlier_frac=0.02)
    codes, scales, ts = oracle_mod.quantize(x, "nv", "rtn")
    xf = workloads.bf16_bits_to_f32(x)
    amax_t = float(np.abs(xf).max())
    assert ts == float(np.float32(amax_t) / np.float32(2688.0))
    # the block holding the tensor maximum takes the largest E4M3 scale
    blocks = _block_view(xf.astype(np.float64), 16)
    bmax = np.abs(blocks).max(axis=-1)
    i, j = np.unravel_index(np.argmax(bmax), bmax.shape)
    assert scales[i, j] == 0x7E
    # every block scale is the smallest E4M3 >= absmax / (6 s_t)
    e4 = np.array([oracle_mod.e4m3_value(b) for b in range(0x7F)])
    r = (bmax.astype(np.float32) / np.float32(6.0 * ts)).astype(np.float32)
    sb = e4[scales]
    assert np.all(sb >= r)
    assert np.all((scales == 0) | (e4[np.maximum(scales.astype(int) - 1, 0)] < r))


def test_nv_tiny_and_zero_tensors(oracle_mod):
    z = np.zeros((4, 32), dtype=np.uint16)
    codes, scales, ts = oracle_mod.quantize(z, "nv", "rtn")
    assert ts == 1.0 and not codes.any() and not scales.any()
    tiny = bf16_of(np.full((2, 32), 1e-37))
    codes, scales, ts = oracle_mod.quantize(tiny, "nv", "rtn")
    assert ts == 2.0 ** -117          # the floor keeps s_b * s_t a normal number


def test_nonfinite_blocks(oracle_mod):
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, 3] = np.inf
    x[1, 40] = np.nan
    x[1, 0] = 1.0
    for fmt, nanbyte in (("mx", 0xFF), ("nv", 0x7F)):
        codes, scales, ts = oracle_mod.quantize(bf16_of(x), fmt, "rtn")
        bs = 32 if fmt == "mx" else 16
        assert scales[0, 3 // bs] == nanbyte and scales[1, 40 // bs] == nanbyte
        assert not codes[0, :bs // 2].any()
        assert scales[1, 0] != nanbyte
        if fmt == "nv":
            assert ts == float(np.float32(1.0) / np.float32(2688.0))


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_sr_is_unbiased_over_seeds(oracle_mod, fmt):
    """Mean of the dequantized SR output over many seeds equals the input
    (up to the deterministic scale) within 6 standard errors."""
    x = workloads.small_normal_bf16((1, 64), 1.0, seed=6)
    n = 2000
    acc = np.zeros(64)
    acc2 = np.zeros(64)
    for s in range(n):
        codes, scales, ts = oracle_mod.quantize(x, fmt, "sr", seed=s)
        d = oracle_mod.dequantize(fmt, codes, scales, ts).astype(np.float64)[0]
        acc += d
        acc2 += d * d
    mean = acc / n
    var = np.maximum(acc2 / n - mean ** 2, 1e-30)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)[0]
    if fmt == "nv":
        # NV scales the element by a rounded reciprocal: the target is the
        # scaled value mapped back, which differs from x by a few ulp
        assert np.all(np.abs(mean - xf) <= 6 * np.sqrt(var / n) + 1e-6 * np.abs(xf))
    else:
        assert np.all(np.abs(mean - xf) <= 6 * np.sqrt(var / n) + 1e-12)


def test_sr_counts_match_probability_per_element(oracle_mod):
    """One fixed input, many counters: the fraction of round-ups per element
    passes a binomial test against t / 2^16."""
    from scipy.stats import binomtest
    vals = [1.0 + 2 ** -16, 1.25, 2.75, 0.1, 5.5]
    for v in vals:
        x = bf16_of(np.full((1, 4096), v))
        codes, scales, _ = oracle_mod.quantize(x, "mx", "sr", seed=9)
        e = int(scales[0, 0]) - 127
        a = float(workloads.bf16_bits_to_f32(x)[0, 0]) / 2.0 ** e
        lo = GRID[GRID <= a].max()
        hi = GRID[GRID >= a].min()
        c = unpack_codes(codes)[0]
        ups = int(np.sum(GRID[c & 7] == hi)) if hi != lo else 0
        p = np.floor((a - lo) / (hi - lo) * 65536) / 65536 if hi != lo else 0.0
        if 0 < p < 1:
            assert binomtest(ups, 4096, p).pvalue > 1e-4, v


def _rel_mse(x, y):
    return float(np.sum((x - y) ** 2) / np.sum(x ** 2))


def test_pages_claims_nvfp4_beats_mxfp4_and_rotation_helps(oracle_mod):
    """Qualitative claims (not parity): NVFP4 quantizes more accurately than
    MXFP4, and block Hadamard rotation reduces MXFP4 error on heavy-tailed
    data (Bridging the Gap ..., abstract and digest step 3)."""
    x = workloads.small_t_bf16((64, 1024), 4.0, seed=7)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    mx = oracle_mod.dequantize("mx", *oracle_mod.quantize(x, "mx", "rtn")[:2])
    nv_c, nv_s, nv_t = oracle_mod.quantize(x, "nv", "rtn")
    nv = oracle_mod.dequantize("nv", nv_c, nv_s, nv_t)
    assert _rel_mse(xf, nv) < _rel_mse(xf, mx)
    # rotated error, measured in the rotated domain (the rotation is orthonormal)
    c, s, _ = oracle_mod.quantize(x, "mx", "rtn", hadamard=True)
    yq = oracle_mod.dequantize("mx", c, s).astype(np.float64)
    y = np.stack([np.concatenate([oracle_mod.fwht32(r[k:k + 32]) for k in range(0, 1024, 32)])
                  for r in xf.astype(np.float32)]).astype(np.float64)
    assert _rel_mse(y, yq) < _rel_mse(xf, mx)


def test_pages_claim_fp_grid_beats_int4_on_heavy_tails(oracle_mod):
    """FP grids are denser near zero, so they fit Student-t data better than
    a uniform INT4 grid (digest of Bridging the Gap ..., grid discussion).
    INT4 here: symmetric -7..7 with a per-32-block absmax/7 scale."""
    x = workloads.small_t_bf16((64, 1024), 3.0, seed=8)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    b = _block_view(xf, 32)
    s = np.abs(b).max(axis=-1, keepdims=True) / 7.0
    s[s == 0] = 1.0
    int4 = (np.clip(np.round(b / s), -7, 7) * s).reshape(xf.shape)
    nv_c, nv_s, nv_t = oracle_mod.quantize(x, "nv", "rtn")
    nv = oracle_mod.dequantize("nv", nv_c, nv_s, nv_t)
    assert _rel_mse(xf, nv) < _rel_mse(xf, int4)


@pytest.mark.parametrize("axis", [0, 1])
def test_sr_stream_follows_the_stated_counter_layout(oracle_mod, axis):
    """The tensor-level SR draws element (i, k) of the contraction-major output
    with rnd16(seed, i*K + k, axis) -- the counter layout is a reading (the
    pages fix only stochastic rounding), so this pins the implementation to the
    stated layout, element by element."""
    x = workloads.small_normal_bf16((64, 96), 1.0, seed=15)
    seed = 0xABCDEF12345
    codes, scales, _ = oracle_mod.quantize(x, "mx", "sr", axis=axis, seed=seed)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    v = xf if axis == 1 else xf.T
    rows, K = v.shape
    c = unpack_codes(codes)
    for i in range(0, rows, 7):
        for k in range(0, K, 5):
            e = int(scales[i, k // 32]) - 127
            xs = v[i, k] / 2.0 ** e
            expect = oracle_mod.sr_code(xs, oracle_mod.rnd16(seed, i * K + k, axis))
            assert c[i, k] == expect, (i, k)


def test_rows_at_equals_the_whole_tensor():
    """quantize_rows_at (used to check samples of very large tensors) gives
    exactly the whole tensor's codes and scales on those rows, stochastic
    rounding stream included."""
    import oracle
    x = workloads.small_t_bf16((64, 512), 3.0, seed=91)
    for rnd, had in (("sr", False), ("sr", True), ("rtn", True)):
        full = oracle.quantize(x, "mx", rnd, had, 1, 12)
        for r0, r1 in ((0, 5), (17, 40), (63, 64)):
            part = oracle.quantize_rows_at(x[r0:r1], r0, rnd, had, 12)
            assert np.array_equal(full[0][r0:r1], part[0]) and np.array_equal(full[1][r0:r1], part[1])
