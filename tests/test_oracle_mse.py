"""Pins of the oracle's MSE-fitted scales (the digest of the MR-GPTQ paper,
step 1: the grid is fitted for mean squared error, block scales and the
tensor scale in turn).

Reading: each block keeps, among the scales at or below its absmax scale, the
one whose round-to-nearest encoding has the smallest squared error (a tie
keeps the larger scale); the NVFP4 tensor step is the least-squares scale for
fixed bytes and codes.  The pins check the oracle against exact rational
arithmetic written here from that definition (every candidate scale tried,
no search cut), against hand-worked blocks in which the lowest scale the
GPU search tries wins (MXFP4 e0 - 1, NVFP4 b0 - 5), and check that the
checker the GPU tests use flags a planted wrong choice."""
import json
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
import workloads

MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mse_blocks_worked.json")


def y_of(xb):
    return (xb.astype(np.uint32) << 16).view(np.float32)


def rtn_idx(a):
    """Nearest E2M1 magnitude index of a >= 0 (saturating at 6), ties to the
    even code: brute force over the 8 magnitudes."""
    a = min(abs(float(a)), 6.0)
    return min(range(8), key=lambda i: (abs(a - MAG[i]), i % 2))


def e4m3(b):
    e, m = b >> 3, b & 7
    return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)


def mx_errors(y):
    """{exponent: exact squared error} for every exponent from the absmax one
    down to -127 (no cut)."""
    amax = max(abs(float(v)) for v in y)
    e0 = -127 if amax == 0 else next(e for e in range(-127, 128) if 6.0 * 2.0 ** e >= amax)
    out = {}
    for e in range(e0, -128, -1):
        s = Fr(2) ** e
        out[e] = sum((Fr(float(v)) - (-1 if np.signbit(v) else 1) * Fr(MAG[rtn_idx(Fr(float(v)) / s)]) * s) ** 2
                     for v in y)
    return out


def nv_errors(y, st):
    """{byte: exact squared error} for every E4M3 byte from the absmax one
    down to 1 (no cut); elements encoded as RN(y * RN(1 / RN(s_b * s_t)))."""
    st = np.float32(st)
    amax = np.float32(max(abs(float(v)) for v in y))
    r = np.float32(amax / np.float32(np.float32(6.0) * st))
    b0 = next((b for b in range(0, 127) if e4m3(b) >= float(r)), 126)
    out = {}
    for b in range(b0, 0, -1):
        sb = np.float32(e4m3(b))
        inv = np.float32(np.float32(1.0) / np.float32(sb * st))
        tot = Fr(0)
        for v in y:
            q = np.float32(np.float32(v) * inv)
            val = (-1 if np.signbit(q) else 1) * Fr(MAG[rtn_idx(q)]) * Fr(float(sb)) * Fr(float(st))
            tot += (Fr(float(v)) - val) ** 2
        out[b] = tot
    return out, b0


def argmin_larger_first(errs):
    best = None
    for s in sorted(errs, reverse=True):     # larger scale first: a tie keeps it
        if best is None or errs[s] < errs[best]:
            best = s
    return best


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_block_choice_is_the_exact_argmin_over_all_smaller_scales(fmt):
    xb = workloads.small_t_bf16((6, 256), 3.0, seed=61, outlier_frac=0.03)
    codes, scales, st = oracle.quantize_mse(xb, fmt, False, 1, 0)
    y = y_of(xb)
    bs = 32 if fmt == "mx" else 16
    for i in range(y.shape[0]):
        for b in range(y.shape[1] // bs):
            blk = y[i, b * bs:(b + 1) * bs]
            if fmt == "mx":
                want = argmin_larger_first(mx_errors(blk)) + 127
            else:
                errs, b0 = nv_errors(blk, st)
                want = argmin_larger_first(errs) if b0 > 0 else 0
            assert scales[i, b] == want, (fmt, i, b, int(scales[i, b]), want)


def test_lowest_searched_scales_win_on_hand_worked_blocks():
    g = json.load(open(GOLDEN))
    mxb = np.full((1, 32), 0.25, dtype=np.float32)
    mxb[0, 5] = 3.25
    q = oracle.quantize_mse(workloads.f32_to_bf16_bits(mxb), "mx", False, 1, 0)
    assert q[1].tolist() == [[g["mx_block"]["expected_scale_byte"]]]
    assert q[0].ravel().tolist() == g["mx_block"]["expected_codes"]

    nvb = np.zeros((2, 16), dtype=np.float32)
    nvb[0] = [0.087890625] * 7 + [0.140625] * 6 + [0.15234375] * 2 + [0.1884765625]
    nvb[1, 0] = 2688.0
    xb = workloads.f32_to_bf16_bits(nvb)
    assert np.array_equal(y_of(xb), nvb)
    q = oracle.quantize_mse(xb, "nv", False, 1, 0)
    assert q[2] == 1.0
    assert q[1].ravel().tolist() == g["nv_block"]["expected_scale_bytes"]
    assert q[0][0].tolist() == g["nv_block"]["expected_codes_row0"]
    assert q[0][1].tolist() == g["nv_block"]["expected_codes_row1"]
    # the two errors of the derivation, from the exact definition here
    errs, b0 = nv_errors(nvb[0], 1.0)
    assert b0 == 17
    assert errs[17] == Fr(*g["nv_block"]["expected_error_b0"])
    assert errs[12] == Fr(*g["nv_block"]["expected_error_chosen"])
    # the absmax quantizer keeps b0
    assert oracle.quantize(xb, "nv", "rtn")[1][0, 0] == 17


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_never_worse_than_absmax_per_block(fmt):
    xb = workloads.small_t_bf16((32, 512), 4.0, seed=62)
    bs = 32 if fmt == "mx" else 16
    qa = oracle.quantize(xb, fmt, "rtn")
    qm = oracle.quantize_mse(xb, fmt, False, 1, 0)
    da = oracle.dequantize(fmt, *qa).astype(np.float64)
    dm = oracle.dequantize(fmt, *qm).astype(np.float64)
    y = y_of(xb).astype(np.float64)
    ea = ((y - da) ** 2).reshape(32, -1, bs).sum(-1)
    em = ((y - dm) ** 2).reshape(32, -1, bs).sum(-1)
    assert np.all(em <= ea * (1 + 1e-12))
    assert em.sum() < ea.sum()


def rn_f32(fr: Fr) -> np.float32:
    """Round a positive rational to the nearest binary32 (ties to even)."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
    d = [abs(Fr(float(c)) - fr) for c in cands]
    m = min(d)
    best = [c for c, dd in zip(cands, d) if dd == m]
    return min(best, key=lambda c: int(np.float32(c).view(np.uint32)) & 1)


def test_nv_tensor_step_is_the_exact_least_squares_scale():
    xb = workloads.small_t_bf16((24, 128), 3.0, seed=63, outlier_frac=0.01)
    c0, s0, st0 = oracle.quantize_mse(xb, "nv", False, 1, 0)
    _, _, st1 = oracle.quantize_mse(xb, "nv", False, 1, 1)
    y = y_of(xb)
    num, den = Fr(0), Fr(0)
    for i in range(24):
        for k in range(128):
            code = (int(c0[i, k // 2]) >> (4 * (k & 1))) & 0xF
            p = (-1 if code & 8 else 1) * Fr(MAG[code & 7]) * Fr(e4m3(int(s0[i, k // 16])))
            num += Fr(float(y[i, k])) * p
            den += p * p
    assert np.float32(st1) == rn_f32(num / den), (st1, float(num / den))
    assert st1 != st0
    # the oracle's separate tensor step gives the same scale from the same bytes
    assert oracle.mse_tensor_step(xb, (c0, s0, st0), False, 1, st0) == st1


def test_alternation_lowers_the_error_here():
    """Observed on this input (not a theorem: the candidate set moves with
    the tensor scale): the squared error does not grow over the rounds."""
    xb = workloads.small_t_bf16((64, 256), 3.0, seed=64)
    y = y_of(xb).astype(np.float64)
    errs = []
    for it in range(4):
        q = oracle.quantize_mse(xb, "nv", False, 1, it)
        errs.append(float(np.sum((y - oracle.dequantize("nv", *q)) ** 2)))
    assert all(b <= a for a, b in zip(errs, errs[1:])), errs
    assert errs[-1] < float(np.sum((y - oracle.dequantize("nv", *oracle.quantize(xb, "nv", "rtn"))) ** 2))


def test_grid_exact_blocks_keep_the_absmax_scale():
    rng = np.random.default_rng(65)
    vals = MAG[rng.integers(0, 8, size=(4, 128))] * 2.0 ** 5
    vals[:, ::32] = 6.0 * 2.0 ** 5
    xb = workloads.f32_to_bf16_bits(vals.astype(np.float32))
    qa = oracle.quantize(xb, "mx", "rtn")
    qm = oracle.quantize_mse(xb, "mx", False, 1, 0)
    assert np.array_equal(qa[0], qm[0]) and np.array_equal(qa[1], qm[1])


def test_mse_rotated_and_transposed_match_definitions():
    """axis 0 is the transpose of axis 1; with the rotation the error is
    still no worse than the absmax quantizer's, block by block."""
    xb = workloads.small_normal_bf16((64, 96), 1.0, seed=66)
    a0 = oracle.quantize_mse(xb, "nv", False, 0, 1)
    a1 = oracle.quantize_mse(np.ascontiguousarray(xb.T), "nv", False, 1, 1)
    assert all(np.array_equal(u, v) for u, v in zip(a0[:2], a1[:2])) and a0[2] == a1[2]
    xh = workloads.small_t_bf16((16, 256), 4.0, seed=67)
    qa = oracle.quantize(xh, "mx", "rtn", True)
    qm = oracle.quantize_mse(xh, "mx", True, 1, 0)
    ya = oracle.dequantize("mx", *qa).astype(np.float64)
    ym = oracle.dequantize("mx", *qm).astype(np.float64)
    # the rotated operand, through the oracle's own rotation
    y = np.stack([np.concatenate([oracle.fwht32(y_of(xh)[i, 32 * b:32 * b + 32]) for b in range(8)])
                  for i in range(16)]).astype(np.float64)
    assert np.all(((y - ym) ** 2).reshape(16, 8, 32).sum(-1) <= ((y - ya) ** 2).reshape(16, 8, 32).sum(-1) * (1 + 1e-12))


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_checker_accepts_the_oracle_and_flags_planted_mistakes(fmt):
    """The checker the GPU tests rely on: the oracle's own output passes; a
    block moved to another candidate (re-encoded consistently) fails the
    error test; a flipped code fails the encoding test."""
    xb = workloads.small_t_bf16((16, 128), 3.0, seed=68, outlier_frac=0.05)
    q = oracle.quantize_mse(xb, fmt, False, 1, 0)
    r = oracle.mse_check(xb, q, fmt, False, 1)
    assert r["bad_encoding"] == 0 and r["bad_error"] == 0 and r["differ_from_oracle"] == 0
    bs = 32 if fmt == "mx" else 16
    qa = oracle.quantize(xb, fmt, "rtn")
    # a block where the MSE choice is not the absmax scale: give it the absmax
    # choice (a valid candidate with a larger error)
    diff = np.argwhere(qa[1] != q[1])
    assert len(diff) > 0
    i, b = diff[0]
    codes, scales = q[0].copy(), q[1].copy()
    scales[i, b] = qa[1][i, b]
    codes[i, b * bs // 2:(b + 1) * bs // 2] = qa[0][i, b * bs // 2:(b + 1) * bs // 2]
    r = oracle.mse_check(xb, (codes, scales, q[2]), fmt, False, 1, rel_tol=1e-12)
    assert r["bad_error"] == 1 and r["bad_encoding"] == 0 and r["first_bad"] == i * (128 // bs) + b
    codes2 = q[0].copy()
    codes2[3, 2] ^= 0x01
    r = oracle.mse_check(xb, (codes2, q[1], q[2]), fmt, False, 1)
    assert r["bad_encoding"] == 1 and r["first_bad"] == 3 * (128 // bs) + 2 * 2 // bs
