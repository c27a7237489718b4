"""Pins of the oracle's number formats (E2M1 elements, E8M0 and E4M3 scales).

E2M1 is named by "FP4 All the Way: Fully Quantized Training of LLMs"
(abstract); its eight magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} are the grid the
hot path's specification lists.  E8M0 (power-of-two scale) follows the MXFP4
power-of-two scale of "Bridging the Gap Between Promise and Performance for
Microscaling FP4 Quantization" (abstract); E4M3 is the NVFP4 block scale of the
FQT abstract.  Decoders are pinned against PyTorch's float8 dtypes, a library
implementation independent of the oracle.
"""
import math

import numpy as np
import torch

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_is_the_fp4_grid(oracle_mod):
    vals = [oracle_mod.e2m1_value(c) for c in range(16)]
    assert vals[:8] == GRID
    assert vals[8:] == [-g for g in GRID]
    assert math.copysign(1.0, vals[8]) == -1.0  # code 0x8 is -0
    # magnitudes strictly increase with the code: codes order like the values
    assert all(vals[i] < vals[i + 1] for i in range(7))


def test_e8m0_decode_matches_torch(oracle_mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    ours = np.array([oracle_mod.e8m0_value(b) for b in range(256)])
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(ours[:255], ref[:255])


def test_e4m3_decode_matches_torch(oracle_mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle_mod.e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert oracle_mod.e4m3_value(0x7E) == 448.0 and oracle_mod.e4m3_value(1) == 2.0 ** -9


def _e4m3_round_up_reference(r: float) -> int:
    """Independent derivation: torch's round-to-nearest E4M3 conversion, then
    step up one code if the nearest value is below r; saturate at 448."""
    if r > 448.0:
        return 0x7E
    b = int(torch.tensor([r], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    if b == 0x7F:          # rounds beyond 448 -> saturate
        return 0x7E
    v = float(torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])
    if v < r:
        b += 1
    return min(b, 0x7E)


def test_e4m3_round_up_dense_and_boundaries(oracle_mod):
    vals = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    probes = [0.0, 1e-30, 2.0 ** -10, 448.0, 448.5, 1e6]
    for v in vals:
        v32 = np.float32(v)
        probes += [float(v32), float(np.nextafter(v32, np.float32(np.inf))),
                   float(np.nextafter(v32, np.float32(0)))]
    rng = np.random.default_rng(5)
    probes += list((10.0 ** rng.uniform(-4, 2.7, size=3000)).astype(np.float32).astype(float))
    for r in probes:
        r32 = float(np.float32(r))
        got = oracle_mod.e4m3_round_up(r32)
        assert got == _e4m3_round_up_reference(r32), r32
        # definition: smallest value >= r (or 448 when none exists)
        gv = oracle_mod.e4m3_value(got)
        assert gv >= r32 or got == 0x7E
        if got > 0:
            assert oracle_mod.e4m3_value(got - 1) < r32


def test_mx_scale_exponent_exhaustive_over_bf16(oracle_mod):
    """For every positive finite bf16 absmax the scale 2^e puts amax/2^e in
    (3, 6] -- inside the E2M1 range, and no smaller power of two would --
    except at the clamp e = -127."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << np.uint32(16)
    amaxes = bits.view(np.float32)
    for a in amaxes.tolist():
        e = oracle_mod.mx_scale_exponent(a)
        assert -127 <= e <= 127
        q = a / 2.0 ** e
        assert q <= 6.0
        if e > -127:
            assert q > 3.0
        else:
            assert a <= 6.0 * 2.0 ** -127
    assert oracle_mod.mx_scale_exponent(0.0) == -127
    assert oracle_mod.mx_scale_exponent(6.0) == 0
    assert oracle_mod.mx_scale_exponent(float(np.nextafter(np.float32(6), np.float32(7)))) == 1
    assert oracle_mod.mx_scale_exponent(3.0) == -1
    assert oracle_mod.mx_scale_exponent(float(np.nextafter(np.float32(3), np.float32(4)))) == 0
