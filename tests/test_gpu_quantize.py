"""GPU parity of the quantizer (HIP kernels through the C ABI) against the
CPU oracle: bit-exact codes, scale bytes and NVFP4 tensor scale."""
import numpy as np
import pytest

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_codes_equal

pytestmark = pytest.mark.gpu

COMBOS = [(f, r, h, a) for f in ("mx", "nv") for r in ("rtn", "sr") for h in (False, True) for a in (1, 0)]


def _run(mx, oracle_mod, bits, fmt, rnd, had, axis, seed=1234, pad=0, what=""):
    say("quantize", what, fmt, rnd, "H" if had else "-", f"axis{axis}", bits.shape, f"pad{pad}")
    x = to_device_bf16(bits, pad)
    q = mx.mxfp4_quantize(x, fmt, rnd, had, axis, seed)
    got = q_to_host(q)
    want = oracle_mod.quantize(bits, fmt, rnd, had, axis, seed)
    assert_codes_equal(got, want, f"{what} {fmt} {rnd} H={had} axis={axis}")


@pytest.mark.parametrize("fmt,rnd,had,axis", COMBOS)
def test_small_all_variants(oracle_mod, fmt, rnd, had, axis):
    mx = need_gpu()
    bits = workloads.small_t_bf16((96, 320), 3.0, seed=21, outlier_frac=0.03)
    _run(mx, oracle_mod, bits, fmt, rnd, had, axis, what="t3-outliers")


@pytest.mark.parametrize("fmt,rnd,had,axis", COMBOS)
def test_ragged_and_strided(oracle_mod, fmt, rnd, had, axis):
    """Row counts that are not multiples of any tile, padded row strides, and
    (NVFP4, axis 0) a contraction length with a 16-row tail."""
    mx = need_gpu()
    if axis == 1:
        shape = (37, 224)
    else:
        shape = (112 if (fmt == "nv" and not had) else 96, 45)
    bits = workloads.small_normal_bf16(shape, 0.7, seed=22)
    _run(mx, oracle_mod, bits, fmt, rnd, had, axis, pad=8, what="ragged-pad8")
    _run(mx, oracle_mod, bits, fmt, rnd, had, axis, pad=3, what="ragged-pad3")


@pytest.mark.parametrize("fmt,rnd,had", [(f, r, h) for f in ("mx", "nv") for r in ("rtn", "sr") for h in (False, True)])
def test_transpose_tile_edges(oracle_mod, fmt, rnd, had):
    """axis 0 through the LDS-tiled transpose: more than one 256-row tile with
    a ragged last one (a 16-row NVFP4 tail when unrotated), a column count
    that is a multiple of 8 but not of 64, packed and padded rows."""
    mx = need_gpu()
    shape = (304 if (fmt == "nv" and not had) else 288, 200)
    bits = workloads.small_t_bf16(shape, 3.0, seed=27, outlier_frac=0.02)
    _run(mx, oracle_mod, bits, fmt, rnd, had, 0, what="tile-edges")
    _run(mx, oracle_mod, bits, fmt, rnd, had, 0, pad=8, what="tile-edges-pad8")


def _offset_view(bits: np.ndarray, pad: int):
    """A device view whose first element sits 2 bytes past a 16-byte boundary."""
    import torch
    R, C = bits.shape
    ld = C + pad
    flat = np.zeros(R * ld + 1, dtype=np.uint16)
    flat[1:].reshape(R, ld)[:, :C] = bits
    t = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
    return t[1:].view(R, ld)[:, :C]


@pytest.mark.parametrize("fmt,rnd,had,axis", COMBOS)
def test_unaligned_input(oracle_mod, fmt, rnd, had, axis):
    """Inputs that are not 16-byte aligned take the element-load paths;
    packed (ldx == C) and padded rows."""
    mx = need_gpu()
    bits = workloads.small_normal_bf16((96, 256), 0.9, seed=28)
    for pad in (0, 5):
        say("quantize unaligned", fmt, rnd, had, axis, f"pad{pad}")
        q = mx.mxfp4_quantize(_offset_view(bits, pad), fmt, rnd, had, axis, 99)
        assert_codes_equal(q_to_host(q), oracle_mod.quantize(bits, fmt, rnd, had, axis, 99),
                           f"unaligned pad{pad} {fmt} {rnd} H={had} axis={axis}")


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("axis", [1, 0])
def test_special_values(oracle_mod, fmt, axis):
    """Zero blocks, NaN/Inf blocks, bf16 subnormals, huge values, exact ties
    and values straddling every rounding boundary."""
    mx = need_gpu()
    rng = np.random.default_rng(23)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[0, :] = 0.0
    x[1, :32] = -0.0
    x[2, 5] = np.inf
    x[3, 40] = np.nan
    x[4, :] = rng.standard_normal(256) * 1e-39          # subnormals
    x[5, :] = rng.standard_normal(256) * 1e37
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0])
    x[6, :] = np.resize(np.concatenate([ties, -ties]), 256)
    x[6, 0] = 6.0                                       # absmax 6 -> scale 1 for MX
    x[7, :] = np.resize(np.concatenate([ties * 1.0078125, ties * 0.9921875]), 256)
    x[8, :] = 1.0
    x[9, :] = np.ldexp(1.0, rng.integers(-130, 120, size=256)) * rng.choice([-1, 1], size=256)
    bits = workloads.f32_to_bf16_bits(x)
    for rnd in ("rtn", "sr"):
        for had in (False, True):
            _run(mx, oracle_mod, bits, fmt, rnd, had, axis, seed=77, what="special")


def test_nv_scale_rounding_sweep(oracle_mod):
    """Block maxima swept over many binades and every E4M3 mantissa step, so
    the E4M3 round-up of the kernels meets the oracle's brute force."""
    mx = need_gpu()
    rng = np.random.default_rng(24)
    R = 512
    x = rng.standard_normal((R, 64)).astype(np.float32) * 0.1
    peaks = np.ldexp(rng.uniform(1, 2, size=(R, 4)), rng.integers(-20, 12, size=(R, 4)))
    for b in range(4):
        x[:, 16 * b + 3] = peaks[:, b]
    x[0, 0] = 3000.0                                      # tensor max
    bits = workloads.f32_to_bf16_bits(x)
    for axis in (1, 0):
        _run(mx, oracle_mod, bits if axis == 1 else np.ascontiguousarray(bits.T), "nv", "rtn", False, axis,
             what="nv-scale-sweep")


def test_empty_inputs(oracle_mod):
    mx = need_gpu()
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = mx.mxfp4_quantize(x, "mx")
    assert q.codes.shape == (0, 32)
    q = mx.mxfp4_quantize(x, "nv")
    assert q.codes.shape == (0, 32)


def test_sr_seed_changes_codes_and_is_deterministic(oracle_mod):
    mx = need_gpu()
    bits = workloads.small_normal_bf16((64, 256), 1.0, seed=25)
    x = to_device_bf16(bits)
    a = q_to_host(mx.mxfp4_quantize(x, "mx", "sr", seed=1))
    b = q_to_host(mx.mxfp4_quantize(x, "mx", "sr", seed=1))
    c = q_to_host(mx.mxfp4_quantize(x, "mx", "sr", seed=2))
    assert np.array_equal(a[0], b[0])
    assert not np.array_equal(a[0], c[0])


FULL = [
    # (cfg, tensor, fmt, rounding, hadamard, axis)
    (0, "A", "mx", "rtn", False, 1),
    (0, "B", "mx", "rtn", False, 1),
    (1, "X", "mx", "rtn", False, 1),
    (1, "W", "mx", "rtn", False, 1),
    (2, "X", "nv", "rtn", False, 1),
    (2, "W", "nv", "rtn", False, 1),
    (3, "x_pre_up", "mx", "rtn", True, 1),
    (3, "x_dec_down", "mx", "rtn", True, 1),
    (3, "W_down", "mx", "rtn", True, 1),
    (4, "dY1", "mx", "sr", False, 1),
    (4, "dY1", "mx", "sr", False, 0),
    (4, "X1", "mx", "sr", False, 0),
    (4, "W1", "mx", "sr", False, 0),
    (5, "X", "nv", "rtn", False, 1),
    (5, "dY_o", "nv", "sr", False, 0),
    (5, "W_o", "nv", "sr", False, 0),
]


@pytest.mark.parametrize("cfg,name,fmt,rnd,had,axis", FULL)
def test_full_size_tensors(oracle_mod, cfg, name, fmt, rnd, had, axis):
    """The configurations' own tensors at full size, bit-exact."""
    mx = need_gpu()
    bits = workloads.make_tensor(cfg, name)
    _run(mx, oracle_mod, bits, fmt, rnd, had, axis, seed=3 if rnd == "sr" else 0, what=f"cfg{cfg}-{name}")


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_dequantize_matches_oracle(oracle_mod, fmt):
    mx = need_gpu()
    bits = workloads.small_t_bf16((80, 192), 3.0, seed=26, outlier_frac=0.05)
    say("dequantize", fmt)
    q = mx.mxfp4_quantize(to_device_bf16(bits), fmt, "rtn")
    y = mx.mxfp4_dequantize(q).cpu().numpy()
    codes, scales, ts = oracle_mod.quantize(bits, fmt, "rtn")
    want = oracle_mod.dequantize(fmt, codes, scales, ts)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
