"""GPU parity of the GEMM with bf16 output (mxfp4_gemm_bf16).

Against the binary64 oracle: |C_bf16 - C| <= 1e-5 * sum_k |a_ik b_jk|
(the FP32 GEMM's bound) plus the bf16 rounding, at most half a unit in the
last place of 8 significant bits, 2^-8 |C|, per element.  And the property
the entry point states: every element equals the FP32 value mxfp4_gemm
writes for the same operands, rounded to nearest even (checked bit for bit
through torch's own FP32 -> bf16 rounding on the host)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host

pytestmark = pytest.mark.gpu


def _quant_pair(mx, oracle_mod, A_bits, B_bits, fmt):
    qa = mx.mxfp4_quantize(to_device_bf16(A_bits), fmt, "rtn", False, 1, 0)
    qb = mx.mxfp4_quantize(to_device_bf16(B_bits), fmt, "rtn", False, 1, 1)
    oa = oracle_mod.quantize(A_bits, fmt, "rtn", False, 1, 0)
    ob = oracle_mod.quantize(B_bits, fmt, "rtn", False, 1, 1)
    ga, gb = q_to_host(qa), q_to_host(qb)
    assert np.array_equal(ga[0], oa[0]) and np.array_equal(ga[1], oa[1])
    assert np.array_equal(gb[0], ob[0]) and np.array_equal(gb[1], ob[1])
    return qa, qb, oa, ob


def _assert_bf16_within(Cb: np.ndarray, Co: np.ndarray, So: np.ndarray, what: str):
    err = np.abs(Cb.astype(np.float64) - Co)
    bound = 1e-5 * So * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Co)
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} elements out of bound; first {list(i)}: "
                             f"gpu {Cb[i]!r} oracle {Co[i]!r} S {So[i]!r}")


def _assert_same_bf16(got: torch.Tensor, want: torch.Tensor, what: str):
    """Bit for bit, except that a NaN only has to meet a NaN (the payload of
    a rounded NaN is not specified)."""
    g, w = got.cpu(), want.cpu()
    gn, wn = torch.isnan(g.float()), torch.isnan(w.float())
    assert torch.equal(gn, wn), f"{what}: NaN positions differ"
    gb, wb = g.view(torch.int16), w.view(torch.int16)
    diff = (gb != wb) & ~gn
    assert not diff.any(), f"{what}: {int(diff.sum())} elements differ, first {diff.nonzero()[0].tolist()}"


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("M,N,K", [(256, 256, 1024), (300, 200, 384), (17, 529, 256), (64, 96, 8192),
                                   (1, 1, 128), (16, 1000, 4096)])
def test_gemm_bf16_small(oracle_mod, fmt, M, N, K):
    """Ragged tiles, short and split-K contractions (64 x 96 x 8192 and the
    decode-shaped 16 x 1000 x 4096 write their bf16 output from the split
    reduction), a 1 x 1 output; every element checked both ways."""
    mx = need_gpu()
    A = workloads.small_t_bf16((M, K), 3.0, seed=61, outlier_frac=0.02)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=62)
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, fmt)
    say("gemm bf16", fmt, M, N, K, "ws", mx.mxfp4_gemm_workspace_bytes(qa, qb))
    Cb = mx.mxfp4_gemm_bf16(qa, qb)
    C32 = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    assert Cb.dtype == torch.bfloat16 and Cb.shape == (M, N)
    _assert_same_bf16(Cb, C32.cpu().to(torch.bfloat16), f"{fmt} {M}x{N}x{K} vs rounded FP32")
    Co, So = oracle_mod.gemm(fmt, oa, ob)
    _assert_bf16_within(Cb.float().cpu().numpy(), Co, So, f"{fmt} {M}x{N}x{K}")


def test_gemm_bf16_strided_output(oracle_mod):
    """ldc > N, the columns around the written block untouched."""
    mx = need_gpu()
    A = workloads.small_normal_bf16((130, 256), 1.0, seed=63)
    B = workloads.small_normal_bf16((97, 256), 1.0, seed=64)
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, "mx")
    big = torch.full((130, 201), 7.0, dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_gemm_bf16(qa, qb, out=big[:, 51:148])
    host = big.float().cpu().numpy()
    assert (host[:, :51] == 7.0).all() and (host[:, 148:] == 7.0).all()
    Co, So = oracle_mod.gemm("mx", oa, ob)
    _assert_bf16_within(host[:, 51:148], Co, So, "strided")


def test_gemm_bf16_specials():
    """Overflow past the bf16 range rounds to infinity and a NaN scale gives
    NaN, as the FP32 result rounds (compared bit for bit)."""
    mx = need_gpu()
    M, N, K = 64, 64, 256
    A = workloads.small_normal_bf16((M, K), 1.0, seed=65)
    B = workloads.small_normal_bf16((N, K), 1.0, seed=66)
    qa = mx.mxfp4_quantize(to_device_bf16(A), "mx", "rtn", False, 1, 0)
    qb = mx.mxfp4_quantize(to_device_bf16(B), "mx", "rtn", False, 1, 1)
    # large scales on row 0 of A (products near 2^254 overflow FP32 and
    # bf16) and the NaN scale byte on row 1
    qa.scales[0] = 254
    qa.scales[1] = 0xFF
    Cb = mx.mxfp4_gemm_bf16(qa, qb)
    C32 = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _assert_same_bf16(Cb, C32.cpu().to(torch.bfloat16), "specials")
    assert torch.isinf(Cb[0].float()).any() and torch.isnan(Cb[1].float()).all()


def test_gemm_bf16_headline_sampled(oracle_mod):
    """4096 x 14336 x 8192 MXFP4: bit-identical to the rounded FP32 output in
    full, and sampled rows checked against the oracle."""
    mx = need_gpu()
    A = workloads.make_tensor(0, "A")
    B = workloads.make_tensor(0, "B")
    say("bf16 headline quantize")
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, "mx")
    Cb = mx.mxfp4_gemm_bf16(qa, qb)
    C32 = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _assert_same_bf16(Cb, C32.cpu().to(torch.bfloat16), "headline vs rounded FP32")
    rows = np.arange(0, 4096, 331)
    Cr = Cb[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    Co, So = oracle_mod.gemm("mx", oa, ob, rows=rows)
    _assert_bf16_within(Cr, Co, So, "headline rows")
