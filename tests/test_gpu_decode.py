"""GPU parity of the decode-shaped MXFP4 GEMM (up to 128 activation rows
against a weight of at least 2048 rows, or with few operand bytes per
workgroup: 16-column workgroups over the whole contraction, the waves'
partial sums added in LDS in wave order).  Every element against the binary64
oracle within 1e-5 * sum|ab|: one to eight 16-row activation tiles, ragged
weight rows, step counts that do not divide evenly among the waves,
contractions of a single step; fp32 and bf16 C into strided and misaligned
outputs (same bits as the contiguous call, nothing outside the view
written); NaN scale bytes; no workspace."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_gemm_within

pytestmark = pytest.mark.gpu


def _pair(mx, oracle_mod, A, B, had=False):
    qa = mx.mxfp4_quantize(to_device_bf16(A), "mx", "rtn", had)
    qb = mx.mxfp4_quantize(to_device_bf16(B), "mx", "rtn", had)
    oa = oracle_mod.quantize(A, "mx", "rtn", had)
    ob = oracle_mod.quantize(B, "mx", "rtn", had)
    ga, gb = q_to_host(qa), q_to_host(qb)
    assert np.array_equal(ga[0], oa[0]) and np.array_equal(ga[1], oa[1])
    assert np.array_equal(gb[0], ob[0]) and np.array_equal(gb[1], ob[1])
    return qa, qb, oa, ob


@pytest.mark.parametrize("M,N,K", [(1, 2048, 128), (16, 2064, 256), (5, 2056, 1152), (17, 2050, 384),
                                   (32, 4096, 640), (24, 3000, 4224), (16, 2048, 13 * 128), (16, 3000, 8192),
                                   (16, 8200, 4224), (20, 8192, 512), (32, 8224, 4096), (30, 8208, 4608),
                                   (33, 2048, 256), (48, 300, 1152), (64, 8200, 4224), (80, 2050, 640),
                                   (100, 4096, 4224), (128, 8192, 512), (128, 300, 2048), (97, 96, 128)])
def test_decode_gemm_full_check(oracle_mod, M, N, K):
    """One to eight activation tiles (partial last tiles), one and two weight
    tiles per workgroup (from 8192 weight rows; 8200 and 8208 leave a
    workgroup with a partial or missing second tile), weights shorter than
    2048 rows, short contractions (one round of loads in flight) and long
    ones (fewer slots where the activation tiles fill LDS), step counts that
    leave the last round partial."""
    mx = need_gpu()
    A = workloads.small_t_bf16((M, K), 3.0, seed=51, outlier_frac=0.02)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=52)
    qa, qb, oa, ob = _pair(mx, oracle_mod, A, B)
    assert mx.mxfp4_gemm_workspace_bytes(qa, qb) == 0
    say("decode gemm", M, N, K)
    C = mx.mxfp4_gemm(qa, qb)
    Cb = mx.mxfp4_gemm_bf16(qa, qb)
    torch.cuda.synchronize()
    Co, So = oracle_mod.gemm("mx", oa, ob)
    assert_gemm_within(C.cpu().numpy(), Co, So, f"decode {M}x{N}x{K}")
    # bf16 C is the fp32 result rounded to nearest even
    assert torch.equal(Cb.view(torch.int16), C.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("bf16", [False, True])
def test_decode_gemm_strided_misaligned_output(oracle_mod, bf16):
    """C at an odd row stride and 4 (bf16: 2) bytes into the buffer: the
    element-wise stores; the result has the contiguous call's bits."""
    mx = need_gpu()
    M, N, K = 20, 2058, 512
    A = workloads.small_t_bf16((M, K), 3.0, seed=53)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=54)
    qa, qb, oa, ob = _pair(mx, oracle_mod, A, B, had=True)
    say("decode gemm strided", bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    gemm = mx.mxfp4_gemm_bf16 if bf16 else mx.mxfp4_gemm
    ref = gemm(qa, qb)
    big = torch.full((M, N + 3), 5.0, dtype=dt, device="cuda")
    gemm(qa, qb, out=big[:, 1:N + 1])
    torch.cuda.synchronize()
    bits = torch.int16 if bf16 else torch.int32
    assert torch.equal(ref.view(bits), big[:, 1:N + 1].contiguous().view(bits))
    host = big.float().cpu().numpy()
    assert (host[:, 0] == 5.0).all() and (host[:, N + 1:] == 5.0).all()
    if not bf16:
        Co, So = oracle_mod.gemm("mx", oa, ob)
        assert_gemm_within(host[:, 1:N + 1], Co, So, "decode strided")


def test_decode_gemm_nan_blocks(oracle_mod):
    """A block holding NaN gets the NaN scale byte: its activation row, and the
    output column of a weight row with one, come out all NaN (and only they)."""
    mx = need_gpu()
    M, N, K = 12, 2080, 1024
    A = workloads.small_normal_bf16((M, K), 1.0, seed=55).copy()
    B = workloads.small_normal_bf16((N, K), 0.02, seed=56).copy()
    A[3, 517] = 0x7FC0
    B[2071, 40] = 0x7FC0
    qa, qb, oa, ob = _pair(mx, oracle_mod, A, B)
    say("decode gemm nan blocks")
    C = mx.mxfp4_gemm(qa, qb).cpu().numpy()
    nan = np.zeros((M, N), dtype=bool)
    nan[3, :] = True
    nan[:, 2071] = True
    assert np.array_equal(np.isnan(C), nan)
    Co, So = oracle_mod.gemm("mx", oa, ob)
    assert np.array_equal(np.isnan(Co), nan)
    assert_gemm_within(C, Co, So, "decode nan")
