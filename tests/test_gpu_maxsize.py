"""Maximum sizes: a row-quantized tensor of more than 2^32 chunks of 8
elements (68.7 GB of bf16: the launch is cut into slices below 2^31 chunks,
and the stochastic-rounding counter crosses 2^32), and a transposed
quantization with more than 65535 tiles of 256 rows (the grid is cut into
slabs), both checked against the oracle (on rows sampled at every boundary,
or in full); and GEMMs over the longest contraction the library takes
(2^24), checked on sampled outputs.  The fused quantize + noise sums at the
same slicing and slab boundaries, against the unfused calls."""
import numpy as np
import pytest
import torch

from gpu_common import need_gpu, say, q_to_host, assert_codes_equal

pytestmark = pytest.mark.gpu


def _fill_normal(x, seed, rows_per_slab=1 << 16, std=1.0):
    g = torch.Generator(device=x.device)
    g.manual_seed(seed)
    for r0 in range(0, x.shape[0], rows_per_slab):
        r1 = min(r0 + rows_per_slab, x.shape[0])
        x[r0:r1] = (torch.randn((r1 - r0, x.shape[1]), generator=g, device=x.device) * std).to(torch.bfloat16)


def _bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def test_rows_beyond_2_to_the_32_chunks(oracle_mod):
    mx = need_gpu()
    R, C = (1 << 22) + 1, 8192            # R * C / 8 = 2^32 + 1024 chunks
    free, _ = torch.cuda.mem_get_info()
    if free < 100 * (1 << 30):
        pytest.skip("needs about 90 GB of device memory")
    say("max size rows", R, C)
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    _fill_normal(x, 93)
    q = mx.mxfp4_quantize(x, "mx", "sr", False, 1, 77)
    torch.cuda.synchronize()
    # rows at the slice boundaries (2^30 chunks = 2^20 rows) and where the
    # chunk counter passes 2^31 and 2^32
    for r in (0, 1, (1 << 20) - 1, 1 << 20, (1 << 21) - 1, 1 << 21, (1 << 22) - 1, 1 << 22):
        xr = _bits(x[r:r + 1])
        want = oracle_mod.quantize_rows_at(xr, r, "sr", False, 77)
        got = (q.codes[r:r + 1].cpu().numpy(), q.scales[r:r + 1].cpu().numpy(), None)
        assert_codes_equal(got, (want[0], want[1], None), f"max-size row {r}")
    del x, q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,rnd", [("mx", "rtn"), ("nv", "sr")])
def test_transposed_beyond_65535_row_tiles(oracle_mod, fmt, rnd):
    mx = need_gpu()
    R, C = 65538 * 256, 64                 # 65538 tiles of 256 rows along the contraction
    say("max size transposed", fmt, rnd, R, C)
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    _fill_normal(x, 94, std=0.5)
    q = mx.mxfp4_quantize(x, fmt, rnd, False, 0, 5)
    got = q_to_host(q)
    X = _bits(x)
    del x, q
    torch.cuda.empty_cache()
    assert_codes_equal(got, oracle_mod.quantize(X, fmt, rnd, False, 0, 5), f"max-size transposed {fmt}")


@pytest.mark.parametrize("fmt,M,N", [("mx", 33, 300), ("mx", 300, 256), ("nv", 40, 260)])
def test_gemm_longest_contraction(oracle_mod, fmt, M, N):
    """K = 2^24, the longest contraction the GEMM takes (narrow and wide MXFP4
    tiles, NVFP4), split along K; sampled outputs against the oracle."""
    mx = need_gpu()
    K = 1 << 24
    say("max size gemm", fmt, M, N, K)
    a = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    _fill_normal(a, 95, rows_per_slab=16)
    _fill_normal(b, 96, rows_per_slab=16, std=0.02)
    qa = mx.mxfp4_quantize(a, fmt, "rtn", False, 1, 0)
    qb = mx.mxfp4_quantize(b, fmt, "rtn", False, 1, 0)
    del a, b
    assert mx.mxfp4_gemm_workspace_bytes(qa, qb) > 0
    C = mx.mxfp4_gemm(qa, qb).cpu().numpy()
    rows = np.array([0, M // 2, M - 1])
    cols = np.array([0, N // 3, N - 1])
    ta = float(qa.tensor_scale.cpu()[0]) if fmt == "nv" else None
    tb = float(qb.tensor_scale.cpu()[0]) if fmt == "nv" else None
    oa = (qa.codes[torch.from_numpy(rows).cuda()].cpu().numpy(), qa.scales[torch.from_numpy(rows).cuda()].cpu().numpy(), ta)
    ob = (qb.codes[torch.from_numpy(cols).cuda()].cpu().numpy(), qb.scales[torch.from_numpy(cols).cuda()].cpu().numpy(), tb)
    del qa, qb
    torch.cuda.empty_cache()
    Co, So = oracle_mod.gemm(fmt, oa, ob)
    err = np.abs(C[np.ix_(rows, cols)].astype(np.float64) - Co)
    assert np.all(err <= 1e-5 * So), (err, So)


def _same_stats(a, b, what):
    a, b = a.cpu().numpy(), b.cpu().numpy()
    for j in (0, 1):
        assert abs(a[j] - b[j]) <= 1e-12 * max(abs(b[j]), 1e-300), (what, j, a[j], b[j])
    assert a[2] == b[2], (what, a[2], b[2])


@pytest.mark.parametrize("strided", [False, True])
def test_quantize_noise_sliced_launches(strided):
    """mxfp4_quantize_noise past 2^30 chunks of 8 elements, where the row
    quantizer is launched in slices (packed rows: contiguous chunk ranges;
    padded rows: ranges of whole rows) and each slice writes its own run of
    partial sums: the tensor equals mxfp4_quantize's bit for bit and the sums
    equal those of the separate noise pass (both are checked against the
    oracle at smaller sizes)."""
    mx = need_gpu()
    R, C = (1 << 20) + 1, 8192             # 2^30 + 1024 chunks
    free, _ = torch.cuda.mem_get_info()
    if free < 60 * (1 << 30):
        pytest.skip("needs about 50 GB of device memory")
    say("max size quantize+noise", "strided" if strided else "packed", R, C)
    base = torch.empty((R, C + (64 if strided else 0)), dtype=torch.bfloat16, device="cuda")
    x = base[:, :C]
    _fill_normal(base, 95, rows_per_slab=1 << 15, std=0.01)
    q, st = mx.mxfp4_quantize_noise(x, "mx", "sr", False, 1, 41)
    q2 = mx.mxfp4_quantize(x, "mx", "sr", False, 1, 41)
    assert torch.equal(q.codes, q2.codes) and torch.equal(q.scales, q2.scales)
    st2 = mx.mxfp4_quantization_noise(x, q2, 1)
    _same_stats(st, st2, "sliced quantize+noise")
    del base, x, q, q2
    torch.cuda.empty_cache()


def test_quantize_noise_transposed_slabs():
    """The tiled transposing quantizer with sums past 65535 row tiles (two
    grid slabs, each with its own run of partial sums)."""
    mx = need_gpu()
    R, C = 65538 * 256, 64
    say("max size transposed quantize+noise", R, C)
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    _fill_normal(x, 96, std=0.5)
    q, st = mx.mxfp4_quantize_noise(x, "nv", "sr", False, 0, 9)
    q2 = mx.mxfp4_quantize(x, "nv", "sr", False, 0, 9)
    assert torch.equal(q.codes, q2.codes) and torch.equal(q.scales, q2.scales)
    assert torch.equal(q.tensor_scale, q2.tensor_scale)
    st2 = mx.mxfp4_quantization_noise(x, q2, 0)
    _same_stats(st, st2, "transposed slabs quantize+noise")
