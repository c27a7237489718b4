"""GPU parity of the block-scaled FP4 GEMM against the binary64 oracle:
|C_gpu - C| <= 1e-5 * sum_k |a_ik b_jk| per element."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_gemm_within

pytestmark = pytest.mark.gpu


def _quant_pair(mx, oracle_mod, A_bits, B_bits, fmt, had=False, rnd="rtn", axis_a=1, axis_b=1, seeds=(0, 1)):
    qa = mx.mxfp4_quantize(to_device_bf16(A_bits), fmt, rnd, had, axis_a, seeds[0])
    qb = mx.mxfp4_quantize(to_device_bf16(B_bits), fmt, rnd, had, axis_b, seeds[1])
    oa = oracle_mod.quantize(A_bits, fmt, rnd, had, axis_a, seeds[0])
    ob = oracle_mod.quantize(B_bits, fmt, rnd, had, axis_b, seeds[1])
    # the GEMM test relies on identical operands on both sides
    ga, gb = q_to_host(qa), q_to_host(qb)
    assert np.array_equal(ga[0], oa[0]) and np.array_equal(ga[1], oa[1])
    assert np.array_equal(gb[0], ob[0]) and np.array_equal(gb[1], ob[1])
    return qa, qb, oa, ob


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("M,N,K", [(256, 256, 1024), (300, 200, 384), (17, 529, 256), (512, 768, 2048),
                                   (64, 96, 8192), (1, 1, 128), (128, 160, 640), (64, 64, 4224),
                                   (64, 96, 32768), (100, 64, 12672)])
def test_gemm_small_full_check(oracle_mod, fmt, M, N, K):
    """Several tiles with ragged edges, short contractions, contractions that
    end half way into a 256-wide stage (384, 640, 128, 4224, 12672), a 1 x 1
    output; MXFP4 rows up to 128 take the decode kernel (64 x 96 x 8192 and
    the other small ones), and the narrow kernel split along K where a decode
    workgroup's operands would pass its limit (64 x 96 x 32768; 100 x 64 x
    12672 with an odd stage count in the last split); NVFP4 splits the wide
    kernel (64 x 96 x 8192 and the long ones); every element checked."""
    mx = need_gpu()
    A = workloads.small_t_bf16((M, K), 3.0, seed=31, outlier_frac=0.02)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=32)
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, fmt)
    say("gemm", fmt, M, N, K, "ws", mx.mxfp4_gemm_workspace_bytes(qa, qb))
    C = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    Co, So = oracle_mod.gemm(fmt, oa, ob)
    assert_gemm_within(C.cpu().numpy(), Co, So, f"{fmt} {M}x{N}x{K}")


def test_gemm_config1_full(oracle_mod):
    """MXFP4 RTN 256 x 256 x 1024: N(0,1) activations, N(0,0.02) weights."""
    mx = need_gpu()
    X = workloads.make_tensor(1, "X")
    W = workloads.make_tensor(1, "W")
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, X, W, "mx")
    say("gemm config 1")
    C = mx.mxfp4_gemm(qa, qb).cpu().numpy()
    Co, So = oracle_mod.gemm("mx", oa, ob)
    assert_gemm_within(C, Co, So, "config1")


def test_gemm_one_hot_exact(oracle_mod):
    """Codes of +-1 with unit scales: the result is an exact integer count."""
    mx = need_gpu()
    rng = np.random.default_rng(33)
    M, N, K = 256, 256, 512
    va = rng.choice([-1.0, 0.0, 1.0], size=(M, K))
    vb = rng.choice([-1.0, 1.0], size=(N, K))
    va[:, 0] = 4.0
    vb[:, 0] = 4.0      # absmax 4 -> e = 0 so +-1 maps to the codes of +-1
    A = workloads.f32_to_bf16_bits(va.astype(np.float32))
    B = workloads.f32_to_bf16_bits(vb.astype(np.float32))
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, "mx")
    C = mx.mxfp4_gemm(qa, qb).cpu().numpy()
    assert np.array_equal(C.astype(np.float64), va @ vb.T)


def test_gemm_writes_into_strided_output(oracle_mod):
    mx = need_gpu()
    A = workloads.small_normal_bf16((128, 256), 1.0, seed=34)
    B = workloads.small_normal_bf16((96, 256), 1.0, seed=35)
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, "mx")
    big = torch.full((128, 200), 7.0, device="cuda")
    mx.mxfp4_gemm(qa, qb, out=big[:, 50:146])
    host = big.cpu().numpy()
    Co, So = oracle_mod.gemm("mx", oa, ob)
    assert_gemm_within(host[:, 50:146], Co, So, "strided")
    assert (host[:, :50] == 7.0).all() and (host[:, 146:] == 7.0).all()


def stratified(n, block, nrand, rng):
    """Indices 0 and n - 1, one random index inside every block of `block`
    consecutive indices (so every output tile row / column is compared), and
    nrand more at random."""
    per_block = [int(rng.integers(b, min(b + block, n))) for b in range(0, n, block)]
    extra = rng.choice(n, size=min(nrand, n), replace=False)
    return np.unique(np.concatenate([[0, n - 1], per_block, extra]).astype(np.int64))


def _sampled_check(mx, oracle_mod, qa, qb, oa, ob, fmt, what, nsample=48, seed=0):
    """Full rows and full columns of C against the oracle: one row in every
    256-row tile row and one column in every 128-column half tile, plus
    rows / columns 0 and the last, plus nsample random ones each."""
    C = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    M, N = qa.rows, qb.rows
    rows = stratified(M, 256, nsample, rng)
    cols = stratified(N, 128, nsample, rng)
    Cr = C[torch.from_numpy(rows).cuda()].cpu().numpy()
    Cc = C[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    del C
    # full rows and full columns of C
    Co_r, So_r = oracle_mod.gemm(fmt, oa, ob, rows=rows)
    e1 = assert_gemm_within(Cr, Co_r, So_r, what + " rows")
    del Co_r, So_r
    Co_c, So_c = oracle_mod.gemm(fmt, oa, ob, cols=cols)
    e2 = assert_gemm_within(Cc, Co_c, So_c, what + " cols")
    say(what, f"{len(rows)} rows, {len(cols)} cols; max |err|/S", max(e1, e2))


def test_gemm_headline_sampled(oracle_mod):
    """4096 x 14336 x 8192 MXFP4 (the benchmark's launch), checked on full
    sampled rows and columns of C."""
    mx = need_gpu()
    A = workloads.make_tensor(0, "A")
    B = workloads.make_tensor(0, "B")
    say("headline quantize")
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, "mx")
    _sampled_check(mx, oracle_mod, qa, qb, oa, ob, "mx", "headline", nsample=24)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_gemm_balanced_half_tiles(oracle_mod, fmt):
    """More 256 x 256 tiles than compute units, not a multiple of them: the
    remainder tiles run as 256 x 128 halves at the start and at the end of
    the launch (MXFP4; the NVFP4 kernel runs the same shape as whole tiles).  M = 4352 (17 tile rows), N = 3904 (the last tile column has
    64 valid columns, so its second half lies wholly past N); the 16
    remainder tiles are the bottom tile row, checked in full."""
    mx = need_gpu()
    M, N, K = 4352, 3904, 512
    A = workloads.small_t_bf16((M, K), 3.0, seed=36, outlier_frac=0.01)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=37)
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, fmt)
    say("gemm balanced", fmt, M, N, K)
    C = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(4096, M), np.arange(0, 4096, 97)])
    Cr = C[torch.from_numpy(rows).cuda()].cpu().numpy()
    Co, So = oracle_mod.gemm(fmt, oa, ob, rows=rows)
    assert_gemm_within(Cr, Co, So, "balanced rows")
    cols = np.array([0, 1, 127, 128, 255, 256, 3839, 3840, 3871, 3872, N - 1])
    Cc = C[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    Co, So = oracle_mod.gemm(fmt, oa, ob, cols=cols)
    assert_gemm_within(Cc, Co, So, "balanced cols")


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_gemm_balanced_halves_partial_column(oracle_mod, fmt):
    """Tile count = 1.5 x 256: 128 remainder tiles run as 256 x 128 halves at
    the start and at the end of the launch.  M = 3072, N = 8128 (the last tile
    column has 192 valid columns, so its second half is partly past N),
    K = 256; rows of the remainder tiles checked across all columns."""
    mx = need_gpu()
    M, N, K = 3072, 8128, 256
    A = workloads.small_t_bf16((M, K), 3.0, seed=38, outlier_frac=0.01)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=39)
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, fmt)
    say("gemm halves, partial column", fmt, M, N, K)
    C = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(1024, 3072, 7), np.arange(0, 1024, 61), [M - 1]])
    Cr = C[torch.from_numpy(rows).cuda()].cpu().numpy()
    Co, So = oracle_mod.gemm(fmt, oa, ob, rows=rows)
    assert_gemm_within(Cr, Co, So, "halves rows")
    cols = np.array([0, 63, 64, 127, 128, 191, 192, 255, 4096, 4160, 4288, 4351, 7936, 8000, 8127])
    Cc = C[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    Co, So = oracle_mod.gemm(fmt, oa, ob, cols=cols)
    assert_gemm_within(Cc, Co, So, "halves cols")


def test_gemm_config2_sampled(oracle_mod):
    """NVFP4 8192 x 4096 x 4096, Student-t(3) activations with 1% x50 outlier channels."""
    mx = need_gpu()
    X = workloads.make_tensor(2, "X")
    W = workloads.make_tensor(2, "W")
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, X, W, "nv")
    _sampled_check(mx, oracle_mod, qa, qb, oa, ob, "nv", "config2", nsample=32)


def test_gemm_config3_decode_and_prefill_sampled(oracle_mod):
    """MXFP4 with block Hadamard on both operands: decode M = 16 and prefill."""
    mx = need_gpu()
    W = workloads.make_tensor(3, "W_up")
    qw = mx.mxfp4_quantize(to_device_bf16(W), "mx", "rtn", True)
    ow = oracle_mod.quantize(W, "mx", "rtn", True)
    for name in ("x_dec_up", "x_pre_up"):
        X = workloads.make_tensor(3, name)
        qx = mx.mxfp4_quantize(to_device_bf16(X), "mx", "rtn", True)
        ox = oracle_mod.quantize(X, "mx", "rtn", True)
        _sampled_check(mx, oracle_mod, qx, qw, ox, ow, "mx", "config3 " + name, nsample=24)


def test_gemm_config4_wgrad_split_k(oracle_mod):
    """ViT fc2 wgrad dW = dY^T X: 768 x 3072 x 50432 with both operands
    quantized along the token axis (axis 0) with stochastic rounding."""
    mx = need_gpu()
    dY = workloads.make_tensor(4, "dY2")       # [50432, 768]
    X = workloads.make_tensor(4, "X2")         # [50432, 3072]
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, dY, X, "mx", rnd="sr", axis_a=0, axis_b=0, seeds=(2, 3))
    assert mx.mxfp4_gemm_workspace_bytes(qa, qb) > 0          # split along K
    _sampled_check(mx, oracle_mod, qa, qb, oa, ob, "mx", "config4 wgrad fc2", nsample=16)


@pytest.mark.parametrize("fmt,M,N,K", [("mx", 300, 300, 16384), ("mx", 40, 260, 32768), ("mx", 300, 300, 4096),
                                       ("nv", 200, 260, 8192)])
def test_splitk_reduction_load_widths_agree(oracle_mod, fmt, M, N, K):
    """The split-K reduction adds the partials in split order whether it reads
    them four outputs at a time (contiguous, 16-byte aligned C, more than four
    splits: 16 or 32 here, wide and narrow tiles, NVFP4) or one at a time (C at
    an odd row stride and a 4-byte offset; 4 splits): the same bits, fp32 and bf16 C,
    and the oracle within tolerance on sampled rows."""
    mx = need_gpu()
    A = workloads.small_normal_bf16((M, K), 1.0, seed=41)
    B = workloads.small_normal_bf16((N, K), 0.02, seed=42)
    qa, qb, oa, ob = _quant_pair(mx, oracle_mod, A, B, fmt)
    assert mx.mxfp4_gemm_workspace_bytes(qa, qb) > 0
    say("split-K reduction widths", fmt, M, N, K)
    c_vec = mx.mxfp4_gemm(qa, qb)
    big = torch.full((M, N + 3), 5.0, device="cuda")
    mx.mxfp4_gemm(qa, qb, out=big[:, 1:N + 1])
    h_vec, h_big = c_vec.cpu().numpy(), big.cpu().numpy()
    assert np.array_equal(h_vec.view(np.uint32), h_big[:, 1:N + 1].view(np.uint32))
    assert (h_big[:, 0] == 5.0).all() and (h_big[:, N + 1:] == 5.0).all()
    b_vec = mx.mxfp4_gemm_bf16(qa, qb)
    bbig = torch.full((M, N + 3), 5.0, dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_gemm_bf16(qa, qb, out=bbig[:, 1:N + 1])
    assert torch.equal(b_vec.view(torch.int16), bbig[:, 1:N + 1].contiguous().view(torch.int16))
    rows = np.array([0, M // 2, M - 1])
    Co, So = oracle_mod.gemm(fmt, oa, ob, rows=rows)
    assert_gemm_within(h_vec[rows], Co, So, f"split-K {fmt} {M}x{N}x{K}")


def test_gemm_format_mismatch_rejected(oracle_mod):
    mx = need_gpu()
    A = workloads.small_normal_bf16((64, 256), 1.0, seed=36)
    qa = mx.mxfp4_quantize(to_device_bf16(A), "mx", "rtn", False)
    qh = mx.mxfp4_quantize(to_device_bf16(A), "mx", "rtn", True)
    with pytest.raises(mx.MxFp4Error) as e:
        mx.mxfp4_gemm(qa, qh)
    assert e.value.status == -3


@pytest.mark.parametrize("fmt,M,N,K", [("mx", 768, 3072, 50432), ("nv", 512, 768, 8192), ("mx", 16, 14336, 4096)])
def test_gemm_is_deterministic(fmt, M, N, K):
    """Split-K partials are added in a fixed order and every tile's MFMA
    sequence is fixed: two calls on the same operands give the same bits."""
    mx = need_gpu()
    g = torch.Generator(device="cuda")
    g.manual_seed(81)
    a = (torch.randn((M, K), generator=g, device="cuda")).to(torch.bfloat16)
    b = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    qa = mx.mxfp4_quantize(a, fmt, "rtn", False, 1, 0)
    qb = mx.mxfp4_quantize(b, fmt, "rtn", False, 1, 0)
    say("gemm determinism", fmt, M, N, K, "ws", mx.mxfp4_gemm_workspace_bytes(qa, qb))
    c1 = mx.mxfp4_gemm(qa, qb)
    c2 = mx.mxfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


# ---------------------------------------------------------------------------
# Every configuration's GEMM shapes (forward XW^T, dgrad dY.W, wgrad dY^T.X),
# with the operands quantized as the training step quantizes them: forward
# operands round-to-nearest along K, backward operands stochastically rounded
# along their own contraction axis (seeds 0..3 in order of use).
# ---------------------------------------------------------------------------
_TENSORS = {}


def _tensor(cfg, name):
    key = (cfg, name)
    if key not in _TENSORS:
        if len(_TENSORS) > 6:
            _TENSORS.clear()
        _TENSORS[key] = workloads.make_tensor(cfg, name)
    return _TENSORS[key]


def _training_pair(mx, oracle_mod, cfg, fmt, a, b, what, nsample=16):
    """a, b = (tensor name, rounding, axis, seed): quantize both on the GPU and
    in the oracle (bit-exact), then the sampled GEMM check."""
    A, B = _tensor(cfg, a[0]), _tensor(cfg, b[0])
    say(what, "quantize", a, b, A.shape, B.shape)
    qa = mx.mxfp4_quantize(to_device_bf16(A), fmt, a[1], False, a[2], a[3])
    qb = mx.mxfp4_quantize(to_device_bf16(B), fmt, b[1], False, b[2], b[3])
    oa = oracle_mod.quantize(A, fmt, a[1], False, a[2], a[3])
    ob = oracle_mod.quantize(B, fmt, b[1], False, b[2], b[3])
    for g, o, t in ((q_to_host(qa), oa, "A"), (q_to_host(qb), ob, "B")):
        assert np.array_equal(g[0], o[0]) and np.array_equal(g[1], o[1]) and g[2] == o[2], (what, t)
    say(what, "gemm", qa.rows, qb.rows, qa.k, "ws", mx.mxfp4_gemm_workspace_bytes(qa, qb))
    _sampled_check(mx, oracle_mod, qa, qb, oa, ob, fmt, what, nsample=nsample)


def test_gemm_config5_qkv_forward(oracle_mod):
    """NVFP4 16384 x 12288 x 4096: X [16384, 4096] t(3) times W_qkv^T."""
    mx = need_gpu()
    _training_pair(mx, oracle_mod, 5, "nv", ("X", "rtn", 1, 0), ("W_qkv", "rtn", 1, 0), "config5 qkv fwd")


def test_gemm_config5_qkv_dgrad(oracle_mod):
    """NVFP4 16384 x 4096 x 12288: dY_qkv [16384, 12288] along its rows times
    W_qkv quantized along its rows' other axis (axis 0, [4096, 12288])."""
    mx = need_gpu()
    _training_pair(mx, oracle_mod, 5, "nv", ("dY_qkv", "sr", 1, 0), ("W_qkv", "sr", 0, 1), "config5 qkv dgrad")


def test_gemm_config5_qkv_wgrad(oracle_mod):
    """NVFP4 12288 x 4096 x 16384 (a contraction over all 16384 tokens, one
    fp32 accumulator per output: 688 tiles, no split): dY_qkv^T X."""
    mx = need_gpu()
    _training_pair(mx, oracle_mod, 5, "nv", ("dY_qkv", "sr", 0, 2), ("X", "sr", 0, 3), "config5 qkv wgrad")


def test_gemm_config5_down_wgrad(oracle_mod):
    """NVFP4 4096 x 11008 x 16384: dY_down^T X_down (1024 fp16-MFMA steps per
    accumulator, no split)."""
    mx = need_gpu()
    _training_pair(mx, oracle_mod, 5, "nv", ("dY_down", "sr", 0, 2), ("X_down", "sr", 0, 3), "config5 down wgrad")


def test_gemm_config4_fc1_forward_and_dgrad(oracle_mod):
    """MXFP4 50432 x 3072 x 768 (forward, RTN) and 50432 x 768 x 3072 (dgrad,
    stochastic rounding: dY1 along its rows, W1 along axis 0)."""
    mx = need_gpu()
    _training_pair(mx, oracle_mod, 4, "mx", ("X1", "rtn", 1, 0), ("W1", "rtn", 1, 0), "config4 fc1 fwd")
    _training_pair(mx, oracle_mod, 4, "mx", ("dY1", "sr", 1, 0), ("W1", "sr", 0, 1), "config4 fc1 dgrad")


def test_gemm_config3_down_projection(oracle_mod):
    """MXFP4 with block Hadamard: prefill 4096 x 4096 x 14336 (exactly 256
    output tiles, so the 14336 contraction runs unsplit in one accumulator)
    and decode 16 x 4096 x 14336."""
    mx = need_gpu()
    W = _tensor(3, "W_down")
    say("config3 down quantize weights")
    qw = mx.mxfp4_quantize(to_device_bf16(W), "mx", "rtn", True)
    ow = oracle_mod.quantize(W, "mx", "rtn", True)
    gw = q_to_host(qw)
    assert np.array_equal(gw[0], ow[0]) and np.array_equal(gw[1], ow[1])
    for name in ("x_pre_down", "x_dec_down"):
        X = _tensor(3, name)
        qx = mx.mxfp4_quantize(to_device_bf16(X), "mx", "rtn", True)
        ox = oracle_mod.quantize(X, "mx", "rtn", True)
        gx = q_to_host(qx)
        assert np.array_equal(gx[0], ox[0]) and np.array_equal(gx[1], ox[1])
        say("config3 down", name, "ws", mx.mxfp4_gemm_workspace_bytes(qx, qw))
        _sampled_check(mx, oracle_mod, qx, qw, ox, ow, "mx", "config3 down " + name, nsample=16)
