"""GPU parity of mxfp4_qema_quantize (the Q-EMA step: the EMA update fused
with MXFP4 round-to-nearest) with the oracle: the new average bit for bit and
the codes and scale bytes bit for bit, over several steps in a row, with and
without the rotation, on padded rows, NaN blocks and the configuration-4 ViT
weights.  (The method itself is parity unpinned: the page names Q-EMA without
its rule; the test pins this reading of it.)"""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import need_gpu, say, to_device_bf16, q_to_host, assert_codes_equal

pytestmark = pytest.mark.gpu


def _steps(oracle_mod, mx, W_list, m0, beta, had, pad=0, what=""):
    R, C = W_list[0].shape
    m_host = m0.copy()
    if pad:
        full = torch.zeros((R, C + pad), dtype=torch.float32, device="cuda")
        full[:, :C] = torch.from_numpy(m0).cuda()
        m_dev = full[:, :C]
    else:
        m_dev = torch.from_numpy(m0).cuda()
    for step, W in enumerate(W_list):
        say("qema", what, step, beta, had, pad, W.shape)
        q = mx.mxfp4_qema_quantize(to_device_bf16(W, pad_cols=pad), m_dev, beta, had)
        m_host, oq = oracle_mod.qema_quantize(W, m_host, beta, had)
        got = m_dev.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), m_host.view(np.uint32)), (what, step)
        assert_codes_equal(q_to_host(q), oq, f"qema {what} step {step}")


@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("beta", [0.9, 0.999, 0.0, 1.0])
def test_qema_steps_match_oracle(oracle_mod, had, beta):
    mx = need_gpu()
    Ws = [workloads.small_normal_bf16((320, 768), 0.02, seed=110 + s) for s in range(3)]
    m0 = (np.random.default_rng(111).standard_normal((320, 768)) * 0.02).astype(np.float32)
    _steps(oracle_mod, mx, Ws, m0, beta, had, what="small")


def test_qema_padded_rows_and_nan_blocks(oracle_mod):
    mx = need_gpu()
    W = workloads.small_t_bf16((64, 256), 3.0, seed=112).copy()
    W[3, 40] = 0x7FC0
    m0 = (np.random.default_rng(113).standard_normal((64, 256))).astype(np.float32)
    m0[10, 200] = np.inf
    _steps(oracle_mod, mx, [W, W], m0, 0.9, False, pad=8, what="padded+nan")


@pytest.mark.parametrize("name", ["W1", "W2"])
def test_qema_config4_weights(oracle_mod, name):
    mx = need_gpu()
    W = workloads.make_tensor(4, name)
    m0 = workloads.bf16_bits_to_f32(W).copy()
    _steps(oracle_mod, mx, [W, W], m0 * 0.5, 0.99, False, what=f"config 4 {name}")


def test_qema_rejects_bad_arguments():
    mx = need_gpu()
    w = torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda")
    m = torch.zeros((64, 100), dtype=torch.float32, device="cuda")
    with pytest.raises(mx.MxFp4Error) as e:
        mx.mxfp4_qema_quantize(w[:, :96].contiguous(), m[:, :96].contiguous(), 1.5)
    assert e.value.status == -1
