"""The benchmark's clock instruments on the GPU (libmxclock.so, not part of
the quantizer / GEMM library): the MFMA ceiling kernel counts one s_memtime
tick per shader clock, i.e. about 32 ticks per 32x32 MFMA (8 passes of 4
cycles for the scaled FP4 32x32x64 and for the fp16 32x32x16 alike), so the
clock figures of the bench line are shader clocks; and the stamps around a
short stretch of work give a plausible clock on every compute unit."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [0, 1])
def test_ceiling_counts_32_ticks_per_mfma(kind):
    import torch
    import bench
    print(f"mfma ceiling kind {kind}", flush=True)
    c = bench.mfma_ceiling(torch.device("cuda", 0), kind=kind, launches=3, iters=4000)
    # one wave per SIMD issues back-to-back independent MFMAs at the nominal
    # 32 cycles each (measured 32.0-32.3); a wide band so that timing noise
    # cannot fail it, narrow enough to catch a counter at a different rate
    assert 30.0 <= c["ticks_per_mfma"] <= 40.0, c
    assert c["tflops"] > 0 and 100.0 <= c["sclk_mhz"] <= 2600.0, c


def test_clock_stamps_pair_every_compute_unit():
    import torch
    import bench
    dev = torch.device("cuda", 0)
    clock = bench.ClockStamps(dev)
    x = torch.randn(4096, 4096, device=dev)
    clock.stamp(0)
    for _ in range(20):
        x = x @ x.T
        x = x / x.norm()
    clock.stamp(1)
    torch.cuda.synchronize()
    s = clock.summary()
    assert s["compute_units_paired"] >= 200, s
    assert 100.0 <= s["sclk_mhz_median"] <= 2600.0, s
