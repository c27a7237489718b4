"""Host logic of bench.py (no GPU): the one-GPU refusal, the traffic figure
gated on the GEMM source it was measured on, and the rocprofv3 summaries."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def _traffic_file(tmp_path, digest, nbytes=123456.0):
    p = tmp_path / "traffic.txt"
    p.write_text("header line\n" + json.dumps({"bytes_per_launch": nbytes, "gemm_isa_sha256_16": digest}))
    return str(p)


def test_traffic_only_for_the_measured_gemm_source(tmp_path):
    assert bench.gemm_traffic(_traffic_file(tmp_path, bench.kernel_digest(compile_if_stale=True))) == 123456.0
    assert bench.gemm_traffic(_traffic_file(tmp_path, "0" * 16)) is None
    assert bench.gemm_traffic(str(tmp_path / "missing.txt")) is None
    bad = tmp_path / "bad.txt"
    bad.write_text("header\nnot json")
    assert bench.gemm_traffic(str(bad)) is None


def test_committed_traffic_matches_the_gemm_source():
    """The committed PMC summary was taken on the current headline GEMM kernel
    (same gfx950 assembly), so the benchmark reports its traffic figure."""
    bench.kernel_digest(compile_if_stale=True)
    path = os.path.join(ROOT, "profiles", "gemm_mx_headline_traffic.txt")
    assert bench.gemm_traffic(path) is not None


def test_summarize_stats_table(tmp_path):
    csv_path = tmp_path / "stats.csv"
    csv_path.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs"\n'
                        '"gemm_kernel",12,3000000,250000,80.5,240000,260000\n'
                        '"quant_kernel",26,700000,26923,19.5,13000,48000\n')
    out = tmp_path / "out.md"
    bench.summarize_stats(str(csv_path), str(out))
    lines = out.read_text().splitlines()
    assert lines[0].startswith("| kernel | calls | average us")
    assert lines[2] == "| gemm_kernel | 12 | 250.0 | 240.0 | 260.0 | 80.5 |"
    assert lines[3] == "| quant_kernel | 26 | 26.9 | 13.0 | 48.0 | 19.5 |"


def test_summarize_sq_derived_figures(tmp_path):
    """Two counter runs of one kernel (other kernels ignored): averages per
    dispatch, the clock from GRBM_GUI_ACTIVE summed over 8 XCDs, the MFMA
    pipe's share of 1024 SIMDs' cycles and cycles per MFMA instruction."""
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    run_a = tmp_path / "a" / "host"
    run_b = tmp_path / "b" / "host"
    run_a.mkdir(parents=True)
    run_b.mkdir(parents=True)
    # 100 us dispatches; 2e5 cycles per XCD -> 2.0 GHz
    (run_a / "s_counter_collection.csv").write_text(
        head
        + "1,mxfp4::gemm_mx_kernel<0>,GRBM_GUI_ACTIVE,1600000,0,100000\n"
        + "1,mxfp4::gemm_mx_kernel<0>,SQ_VALU_MFMA_BUSY_CYCLES,51200000,0,100000\n"
        + "1,mxfp4::gemm_mx_kernel<0>,SQ_INSTS_MFMA,1600000,0,100000\n"
        + "1,mxfp4::gemm_mx_kernel<0>,SQ_WAVE_CYCLES,1000,0,100000\n"
        + "1,mxfp4::gemm_mx_kernel<0>,SQ_WAIT_INST_ANY,250,0,100000\n"
        + "2,mxfp4::quant_rows_kernel,SQ_WAVE_CYCLES,5,0,100000\n")
    (run_b / "s_counter_collection.csv").write_text(
        head + "1,mxfp4::gemm_mx_kernel<0>,GRBM_GUI_ACTIVE,1600000,0,100000\n"
        + "1,mxfp4::gemm_mx_kernel<0>,SQ_LDS_BANK_CONFLICT,0,0,100000\n")
    out = tmp_path / "sq.md"
    bench.summarize_sq([str(tmp_path / "a"), str(tmp_path / "b")], str(out))
    text = out.read_text()
    assert "over 2 dispatches in 2 runs" in text
    assert "| dispatch duration under counters | 100.0 us |" in text
    assert "| busy cycles per XCD | 2e+05 (2.00 GHz) |" in text
    assert "| MFMA pipe busy, share of SIMD-cycles | 25.0 % |" in text      # 51.2e6 / (1024 * 2e5)
    assert "| MFMA busy cycles per MFMA instruction | 32.0 |" in text
    assert "| SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES | 25.0 % |" in text
    assert "| SQ_LDS_BANK_CONFLICT | 0 |" in text


def test_sweep_plan_covers_every_configuration():
    import workloads
    plan = bench.sweep_plan()
    assert sorted(plan) == [0, 1, 2, 3, 4, 5]
    for cfg, (calls, gemms) in plan.items():
        names = set(workloads.CONFIGS[cfg]["tensors"])
        for name, rnd, axis in calls:
            assert name in names and rnd in ("rtn", "sr") and axis in (0, 1)
        for gname, ca, cb in gemms:
            assert ca in calls and cb in calls
    # the training configurations time the three GEMMs of every linear layer
    for cfg in (4, 5):
        kinds = {g[0].split()[-1] for g in plan[cfg][1]}
        assert kinds == {"fwd", "dgrad", "wgrad"}


def test_clock_library_exports_what_bench_calls():
    """libmxclock.so (the benchmark's clock stamps and MFMA ceiling run) loads
    on the CPU and exports every function bench.py calls."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "microscaling_fp4_quantized_block_amd", "libmxclock.so"))
    for name in ("mxclock_stamp", "mxclock_stamp_slots", "mxclock_wall_rate_khz", "mxclock_mfma_ceiling",
                 "mxclock_ceiling_stamp_slots", "mxclock_ceiling_sink_slots", "mxclock_ceiling_mfmas_per_iter"):
        assert hasattr(lib, name), name
    lib.mxclock_ceiling_mfmas_per_iter.restype = ctypes.c_longlong
    assert lib.mxclock_ceiling_mfmas_per_iter() == 256 * 4 * 16
    assert lib.mxclock_ceiling_stamp_slots() == 512
