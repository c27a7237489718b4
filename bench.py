"""Benchmark of the microscaling-FP4 linear-layer hot path on one MI355X.

One step = quantize the activations A [4096, 8192] and the weights
B [14336, 8192] (bf16 -> MXFP4, round-to-nearest, no rotation), then the
block-scaled FP4 GEMM C = A B^T (M x N x K = 4096 x 14336 x 8192, FP32 out).
Inputs are seeded synthetic bf16 tensors resident in HBM before timing starts
(A ~ N(0, 1), B ~ N(0, 0.02); the pages' own datasets are not available).

Prints one JSON line.  `value` is the whole step's throughput expressed as
GEMM FLOP per second (2 M N K / step time); the per-kernel figures (GEMM
TFLOP/s against the dense-FP4 MFMA peak, quantizer GB/s against HBM) are in
`components`, and `roofline` reports the dominant kernel (the GEMM), timed
with HIP events on the stream it is launched on.  `cpu_baseline` times the
CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 GEMM TFLOPS + quantizer GB/s (4096×14336×8192) and % of 1-GPU roofline"
M, N, K = 4096, 14336, 8192
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense FP4 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
MX_BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0   # bf16 in, packed codes + E8M0 scale out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first: from idle, the GEMM runs 15-30 %% slower for the first "
                         "~10 ms (about 30 steps) and settles within ~70 ms")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "gemm_mx_headline_traffic.txt"),
                    help="HBM bytes per GEMM launch from rocprofv3 counters (written by --summarize-pmc)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy first (calibrates the PMC byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into the traffic file")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "OUT_MD"),
                    help="turn a rocprofv3 --stats kernel_stats.csv into a short markdown summary")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                    help="rocprofv3 --pmc run directories (SQ/GRBM counters) followed by the output .md: "
                         "MFMA-pipe utilisation and wave-cycle shares of the MXFP4 GEMM")
    ap.add_argument("--settle-trace", metavar="OUT_MD",
                    help="GEMM time per headline step over 1500 steps started from an idle GPU (window means)")
    ap.add_argument("--sweep", metavar="OUT_MD", nargs="?", const="-",
                    help="time every quantizer call and GEMM of all workload configurations against their "
                         "rooflines and write a markdown table (to stdout with no file)")
    ap.add_argument("--sweep-reps", type=int, default=10)
    ap.add_argument("--sweep-configs", default="1,2,3,4,5,0", help="comma-separated configurations to sweep")
    ap.add_argument("--quant-profile", action="store_true",
                    help="run a fixed list of quantizer calls (3 each, the MALL evicted before each) for "
                         "rocprofv3 kernel-trace and PMC runs")
    ap.add_argument("--summarize-quant", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR", "OUT_MD"),
                    help="per-kernel HBM traffic and achieved GB/s of the --quant-profile runs")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "mxfp4_build", os.path.join(ROOT, "microscaling_fp4_quantized_block_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def kernel_digest(compile_if_stale=False):
    """SHA-256 (16 hex digits) of the headline GEMM kernel's gfx950 assembly
    (gemm_mx_kernel, FP32 C) as recorded by the build; None when the record is
    missing or older than the sources (unless compile_if_stale)."""
    return _build_module().kernel_digests(compile_if_stale).get("gemm_mx_kernel_f32")


def gemm_traffic(path):
    """HBM bytes per launch of the GEMM kernel measured with rocprofv3 PMC
    counters (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads
    for a plain copy of known size); None when the file is missing or was
    measured on different kernel code."""
    try:
        with open(path) as f:
            d = json.loads(f.read().split("\n", 1)[1])
        digest = kernel_digest()
        if digest is None or d.get("gemm_isa_sha256_16") != digest:
            return None
        return float(d["bytes_per_launch"])
    except (OSError, ValueError, KeyError, IndexError):
        return None


def _pmc_per_kernel(run_dir, counter):
    """Average per-dispatch value of `counter` for each kernel name in a
    rocprofv3 --pmc csv run directory."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
                vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in vals.items()}


def summarize_pmc(fetch_dir, write_dir, out_path):
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    pick = lambda d, key: next(v for k, v in d.items() if key(k))
    is_gemm = lambda k: "gemm_mx_kernel" in k
    # the copy is the elementwise kernel with the largest counts (the fills of
    # the calibration and eviction buffers are separate, smaller or write-only)
    is_copy = lambda k: "elementwise" in k.lower() and "fill" not in k.lower()
    cands_f = [v[0] for k, v in fetch.items() if is_copy(k)]
    cands_w = [v[0] for k, v in write.items() if is_copy(k)]
    g_f, g_w = pick(fetch, is_gemm)[0], pick(write, is_gemm)[0]
    c_f, c_w = max(cands_f), max(cands_w)
    f_scale, w_scale = COPY_BYTES / c_f, COPY_BYTES / c_w     # bytes per counter unit
    fetched, written = g_f * f_scale, g_w * w_scale
    algorithmic = M * K // 2 + N * K // 2 + (M + N) * K // 32 + 4 * M * N
    d = {"bytes_per_launch": fetched + written, "fetched_bytes": fetched, "written_bytes": written,
         "algorithmic_bytes": algorithmic, "copy_calibration": {"bytes": COPY_BYTES, "fetch_counter": c_f,
                                                                "write_counter": c_w},
         "gemm_counters": {"FETCH_SIZE": g_f, "WRITE_SIZE": g_w},
         "gemm_isa_sha256_16": kernel_digest(compile_if_stale=True)}
    with open(out_path, "w") as f:
        f.write("HBM traffic of gemm_mx_kernel, 4096x14336x8192 MXFP4 (rocprofv3 PMC FETCH_SIZE / WRITE_SIZE, "
                "scaled by a 1 GiB copy; commands in profiles/README.md)\n")
        f.write(json.dumps(d, indent=1) + "\n")
    print(json.dumps(d, indent=1))


# The quantizer calls --quant-profile makes: (label, config, tensor, fmt, rounding, hadamard, axis).
QUANT_PROFILE_CALLS = [
    ("headline A", 0, "A", "mx", "rtn", False, 1),
    ("headline B", 0, "B", "mx", "rtn", False, 1),
    ("config 3 W_down (rotated)", 3, "W_down", "mx", "rtn", True, 1),
    ("config 2 X (NVFP4)", 2, "X", "nv", "rtn", False, 1),
    ("config 4 dY1 SR rows", 4, "dY1", "mx", "sr", False, 1),
    ("config 4 dY1 SR transposed", 4, "dY1", "mx", "sr", False, 0),
]


def quant_profile():
    """The calls of QUANT_PROFILE_CALLS, 3 times each, each after a 512 MiB
    write that evicts the MALL (device-drawn inputs with the configurations'
    shapes; the distributions do not change the traffic)."""
    import torch
    import workloads
    import microscaling_fp4_quantized_block_amd as mx
    dev = torch.device("cuda", 0)
    evict = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    for label, cfg, name, fmt, rnd, had, axis in QUANT_PROFILE_CALLS:
        shape = workloads.CONFIGS[cfg]["tensors"][name][0]
        x = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
        R, C = shape
        q = mx.empty_qtensor(fmt, R if axis == 1 else C, C if axis == 1 else R, had, dev)
        ws = torch.empty(max(mx.mxfp4_quantize_workspace_bytes(fmt, R, C, axis), 4), dtype=torch.uint8, device=dev)
        for _ in range(3):
            evict.fill_(1.0)
            mx.mxfp4_quantize(x, fmt, rnd, had, axis, 3, out=q, workspace=ws)
        torch.cuda.synchronize()
        print(f"[quant-profile] {label}: {fmt} {rnd} axis {axis} {R}x{C}", flush=True)
        del x, q, ws


def _dispatches(run_dir, counter=None):
    """Our kernels' dispatches of a rocprofv3 csv run in order: (name, value)
    with value = the counter (summed over its instances) or the duration."""
    import csv
    import glob
    out = {}
    pattern = "*counter_collection.csv" if counter else "*kernel_trace.csv"
    for path in glob.glob(os.path.join(run_dir, "**", pattern), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if counter is not None and r["Counter_Name"] != counter:
                    continue
                key = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
                val = float(r["Counter_Value"]) if counter else (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
                if key in out:
                    out[key] = (name, out[key][1] + val if counter else val)
                else:
                    out[key] = (name, val)
    return [out[k] for k in sorted(out)]


def summarize_quant(fetch_dir, write_dir, trace_dir, out_md):
    fetch, write, trace = _dispatches(fetch_dir, "FETCH_SIZE"), _dispatches(write_dir, "WRITE_SIZE"), _dispatches(trace_dir)
    is_copy = lambda k: "elementwise" in k.lower() and "fill" not in k.lower()
    f_scale = COPY_BYTES / max(v for k, v in fetch if is_copy(k))
    w_scale = COPY_BYTES / max(v for k, v in write if is_copy(k))
    ours = lambda lst: [(k, v) for k, v in lst if "mxfp4::" in k]
    fetch, write, trace = ours(fetch), ours(write), ours(trace)
    assert len(fetch) == len(write) == len(trace), (len(fetch), len(write), len(trace))
    # consecutive dispatches per call: 3 repetitions of one launcher's kernels
    rows, i = [], 0
    for label, cfg, name, fmt, rnd, had, axis in QUANT_PROFILE_CALLS:
        per_call = 3 if fmt == "nv" else 1
        for j in range(per_call):
            idx = [i + rep * per_call + j for rep in range(3)]
            kname = trace[idx[0]][0]
            t = sorted(trace[q][1] for q in idx)[1]
            fb = sum(fetch[q][1] for q in idx) / 3 * f_scale
            wb = sum(write[q][1] for q in idx) / 3 * w_scale
            short = kname.replace("void ", "").replace("mxfp4::", "").split("(")[0]
            rows.append((label, short, t * 1e6, fb / 1e6, wb / 1e6, (fb + wb) / t / 1e9))
        i += 3 * per_call
    with open(out_md, "w") as f:
        f.write("| call | kernel | us (median of 3) | fetched MB | written MB | actual GB/s | % of 8 TB/s |\n"
                "|---|---|---|---|---|---|---|\n")
        for r in rows:
            f.write("| %s | %s | %.1f | %.1f | %.1f | %.0f | %.1f |\n" % (r + (r[5] / PEAK_HBM_GBPS * 100,)))
    print(open(out_md).read())


def summarize_stats(stats_csv, out_md):
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    head = ""
    if os.path.exists(out_md):   # keep an existing file's description above the table
        with open(out_md) as f:
            text = f.read()
        head = text[:text.index("| kernel |")] if "| kernel |" in text else text
    with open(out_md, "w") as f:
        f.write(head)
        f.write("| kernel | calls | average us | min us | max us | share % |\n|---|---|---|---|---|---|\n")
        for r in rows:
            f.write("| %s | %s | %.1f | %.1f | %.1f | %.1f |\n" % (
                r["Name"][:90], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    print(open(out_md).read())


SIMDS, XCDS = 256 * 4, 8   # MI355X: 256 compute units of 4 SIMDs in 8 XCDs


def summarize_sq(dirs, out_md, kernel="gemm_mx_kernel"):
    """Per-dispatch averages of SQ/GRBM counters for one kernel over rocprofv3
    --pmc runs, and what they give: the clock (GRBM_GUI_ACTIVE counts each XCD's
    busy cycles, summed over the 8 XCDs), the MFMA pipe's busy share of all
    SIMD-cycles, busy cycles per MFMA instruction, and the shares of
    resident-wave cycles spent issuing and waiting."""
    import csv
    import glob
    vals, dur = {}, {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if kernel not in r["Kernel_Name"]:
                        continue
                    key = (d, r["Dispatch_Id"])
                    per = vals.setdefault(r["Counter_Name"], {})
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                    dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    mean = {c: sum(v.values()) / len(v) for c, v in vals.items()}
    t = sum(dur.values()) / len(dur)
    lines = [f"SQ/GRBM counters of {kernel} (rocprofv3 --pmc, per-dispatch averages over {len(dur)} dispatches "
             f"in {len(dirs)} runs; commands in profiles/README.md)", "",
             "| counter | per dispatch |", "|---|---|"]
    lines += [f"| {c} | {mean[c]:.4g} |" for c in sorted(mean)]
    lines += ["", f"| derived | value |", "|---|---|", f"| dispatch duration under counters | {t * 1e6:.1f} us |"]
    gui = mean.get("GRBM_GUI_ACTIVE")
    if gui:
        cyc = gui / XCDS
        lines.append(f"| busy cycles per XCD | {cyc:.4g} ({cyc / t / 1e9:.2f} GHz) |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            lines.append(f"| MFMA pipe busy, share of SIMD-cycles | {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * cyc) * 100:.1f} % |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("SQ_INSTS_MFMA"):
        lines.append(f"| MFMA busy cycles per MFMA instruction | {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / mean['SQ_INSTS_MFMA']:.1f} |")
    wc = mean.get("SQ_WAVE_CYCLES")
    if wc:
        for c in ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS"):
            if c in mean:
                lines.append(f"| {c} / SQ_WAVE_CYCLES | {mean[c] / wc * 100:.1f} % |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(out_md).read())


def settle_trace(out_md, steps=1500):
    """Headline steps from an idle GPU (2 s without work first), HIP events
    around each GEMM; the mean, min and max GEMM time per window of steps show
    how long the clock takes to settle."""
    import torch
    import microscaling_fp4_quantized_block_amd as mx
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    A = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    B = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    qa, qb = mx.empty_qtensor("mx", M, K, False, dev), mx.empty_qtensor("mx", N, K, False, dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    time.sleep(2.0)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        mx.mxfp4_quantize(A, "mx", "rtn", False, 1, 0, out=qa)
        mx.mxfp4_quantize(B, "mx", "rtn", False, 1, 0, out=qb)
        evs[i][0].record()
        mx.mxfp4_gemm(qa, qb, out=C)
        evs[i][1].record()
        if i % 100 == 99:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    bounds = list(range(0, 60, 5)) + list(range(60, steps + 1, 60))
    lines = [f"Headline GEMM ({M}x{N}x{K}) time per step, {steps} steps of `bench.py`'s step started after 2 s "
             "without GPU work (HIP events around each GEMM). Command: `python bench.py --settle-trace OUT_MD`.",
             "", "| steps | mean us | min us | max us |", "|---|---|---|---|"]
    for w0, w1 in zip(bounds[:-1], bounds[1:]):
        lines.append(f"| {w0}-{w1 - 1} | {t[w0:w1].mean():.1f} | {t[w0:w1].min():.1f} | {t[w0:w1].max():.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(out_md).read())


class ClockStamps:
    """Shader-clock stamps around the timed steps (libmxclock.so, built next to
    libmxfp4.so): each XCD's average shader clock over the steps is
    d(s_memtime) / d(s_memrealtime) times the real-time counter's rate."""

    def __init__(self, device):
        import ctypes
        import torch
        here = os.path.join(ROOT, "microscaling_fp4_quantized_block_amd", "libmxclock.so")
        self.lib = ctypes.CDLL(here)
        self.lib.mxclock_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.mxclock_stamp.restype = ctypes.c_int
        self.lib.mxclock_stamp_slots.restype = ctypes.c_int
        self.lib.mxclock_wall_rate_khz.restype = ctypes.c_int
        n = self.lib.mxclock_stamp_slots()
        self.buf = [torch.zeros(n, dtype=torch.int64, device=device) for _ in range(2)]
        self.device = device
        self.ctypes = ctypes

    def stamp(self, i):
        import torch
        stream = self.ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        if self.lib.mxclock_stamp(self.ctypes.c_void_p(self.buf[i].data_ptr()), stream) != 0:
            raise RuntimeError("clock stamp launch failed")

    def summary(self):
        rate_khz = self.lib.mxclock_wall_rate_khz()
        a, b = (t.cpu().numpy().view(np.uint64).reshape(-1, 3) for t in self.buf)
        # one stamp per place (XCD + compute unit) and launch; the clock of a
        # place that ran a workgroup of both launches
        s0 = {int(r[0]): r for r in a}
        s1 = {int(r[0]): r for r in b}
        mhz = {}
        for key in sorted(set(s0) & set(s1)):
            dt = int(s1[key][1]) - int(s0[key][1])
            dr = int(s1[key][2]) - int(s0[key][2])
            if dr > 0 and dt > 0:
                mhz[key] = dt / (dr / (rate_khz * 1e3)) / 1e6
        vals = np.array(list(mhz.values()))
        per_xcd = {}
        for key, v in mhz.items():
            per_xcd.setdefault(key >> 8, []).append(v)
        wall = float(np.median(b[:, 2].astype(np.int64) - a[:, 2].astype(np.int64))) / (rate_khz * 1e3) if rate_khz else None
        return {"sclk_mhz_median": round(float(np.median(vals)), 1) if len(vals) else None,
                "sclk_mhz_min": round(float(vals.min()), 1) if len(vals) else None,
                "sclk_mhz_max": round(float(vals.max()), 1) if len(vals) else None,
                "sclk_mhz_per_xcd": [round(float(np.median(per_xcd[x])), 1) for x in sorted(per_xcd)],
                "compute_units_paired": int(len(vals)),
                "wall_s": round(wall, 6) if wall is not None else None,
                "source": "s_memtime / s_memrealtime of each compute unit, stamped before and after the timed steps",
                "note": "s_memtime advances once per shader clock (the MFMA ceiling run counts 32 ticks per "
                        "32-cycle scaled FP4 MFMA)"}


def mfma_ceiling(device, kind=0, launches=6, iters=30000):
    """The MFMA rate the chip sustains with no memory traffic, on pseudo-random
    operands (libmxclock.so's ceiling kernel: one workgroup of four waves per
    compute unit, 16 independent accumulators per wave).  kind 0: the scaled
    FP4 32x32x64 MFMA of the MXFP4 GEMM; kind 1: the fp16 32x32x16 MFMA of the
    NVFP4 GEMM.  Run back to back for ~60 ms; the last launches are timed with
    events, and the kernel's own s_memtime / s_memrealtime stamps give the
    clock during them and the counter ticks per MFMA."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "microscaling_fp4_quantized_block_amd", "libmxclock.so"))
    lib.mxclock_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.mxclock_mfma_ceiling.restype = ctypes.c_int
    lib.mxclock_ceiling_mfmas_per_iter.restype = ctypes.c_longlong
    lib.mxclock_wall_rate_khz.restype = ctypes.c_int
    stamps = torch.zeros(lib.mxclock_ceiling_stamp_slots(), dtype=torch.int64, device=device)
    sink = torch.zeros(lib.mxclock_ceiling_sink_slots(), dtype=torch.float32, device=device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    timed = 2
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for i in range(launches):
        if i == launches - timed:
            ev[0].record()
        if lib.mxclock_mfma_ceiling(kind, iters, ctypes.c_void_p(stamps.data_ptr()),
                                    ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("MFMA ceiling launch failed")
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / timed
    mfmas = lib.mxclock_ceiling_mfmas_per_iter() * iters
    flop_per_mfma = 2.0 * 32 * 32 * (64 if kind == 0 else 16)
    peak = PEAK_FP4_TFLOPS if kind == 0 else PEAK_FP16_TFLOPS
    tflops = mfmas * flop_per_mfma / (ms * 1e-3) / 1e12
    st = stamps.cpu().numpy().view(np.uint64).reshape(-1, 2).astype(np.float64)
    rate_khz = lib.mxclock_wall_rate_khz()
    mhz = float(np.median(st[:, 0] / st[:, 1] * rate_khz / 1e3)) if rate_khz else None
    ticks = float(np.median(st[:, 0])) / (16.0 * iters)   # per wave: 16 MFMAs per iteration
    what = ("scaled FP4 MFMA 32x32x64 alone on pseudo-random codes" if kind == 0 else
            "fp16 MFMA 32x32x16 alone on random fp16 values")
    return {"tflops": round(tflops, 1), "frac_of_nominal_peak": round(tflops / peak, 4),
            "sclk_mhz": round(mhz, 1) if mhz else None, "ticks_per_mfma": round(ticks, 2),
            "ms_per_launch": round(ms, 3),
            "what": what + ", one workgroup of four waves per compute unit, no memory traffic; the clock it "
                           "holds is set by the power of random operands"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline():
    """The CPU oracle on a bounded sample of the step, scaled to the whole step."""
    import oracle
    import workloads
    os.environ.setdefault("OMP_NUM_THREADS", str(len(os.sched_getaffinity(0))))
    cores = int(os.environ["OMP_NUM_THREADS"])       # threads the OpenMP oracle runs with
    oracle._load()
    # about 10-15 s of oracle work on 16 cores: both quantizations whole, and
    # 4096 x 8192 of the 4096 x 14336 GEMM outputs
    qa_rows, qb_rows, g_rows, g_cols = M, N, 4096, 8192
    A = workloads.make_tensor(0, "A", rows=qa_rows)
    B = workloads.make_tensor(0, "B", rows=qb_rows)
    t0 = time.perf_counter()
    qa = oracle.quantize(A, "mx", "rtn")
    t1 = time.perf_counter()
    qb = oracle.quantize(B, "mx", "rtn")
    t2 = time.perf_counter()
    oracle.gemm("mx", qa, qb, rows=np.arange(g_rows), cols=np.arange(g_cols))
    t3 = time.perf_counter()
    step_s = ((t1 - t0) * (M / qa_rows) + (t2 - t1) * (N / qb_rows)
              + (t3 - t2) * (M * N) / (g_rows * g_cols))
    return {
        "value": 2.0 * M * N * K / step_s / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"quantize {qa_rows} of {M} rows of A and {qb_rows} of {N} rows of B, "
                   f"fp64 GEMM of {g_rows}x{g_cols} outputs (K={K}); each part scaled to the full step"),
        "sample_seconds": round(t3 - t0, 2),
        "step_seconds_extrapolated": round(step_s, 1),
    }


PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA (the exact NVFP4 path)

# The hot-path calls of each workload configuration: quantizer calls
# (tensor, rounding, axis) and GEMMs (A call, B call).  Config 3's weights are
# quantized once offline in the method; their quantization is timed too.
# Config 4: fc1 = (X1, W1, dY1), fc2 = (X2, W2, dY2); config 5: one
# (input, weight, output gradient) triple per projection.  Forward X W^T takes
# both operands RTN along K; dgrad dY W takes dY along N (axis 1) and W along
# its rows (axis 0); wgrad dY^T X takes both along the token axis (axis 0);
# backward operands use stochastic rounding.
def _training_gemms(triples):
    calls, gemms = [], []
    for name, (x, w, dy) in triples.items():
        q = [(x, "rtn", 1), (w, "rtn", 1), (dy, "sr", 1), (w, "sr", 0), (dy, "sr", 0), (x, "sr", 0)]
        calls += q
        gemms += [(name + " fwd", q[0], q[1]), (name + " dgrad", q[2], q[3]), (name + " wgrad", q[4], q[5])]
    return calls, gemms


class GraphTimer:
    """GPU time of one call from HIP graphs of `inner` back-to-back calls
    (replays cost no Python, ctypes or event time per call): the graph is
    replayed back to back for ~30 ms first (from idle the clock needs ~10 ms
    of load to settle), then the median of `reps` timed replays, per call.
    With evict_first, each call is preceded by a 512 MiB write that evicts the
    MALL, and that write's own time (timed the same way) is subtracted."""

    inner = 8

    def __init__(self, device, reps):
        import torch
        self.torch = torch
        self.reps = reps
        self.evict = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=device)
        self.t_evict = self.replay_time(self.graph_of(lambda: self.evict.fill_(1.0)))

    def graph_of(self, fn):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(self.inner):
                fn()
        torch.cuda.synchronize()
        return g

    def replay_time(self, g):
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        for _ in range(min(5000, int(30.0 / max(e0.elapsed_time(e1), 1e-3)) + 1)):
            g.replay()
        torch.cuda.synchronize()
        ts = []
        for i in range(self.reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)) * 1e-3 / self.inner

    def timed(self, fn, evict_first):
        """Seconds per call of fn."""
        if evict_first:
            def both():
                self.evict.fill_(1.0)
                fn()
            return max(self.replay_time(self.graph_of(both)) - self.t_evict, 1e-7)
        return self.replay_time(self.graph_of(fn))


def sweep_plan():
    plan = {}
    c = [("X", "rtn", 1), ("W", "rtn", 1)]
    plan[1] = (c, [("fwd", c[0], c[1])])
    plan[2] = (c, [("fwd", c[0], c[1])])
    c3 = [(t, "rtn", 1) for t in ("W_up", "W_down", "x_dec_up", "x_pre_up", "x_dec_down", "x_pre_down")]
    plan[3] = (c3, [("decode up", c3[2], c3[0]), ("prefill up", c3[3], c3[0]),
                    ("decode down", c3[4], c3[1]), ("prefill down", c3[5], c3[1])])
    plan[4] = _training_gemms({"fc1": ("X1", "W1", "dY1"), "fc2": ("X2", "W2", "dY2")})
    plan[5] = _training_gemms({"qkv": ("X", "W_qkv", "dY_qkv"), "o": ("X", "W_o", "dY_o"),
                               "gate": ("X", "W_gate", "dY_gate"), "up": ("X", "W_up", "dY_gate"),
                               "down": ("X_down", "W_down", "dY_down")})
    c0 = [("A", "rtn", 1), ("B", "rtn", 1)]
    plan[0] = (c0, [("fwd", c0[0], c0[1])])
    return plan


def sweep(args):
    """Every quantizer call and GEMM of every configuration, timed with HIP
    events around replays of a HIP graph holding 8 back-to-back calls (median
    of --sweep-reps; for quantizer calls each call is preceded by a 512 MiB
    write that evicts the MALL, whose own time is subtracted), against its
    roofline.  Inputs are drawn
    on the device with the configurations' distributions (normal std, or
    Student-t with outlier channels), seeded."""
    import torch
    import workloads
    import microscaling_fp4_quantized_block_amd as mx
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)

    def draw(cfg, name):
        shape, kw = workloads.CONFIGS[cfg]["tensors"][name]
        gen.manual_seed(1000 * cfg + list(workloads.CONFIGS[cfg]["tensors"]).index(name))
        torch.manual_seed(1000 * cfg + list(workloads.CONFIGS[cfg]["tensors"]).index(name))
        if kw["kind"] == "normal":
            x = torch.randn(shape, generator=gen, device=dev) * kw["std"]
        else:
            nu = kw["nu"]
            z = torch.randn(shape, generator=gen, device=dev)
            chi2 = torch.distributions.Chi2(torch.tensor(nu, device=dev)).sample(shape)
            x = z / torch.sqrt(chi2 / nu)
            if kw.get("outlier_frac", 0.0) > 0:
                ch = torch.randperm(shape[1], generator=gen, device=dev)[: int(round(kw["outlier_frac"] * shape[1]))]
                x[:, ch] *= kw.get("outlier_scale", 50.0)
        return x.to(torch.bfloat16)

    gt = GraphTimer(dev, args.sweep_reps)
    timed = gt.timed

    rows = []

    def add_row(r):
        rows.append(r)
        print("[sweep] " + " | ".join(str(v) for v in r[:5]), file=sys.stderr, flush=True)

    wanted = [int(c) for c in args.sweep_configs.split(",")]
    for cfg, (calls, gemms) in sweep_plan().items():
        if cfg not in wanted:
            continue
        print(f"[sweep] config {cfg}", file=sys.stderr, flush=True)
        spec = workloads.CONFIGS[cfg]
        fmt, had = spec["fmt"], spec["hadamard"]
        bs = 32 if fmt == "mx" else 16
        tens, qs = {}, {}
        for (name, rnd, axis) in dict.fromkeys(calls):
            if name not in tens:
                tens[name] = draw(cfg, name)
            x = tens[name]
            R, Cc = x.shape
            rows_, k = (R, Cc) if axis == 1 else (Cc, R)
            q = mx.empty_qtensor(fmt, rows_, k, had, dev)
            wsb = mx.mxfp4_quantize_workspace_bytes(fmt, R, Cc, axis)
            ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
            f = lambda x=x, q=q, ws=ws, rnd=rnd, axis=axis: mx.mxfp4_quantize(x, fmt, rnd, had, axis, 7, out=q,
                                                                               workspace=ws)
            t = timed(f, True)
            qs[(name, rnd, axis)] = q
            nbytes = R * Cc * (2.0 + 0.5 + 1.0 / bs) + (4 if fmt == "nv" else 0)
            gbps = nbytes / t / 1e9
            add_row((cfg, "quantize", f"{name} {rnd} axis{axis}" + (" H" if had else ""), f"{R}x{Cc}",
                         t * 1e6, gbps, "GB/s", "hbm", gbps / PEAK_HBM_GBPS))
        for (gname, ca, cb) in gemms:
            qa, qb = qs[ca], qs[cb]
            Mg, Ng, Kg = qa.rows, qb.rows, qa.k
            C = torch.empty((Mg, Ng), dtype=torch.float32, device=dev)
            wsb = mx.mxfp4_gemm_workspace_bytes(qa, qb)
            ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
            t = timed(lambda: mx.mxfp4_gemm(qa, qb, out=C, workspace=ws), False)
            flops = 2.0 * Mg * Ng * Kg
            nbytes = (Mg + Ng) * Kg * (0.5 + 1.0 / bs) + 4.0 * Mg * Ng
            peak = PEAK_FP4_TFLOPS if fmt == "mx" else PEAK_FP16_TFLOPS
            bound_t = max(flops / (peak * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9))
            bound = "mfma" if flops / (peak * 1e12) >= nbytes / (PEAK_HBM_GBPS * 1e9) else "hbm"
            tf = flops / t / 1e12
            add_row((cfg, "gemm", gname, f"{Mg}x{Ng}x{Kg}", t * 1e6, tf, "TFLOP/s",
                         bound + ("-fp16" if fmt == "nv" and bound == "mfma" else ""), bound_t / t))
            if cfg in (0, 3):
                # the same GEMM writing bf16 (inference consumers): 2 bytes per output
                Cb = torch.empty((Mg, Ng), dtype=torch.bfloat16, device=dev)
                tb = timed(lambda: mx.mxfp4_gemm_bf16(qa, qb, out=Cb, workspace=ws), False)
                nbytes_b = nbytes - 2.0 * Mg * Ng
                bound_tb = max(flops / (peak * 1e12), nbytes_b / (PEAK_HBM_GBPS * 1e9))
                bound_b = "mfma" if flops / (peak * 1e12) >= nbytes_b / (PEAK_HBM_GBPS * 1e9) else "hbm"
                add_row((cfg, "gemm_bf16", gname, f"{Mg}x{Ng}x{Kg}", tb * 1e6, flops / tb / 1e12, "TFLOP/s",
                             bound_b, bound_tb / tb))
                del Cb
            del C, ws
        if cfg in (2, 3, 5):
            # weights with MSE-fitted scales (two alternations for NVFP4)
            for name in [n for n in tens if n.startswith("W")]:
                x = tens[name]
                R, Cc = x.shape
                q = mx.empty_qtensor(fmt, R, Cc, had, dev)
                wsb = mx.mxfp4_quantize_mse_workspace_bytes(fmt, had, R, Cc, 1)
                ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
                t = timed(lambda: mx.mxfp4_quantize_mse(x, fmt, had, 1, 2, out=q, workspace=ws), True)
                nbytes = R * Cc * (2.0 + 0.5 + 1.0 / bs) + (4 if fmt == "nv" else 0)
                gbps = nbytes / t / 1e9
                add_row((cfg, "quantize_mse", f"{name} rtn axis1" + (" H" if had else "") + (" 2 rounds" if fmt == "nv" else ""),
                             f"{R}x{Cc}", t * 1e6, gbps, "GB/s", "hbm", gbps / PEAK_HBM_GBPS))
                del q, ws
        if cfg in (4, 5):
            # signal / noise sums of the stochastically rounded gradient
            # operands (one pass over x, codes and scales)
            for (name, rnd, axis), q in qs.items():
                if rnd != "sr" or not name.startswith("dY"):
                    continue
                x = tens[name]
                st = torch.empty(3, dtype=torch.float64, device=dev)
                ws = torch.empty(mx.mxfp4_quantization_noise_workspace_bytes(q), dtype=torch.uint8, device=dev)
                t = timed(lambda: mx.mxfp4_quantization_noise(x, q, axis, out=st, workspace=ws), True)
                R, Cc = x.shape
                nbytes = R * Cc * (2.0 + 0.5 + 1.0 / bs)
                gbps = nbytes / t / 1e9
                add_row((cfg, "noise", f"{name} {rnd} axis{axis}", f"{R}x{Cc}", t * 1e6, gbps, "GB/s", "hbm",
                             gbps / PEAK_HBM_GBPS))
                # the same sums computed while quantizing (one pass; bytes:
                # the quantizer's, input once + codes and scales written)
                qf = mx.empty_qtensor(fmt, q.rows, q.k, had, dev)
                fws = torch.empty(mx.mxfp4_quantize_noise_workspace_bytes(fmt, had, R, Cc, axis), dtype=torch.uint8,
                                  device=dev)
                tf = timed(lambda: mx.mxfp4_quantize_noise(x, fmt, rnd, had, axis, 5, out=qf, stats=st,
                                                           workspace=fws), True)
                gbps_f = R * Cc * (2.0 + 0.5 + 1.0 / bs) / tf / 1e9
                add_row((cfg, "quantize+noise", f"{name} {rnd} axis{axis} (fused)", f"{R}x{Cc}", tf * 1e6, gbps_f,
                             "GB/s", "hbm", gbps_f / PEAK_HBM_GBPS))
                del st, ws, qf, fws
        if cfg == 3:
            # the decode linear layer through mxfp4_quantize_gemm (for these
            # shapes: the activations quantized into the workspace, then the
            # decode GEMM), against the same two calls made separately
            for gname, xname, wname in (("decode up", "x_dec_up", "W_up"), ("decode down", "x_dec_down", "W_down")):
                x, qw, qx = tens[xname], qs[(wname, "rtn", 1)], qs[(xname, "rtn", 1)]
                Mg, Kg = x.shape
                Ng = qw.rows
                C = torch.empty((Mg, Ng), dtype=torch.float32, device=dev)
                wsb = mx.mxfp4_quantize_gemm_workspace_bytes(Mg, Kg, had, qw)
                ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
                gws = torch.empty(max(mx.mxfp4_gemm_workspace_bytes(qx, qw), 4), dtype=torch.uint8, device=dev)
                flops = 2.0 * Mg * Ng * Kg
                nbytes = Mg * Kg * 2.0 + Ng * Kg * (0.5 + 1.0 / bs) + 4.0 * Mg * Ng
                bound_t = max(flops / (PEAK_FP4_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9))
                bound = "mfma" if flops / (PEAK_FP4_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBPS * 1e9) else "hbm"
                t_f = timed(lambda: mx.mxfp4_quantize_gemm(x, qw, had, out=C, workspace=ws), False)

                def two():
                    mx.mxfp4_quantize(x, fmt, "rtn", had, 1, 7, out=qx)
                    mx.mxfp4_gemm(qx, qw, out=C, workspace=gws)
                t_2 = timed(two, False)
                for label, t in (("quantize_gemm", t_f), ("quantize, then gemm", t_2)):
                    add_row((cfg, "quantize+gemm", f"{gname} ({label})", f"{Mg}x{Ng}x{Kg}", t * 1e6,
                                 flops / t / 1e12, "TFLOP/s", bound, bound_t / t))
                del C, ws, gws
            # prefill up with its output quantized (rotated) for the down
            # projection, in the GEMM's epilogue, against the two launches it
            # replaces (bf16 GEMM, then quantize); bytes: operands + 0.53 B out
            qx, qw = qs[("x_pre_up", "rtn", 1)], qs[("W_up", "rtn", 1)]
            Mg, Ng, Kg = qx.rows, qw.rows, qx.k
            qo = mx.empty_qtensor("mx", Mg, Ng, True, dev)
            Cb = torch.empty((Mg, Ng), dtype=torch.bfloat16, device=dev)
            gws = torch.empty(max(mx.mxfp4_gemm_workspace_bytes(qx, qw), 4), dtype=torch.uint8, device=dev)
            flops = 2.0 * Mg * Ng * Kg
            t_f = timed(lambda: mx.mxfp4_gemm_quantize(qx, qw, True, out=qo), False)

            def two_q():
                mx.mxfp4_gemm_bf16(qx, qw, out=Cb, workspace=gws)
                mx.mxfp4_quantize(Cb, "mx", "rtn", True, 1, 0, out=qo)
            t_2 = timed(two_q, False)
            nbytes = (Mg + Ng) * Kg * (0.5 + 1.0 / 32) + Mg * Ng * (0.5 + 1.0 / 32)
            bound_t = max(flops / (PEAK_FP4_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9))
            for label, t in (("epilogue", t_f), ("bf16 GEMM + quantize", t_2)):
                add_row((cfg, "gemm+quantize C", f"prefill up, C quantized with H ({label})", f"{Mg}x{Ng}x{Kg}",
                             t * 1e6, flops / t / 1e12, "TFLOP/s", "mfma", bound_t / t))
            del qo, Cb, gws
            # the weights with a fixed grid scale (alpha = 0.75, rotated)
            for name in ("W_up", "W_down"):
                x = tens[name]
                R, Cc = x.shape
                q = mx.empty_qtensor("mx", R, Cc, True, dev)
                t = timed(lambda: mx.mxfp4_quantize_grid(x, 0.75, True, 1, out=q), True)
                gbps = R * Cc * (2.0 + 0.5 + 1.0 / 32) / t / 1e9
                add_row((cfg, "quantize_grid", f"{name} alpha 0.75 H", f"{R}x{Cc}", t * 1e6, gbps, "GB/s", "hbm",
                             gbps / PEAK_HBM_GBPS))
                del q
        if cfg == 4:
            # Q-EMA step of the weights: bf16 w + fp32 average in, fp32
            # average + codes + scales out (10.53 B per element)
            for name in ("W1", "W2"):
                w = tens[name] if name in tens else draw(cfg, name)
                R, Cc = w.shape
                m = w.float().clone()
                q = mx.empty_qtensor("mx", R, Cc, False, dev)
                t = timed(lambda: mx.mxfp4_qema_quantize(w, m, 0.999, False, out=q), True)
                gbps = R * Cc * (2.0 + 4.0 + 4.0 + 0.5 + 1.0 / 32) / t / 1e9
                add_row((cfg, "qema", f"{name} beta 0.999", f"{R}x{Cc}", t * 1e6, gbps, "GB/s", "hbm",
                             gbps / PEAK_HBM_GBPS))
                del m, q
        del tens, qs
        torch.cuda.empty_cache()
    lines = ["| config | kernel | call | shape | time us | achieved | unit | bound | frac of roofline |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %d | %s | %s | %s | %.1f | %.0f | %s | %s | %.3f |" % r)
    # the compute ceilings the chip holds on random operands, measured right
    # after the sweep (the GEMM rows' mfma fractions are against the nominal peaks)
    lines += ["", "MFMA ceilings on random operands, measured right after the rows above "
              "(`mfma_ceiling` in bench.py; no memory traffic):", "",
              "| MFMA | TFLOP/s | frac of nominal peak | clock MHz | s_memtime ticks per MFMA |",
              "|---|---|---|---|---|"]
    for kind, name in ((0, "scaled FP4 32x32x64 (MXFP4 GEMM)"), (1, "fp16 32x32x16 (NVFP4 GEMM)")):
        c = mfma_ceiling(dev, kind)
        lines.append("| %s | %.0f | %.3f | %.0f | %.2f |" % (name, c["tflops"], c["frac_of_nominal_peak"],
                                                             c["sclk_mhz"] or 0.0, c["ticks_per_mfma"]))
    text = "\n".join(lines) + "\n"
    if args.sweep == "-":
        print(text)
    else:
        # an existing file keeps its description above the table
        head = ""
        if os.path.exists(args.sweep):
            old = open(args.sweep).read()
            if lines[0] in old:
                head = old[:old.index(lines[0])]
        with open(args.sweep, "w") as f:
            f.write(head + text)
        print(text)


def main():
    args = parse()
    if args.sweep:
        sweep(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.traffic_file)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_quant:
        summarize_quant(*args.summarize_quant)
        return
    if args.settle_trace:
        settle_trace(args.settle_trace)
        return
    if args.summarize_sq:
        if len(args.summarize_sq) < 2:
            sys.exit("--summarize-sq takes one or more run directories, then the output file")
        summarize_sq(args.summarize_sq[:-1], args.summarize_sq[-1])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library runs the hot path "
              "on a single MI355X; a multi-GPU layer would shard the GEMM's N or M dimension across devices)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    import microscaling_fp4_quantized_block_amd as mx

    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        # a plain elementwise copy of COPY_BYTES whose source is not cache
        # resident (a 512 MiB write in between evicts the 256 MiB MALL)
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        evict = torch.zeros((512 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)          # one elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst, evict
    if args.quant_profile:
        quant_profile()
        return
    A_bits = workloads.make_tensor(0, "A")
    B_bits = workloads.make_tensor(0, "B")
    A = torch.from_numpy(A_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    B = torch.from_numpy(B_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    qa = mx.empty_qtensor("mx", M, K, False, dev)
    qb = mx.empty_qtensor("mx", N, K, False, dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    mx.mxfp4_quantize(A, "mx", "rtn", False, 1, 0, out=qa)
    mx.mxfp4_quantize(B, "mx", "rtn", False, 1, 0, out=qb)
    ws_bytes = mx.mxfp4_gemm_workspace_bytes(qa, qb)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    # ev: events recorded on the launch stream (torch's current stream, which
    # the binding passes to the library) around the GEMM
    def step(ev=None):
        mx.mxfp4_quantize(A, "mx", "rtn", False, 1, 0, out=qa)
        mx.mxfp4_quantize(B, "mx", "rtn", False, 1, 0, out=qb)
        if ev is not None:
            ev[0].record()
        mx.mxfp4_gemm(qa, qb, out=C, workspace=ws)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    new_events = lambda: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    events = new_events()
    clock = ClockStamps(dev)
    torch.cuda.synchronize()
    clock.stamp(0)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    clock.stamp(1)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    g_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    # the quantizer components, after the timed region: each call timed as in
    # the sweep (HIP graphs of 8 back-to-back calls, each after a 512 MiB write
    # that evicts the MALL as the step's GEMM does, that write's time
    # subtracted), so no event or launch gap is counted in a kernel's rate
    gt = GraphTimer(dev, 10)
    qa_ms = 1e3 * gt.timed(lambda: mx.mxfp4_quantize(A, "mx", "rtn", False, 1, 0, out=qa), True)
    qb_ms = 1e3 * gt.timed(lambda: mx.mxfp4_quantize(B, "mx", "rtn", False, 1, 0, out=qb), True)
    del gt
    ceiling = mfma_ceiling(dev)

    flops = 2.0 * M * N * K
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    qa_gbps = M * K * MX_BYTES_PER_ELEM / (qa_ms * 1e-3) / 1e9
    qb_gbps = N * K * MX_BYTES_PER_ELEM / (qb_ms * 1e-3) / 1e9
    traffic = gemm_traffic(args.traffic_file)
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "mx-rtn-4096x14336x8192", "M": M, "N": N, "K": K, "fmt": "mxfp4",
                   "rounding": "rtn", "hadamard": False,
                   "step": "quantize A + quantize B + FP4 GEMM", "parallelism": "none (1 GPU)"},
        "components": {
            "gemm": {"ms": round(g_ms, 4), "tflops": round(gemm_tflops, 1),
                     "frac_of_fp4_peak": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "frac_of_mfma_ceiling": round(gemm_tflops / ceiling["tflops"], 4)},
            "quantize_A": {"ms": round(qa_ms, 4), "gbps": round(qa_gbps, 1),
                           "frac_of_hbm_peak": round(qa_gbps / PEAK_HBM_GBPS, 4)},
            "quantize_B": {"ms": round(qb_ms, 4), "gbps": round(qb_gbps, 1),
                           "frac_of_hbm_peak": round(qb_gbps / PEAK_HBM_GBPS, 4)},
        },
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": traffic},
        "clock": clock.summary(),
        "mfma_ceiling": ceiling,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
