"""Throughput of the fused attention path on one MI355X, next to the CPU oracle.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward (O and LSE) and the recompute backward (row-term preprocess,
dK/dV pass, dQ pass) for the fwd+bwd workload; the forward alone for the
forward-only workloads. Inputs are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line. `value` is algorithmic TFLOP/s of a step (4*d flops per
allowed (query, key) pair forward, 2.5x that backward; masked pairs and the
backward's recomputed products are not credited). The backward runs through
its three pass entry points, with a HIP event between consecutive kernels, so
the same timed steps give each kernel's average launch duration; the
roofline object is computed for the kernel with the largest one.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic_inputs as si  # noqa: E402

METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak at 1 MI355X vs CPU oracle"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEFAULT_WORKLOAD = "c5_bwd_d128"
# Default warm-up: the chip raises its clock over the first few tens of
# milliseconds of load; five steps of a 0.3 ms workload left it measurably
# slower (C3's forward 0.347 ms against 0.272 ms after 100 steps).
WARMUP_MIN_STEPS = 5
WARMUP_SECONDS = 0.3


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps; by default at least %d, and as many as %.1f s of "
                         "steps take, so that the chip's clocks have settled before the timed "
                         "steps (short steps otherwise run at a lower clock)" % (WARMUP_MIN_STEPS, WARMUP_SECONDS))
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(si.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="rough CPU budget for the oracle leg (it times whole heads)")
    ap.add_argument("--calibration-copy-mib", type=int, default=256,
                    help="size of the plain copy kernel run once after timing (its HBM counters "
                         "calibrate the byte counters of the attention kernels); 0 disables")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "BENCH_JSON", "OUT_MD"),
                    help="turn a rocprofv3 --kernel-trace --stats run of this script and the JSON "
                         "line of a bench run into a markdown summary and exit")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE) "
                         "into a traffic summary file and exit")
    ap.add_argument("--summarize-busy", nargs=3, metavar=("GRBM_DIR", "MFMA_DIR", "OUT"),
                    help="turn two rocprofv3 --pmc runs of this script (GRBM_GUI_ACTIVE, then "
                         "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES) into a clock and matrix-core "
                         "busy summary and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "OUT"),
                    help="tabulate the per-dispatch averages of every counter of a rocprofv3 "
                         "--pmc run of this script for the attention kernels and exit")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="time the matrix-core rate probe on N(0,1) bf16 operands (and on zeros) "
                         "and print one JSON line instead of the attention bench")
    ap.add_argument("--summarize-waves", nargs=2, metavar=("PMC_DIR", "OUT"),
                    help="turn a rocprofv3 --pmc run of this script with the SQ wave-state "
                         "counters into a per-kernel breakdown of wave time and exit")
    return ap.parse_args()


def kernel_flop_credit(w):
    """Algorithmic flops credited to each kernel of a step (per launch).

    Forward kernel: 4*d per allowed pair (S = Q K^T and O = P V).
    Backward (5 products, 10*d per pair): the dK/dV pass is credited dV, dK
    and half of the shared recomputed S and dP (6*d per pair); the dQ pass dQ
    and the other halves (4*d per pair). The row-term preprocess does no
    matrix work and is credited its bytes instead.
    """
    pairs = w.pairs() * w.B * w.Hq
    return {
        "fwd": 4.0 * w.d * pairs,
        "bwd_dkdv": 6.0 * w.d * pairs,
        "bwd_dq": 4.0 * w.d * pairs,
    }


# Files each kernel is built from (relative to the package); the build script
# is included because its flags change the generated code.
_COMMON = ["csrc/attn_device.h", "csrc/attn_kernels.h", "build.py"]
KERNEL_SOURCES = {
    "fwd_kernel": ["csrc/attn_fwd.hip", *_COMMON],
    "bwd_dkdv_kernel": ["csrc/attn_bwd.hip", "csrc/attn_bwd_common.h", *_COMMON],
    "bwd_pre_kernel": ["csrc/attn_bwd.hip", "csrc/attn_bwd_common.h", *_COMMON],
    "bwd_dq_kernel": ["csrc/attn_bwd_dq.hip", "csrc/attn_bwd_common.h", *_COMMON],
    "decode_split_kernel": ["csrc/attn_decode.hip", *_COMMON],
    "decode_merge_kernel": ["csrc/attn_decode.hip", *_COMMON],
}
# The decode call launches the split kernel and then the merge kernel; it is
# timed (and its traffic summed) as one unit.
DECODE_UNIT = "decode_split_kernel+decode_merge_kernel"
CALIBRATION_KERNEL = "neg_kernel"


def source_hash(kernel):
    """sha256 over the sources a kernel is built from (traffic numbers are
    only reported for the source they were measured on)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_attention_12_amd", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was measured on other source."""
    if kernel == DECODE_UNIT:
        parts = [read_traffic(k, workload) for k in kernel.split("+")]
        return None if None in parts else sum(parts)
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash(kernel):
        return None
    return float(kv["hbm_bytes_per_launch"])


def summarize_pmc(fetch_dir, write_dir, out_dir, workload, mib):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from two
    rocprofv3 --pmc runs, scaled by what the same counters read for the
    calibration copy (which moves a known number of bytes each way)."""
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        acc = {}
        for f in files:
            for row in csv.DictReader(open(f)):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                acc.setdefault(name, []).append(float(row["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")

    def find(d, key):
        hits = [k for k in d if key in k]
        if not hits:
            raise SystemExit(f"kernel {key} not found in counters: {sorted(d)[:6]}")
        return hits[0]

    cal_f = fetch[find(fetch, CALIBRATION_KERNEL)]
    cal_w = write[find(write, CALIBRATION_KERNEL)]
    # The calibration kernel reads and writes `mib` MiB each (float32 negate).
    known_kib = mib * 1024.0
    sf, sw = known_kib / cal_f, known_kib / cal_w
    os.makedirs(out_dir, exist_ok=True)
    written = []
    for kernel in ("fwd_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel", "bwd_pre_kernel",
                   "decode_split_kernel", "decode_merge_kernel"):
        # the dK/dV pass runs the 64-keys-per-wave kernel on large d = 128 grids,
        # the forward and the dQ pass their 16x16x32-product kernels on large
        # d = 128 grids, the forward the key-split kernel on short sequences
        prefixes = [f"{kernel}<"] + (["bwd_dkdv_wide_kernel<"] if kernel == "bwd_dkdv_kernel" else []) + \
            (["fwd_m16_kernel<", "fwd_split_kernel<"] if kernel == "fwd_kernel" else []) + \
            (["bwd_dq_m16_kernel<"] if kernel == "bwd_dq_kernel" else [])
        hits = [(pf, k) for pf in prefixes for k in fetch if pf in k]
        if not hits:
            continue
        try:
            kf, kw = hits[0][1], find(write, hits[0][0])
        except SystemExit:
            continue
        fb = fetch[kf] * sf * 1024.0
        wb = write[kw] * sw * 1024.0
        path = traffic_file(kernel, workload)
        with open(path, "w") as f:
            f.write(f"# HBM traffic of {kernel} on {workload}, from rocprofv3 counters.\n")
            f.write(f"# Commands (run from the repository root on the MI355X box):\n")
            f.write(f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d <fetch_dir> -- python bench.py "
                    f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline\n")
            f.write(f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d <write_dir> -- python bench.py "
                    f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline\n")
            f.write(f"#   python bench.py --workload {workload} --summarize-pmc <fetch_dir> <write_dir> profiles\n")
            f.write(f"kernel_symbol = {kf}\n")
            f.write(f"fetch_size_kib_per_dispatch = {fetch[kf]:.1f}\n")
            f.write(f"write_size_kib_per_dispatch = {write[kw]:.1f}\n")
            f.write(f"calibration_kernel = {CALIBRATION_KERNEL} ({mib} MiB read + {mib} MiB written)\n")
            f.write(f"calibration_fetch_kib = {cal_f:.1f}\n")
            f.write(f"calibration_write_kib = {cal_w:.1f}\n")
            f.write(f"fetch_scale = {sf:.4f}\n")
            f.write(f"write_scale = {sw:.4f}\n")
            f.write(f"hbm_read_bytes_per_launch = {fb:.0f}\n")
            f.write(f"hbm_write_bytes_per_launch = {wb:.0f}\n")
            f.write(f"hbm_bytes_per_launch = {fb + wb:.0f}\n")
            f.write(f"source_sha256 = {source_hash(kernel)}\n")
        written.append(path)
    print("\n".join(written))


XCDS = 8            # MI355X: 8 accelerator complex dies, 32 CUs each
SIMDS = 256 * 4     # 4 SIMDs per compute unit


def summarize_busy(grbm_dir, mfma_dir, out, workload):
    """Effective clock and matrix-core busy fraction of each attention kernel
    from two rocprofv3 --pmc runs. GRBM_GUI_ACTIVE comes back summed over the
    XCDs, so the cycles of one kernel are its value / XCDS and the clock is
    that over the dispatch's own start/end timestamps.
    SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD, so / SIMDS gives the
    busy cycles of the average SIMD; its ratio to the kernel's cycles is the
    share of the time the matrix cores work."""
    import csv
    import glob

    def rows(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            yield from csv.DictReader(open(f))

    def per_kernel(d, counter):
        acc = {}
        for r in rows(d):
            if r.get("Counter_Name") != counter:
                continue
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            acc.setdefault(r["Kernel_Name"], []).append((float(r["Counter_Value"]), dur))
        return acc

    grbm = per_kernel(grbm_dir, "GRBM_GUI_ACTIVE")
    mfma = per_kernel(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    with open(out, "w") as f:
        f.write(f"# Clock and matrix-core busy fraction on {workload}, from rocprofv3 counters.\n")
        f.write("# Commands (run from the repository root on the MI355X box):\n")
        if os.path.abspath(grbm_dir) == os.path.abspath(mfma_dir):
            f.write(f"#   rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES -f csv -d <dir> -- "
                    f"python bench.py --workload {workload} --steps 2 --no-cpu-baseline\n")
            f.write(f"#   python bench.py --workload {workload} --summarize-busy <dir> <dir> <this file>\n")
        else:
            f.write(f"#   rocprofv3 --pmc GRBM_GUI_ACTIVE -f csv -d <grbm_dir> -- python bench.py "
                    f"--workload {workload} --steps 2 --no-cpu-baseline\n")
            f.write(f"#   rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES -f csv -d <mfma_dir> -- "
                    f"python bench.py --workload {workload} --steps 2 --no-cpu-baseline\n")
            f.write(f"#   python bench.py --workload {workload} --summarize-busy <grbm_dir> <mfma_dir> <this file>\n")
        f.write(f"# cycles = GRBM_GUI_ACTIVE / {XCDS} XCDs; clock = cycles / dispatch duration;\n")
        f.write(f"# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / {SIMDS} SIMDs, as a share of the cycles.\n")
        f.write("# The counter window is a little longer than the dispatch, so kernels shorter than\n"
                "# about 0.1 ms read a clock above the real one; the long kernels are not affected.\n")
        f.write("kernel | dispatches | avg us | clock GHz (min-max) | cycles | MFMA busy cycles per SIMD | busy share\n")
        for name, v in sorted(grbm.items(), key=lambda kv: -sum(d for _, d in kv[1])):
            if "attn::" not in name and "mfma_rate_kernel" not in name:
                continue
            dur = sum(d for _, d in v) / len(v)
            cyc = sum(c for c, _ in v) / len(v) / XCDS
            clk = [c / XCDS / d for c, d in v]
            line = f"{name.split('(')[0]} | {len(v)} | {dur / 1e3:.1f} | {sum(clk) / len(clk):.3f} ({min(clk):.3f}-{max(clk):.3f}) | {cyc:.0f}"
            m = mfma.get(name)
            if m:
                mb = sum(c for c, _ in m) / len(m) / SIMDS
                line += f" | {mb:.0f} | {mb / cyc:.3f}"
            f.write(line + "\n")
    print(out)


WAVE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY",
                 "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
                 "SQ_VALU_MFMA_COEXEC_CYCLES")


def summarize_counters(pmc_dir, out, workload):
    """Per-dispatch averages of every counter a rocprofv3 --pmc run collected,
    for the attention kernels, with the command that collects them."""
    import csv
    import glob

    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if "attn::" in r["Kernel_Name"]:
                acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    names = sorted({c for v in acc.values() for c in v})
    with open(out, "w") as f:
        f.write(f"# Counters of the attention kernels on {workload}, per dispatch (rocprofv3).\n")
        f.write("# Commands (run from the repository root on the MI355X box):\n")
        f.write(f"#   rocprofv3 --pmc {' '.join(names)} -f csv -d <pmc_dir> -- python bench.py "
                f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline\n")
        f.write(f"#   python bench.py --workload {workload} --summarize-counters <pmc_dir> <this file>\n")
        f.write("# Values are summed over the chip by rocprofv3; SQ_INSTS_* count instructions,\n"
                "# SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE count LDS cycles.\n")
        f.write("kernel | " + " | ".join(names) + "\n")
        for name, c in sorted(acc.items()):
            f.write(name.split("(")[0] + " | " + " | ".join(
                f"{sum(c[n]) / len(c[n]):.4g}" if n in c else "-" for n in names) + "\n")
    print(out)


def summarize_waves(pmc_dir, out, workload):
    """Where the waves of each attention kernel spend their time, from one
    rocprofv3 --pmc run with the SQ wave-state counters (all summed over the
    waves, in units of 4 cycles): issuing an instruction (ACTIVE_INST_ANY),
    holding a ready instruction that is not issued yet (WAIT_INST_ANY: the
    unit it needs is busy, e.g. the matrix core), and waiting on a counter
    or barrier (WAIT_ANY: LDS or memory results, s_barrier). The three add
    up to SQ_WAVE_CYCLES, which the summary checks."""
    import csv
    import glob

    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if "attn::" in r["Kernel_Name"] and r["Counter_Name"] in WAVE_COUNTERS:
                acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    with open(out, "w") as f:
        f.write(f"# Wave time of each kernel on {workload}, from rocprofv3 SQ counters.\n")
        f.write("# Commands (run from the repository root on the MI355X box):\n")
        f.write(f"#   rocprofv3 --pmc {' '.join(WAVE_COUNTERS)} -f csv -d <pmc_dir> -- python bench.py "
                f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline\n")
        f.write(f"#   python bench.py --workload {workload} --summarize-waves <pmc_dir> <this file>\n")
        f.write("# Shares of SQ_WAVE_CYCLES: issuing = ACTIVE_INST_ANY, ready-not-issued = WAIT_INST_ANY,\n"
                "# waiting on counters/barrier = WAIT_ANY; the VALU (matrix products included) and LDS\n"
                "# issue shares are parts of 'issuing'.\n")
        f.write("kernel | issuing | ready, not issued | waiting on counters/barrier | sum | VALU issue | LDS issue\n")
        for name, c in sorted(acc.items()):
            avg = {k: sum(v) / len(v) for k, v in c.items()}
            wc = avg["SQ_WAVE_CYCLES"]
            a, wi, wa = avg["SQ_ACTIVE_INST_ANY"] / wc, avg["SQ_WAIT_INST_ANY"] / wc, avg["SQ_WAIT_ANY"] / wc
            f.write(f"{name.split('(')[0]} | {a:.3f} | {wi:.3f} | {wa:.3f} | {a + wi + wa:.3f} | "
                    f"{avg['SQ_ACTIVE_INST_VALU'] / wc:.3f} | {avg['SQ_ACTIVE_INST_LDS'] / wc:.3f}\n")
    print(out)


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def cpu_model():
    """The host CPU's model name (Linux), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def mfma_ceiling(steps):
    """TFLOP/s of attn_probe_mfma_rate and attn_probe_mfma16_rate (independent
    v_mfma_f32_32x32x16_bf16 or v_mfma_f32_16x16x32_bf16 products, two waves
    per SIMD, no other work) on operands drawn like the
    workloads' inputs (N(0,1) rounded to bf16) and on all-zero operands: the
    matrix-core rate the chip sustains under its power management for each
    operand pattern, which bounds every attention kernel's MFMA throughput."""
    import torch

    import exact_attention_12_amd as ea
    blocks, iters = 1024, 1024
    n = ea.probe_mfma_src_elems(blocks)
    g = torch.Generator(device="cpu")
    g.manual_seed(4242)
    out = {}
    stream = torch.cuda.current_stream()
    for name, src in (("random", torch.randn(n, generator=g).to(torch.bfloat16).cuda()),
                      ("zeros", torch.zeros(n, dtype=torch.bfloat16, device="cuda"))):
        dst = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
        for shape, tag in (("32x32x16", ""), ("16x16x32", "m16_")):
            for chains in (1, 2, 4, 8):
                run = lambda: ea.probe_mfma_rate(src, dst, blocks, iters, chains, shape)  # noqa: E731
                flops = run()  # warm-up
                ms = time_loop(run, steps, stream)
                out[f"{tag}{name}_chains{chains}"] = {
                    "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                    "pct_of_bf16_peak": round(100.0 * flops / ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
    line = {"probe": "mfma_ceiling", "op": "v_mfma_f32_32x32x16_bf16 (keys m16_*: v_mfma_f32_16x16x32_bf16)",
            "waves_per_simd": 2, "flops_per_call": blocks * 8 * 8 * iters * 32768.0, "steps": steps, **out}
    print(json.dumps(line), flush=True)


def warm_up(launches, steps):
    """Run the step's launches untimed: `steps` times if given, else at least
    WARMUP_MIN_STEPS times and until WARMUP_SECONDS have passed. Returns the
    number of warm-up steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while True:
        if steps is not None and n >= steps:
            break
        for f in launches:
            f()
        n += 1
        if steps is None and n >= WARMUP_MIN_STEPS and n % WARMUP_MIN_STEPS == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARMUP_SECONDS:
                break
    torch.cuda.synchronize()
    return n


def time_loop(fn, steps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms


def cold_time(fn, steps, stream, scratch_mib=512):
    """Average time of fn when the caches start cold: before each call a
    scratch buffer larger than L2 and the 256 MB MALL is overwritten (not
    timed); each call is bracketed by its own events."""
    import torch
    scratch = torch.empty(scratch_mib * (1 << 18), dtype=torch.float32, device="cuda")
    total = 0.0
    for _ in range(steps):
        scratch.fill_(1.0)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        fn()
        end.record(stream)
        torch.cuda.synchronize()
        total += start.elapsed_time(end)
    del scratch
    return total / steps  # ms


def unfused_baseline(w, g, o_fused, steps, stream, fused_ms):
    """Standard attention as the pages write it ([CANN-FA] standard attention
    code; [FA-seqlen] times it against FlashAttention by sequence length), in
    torch eager bf16 on the same GPU: S = Q K^T * scale, P = softmax(S),
    O = P V, with S and P materialised in HBM (B*H*N^2 16-bit values each).
    Timed over the same number of steps as the fused forward; only for
    unmasked multi-head forward workloads. The right operand of each batched
    product is contiguous."""
    import torch
    q, k, v = g["q"], g["k"], g["v"]
    kt = k.transpose(-1, -2).contiguous()

    def run():
        s = torch.matmul(q, kt) * w.scale
        return torch.matmul(torch.softmax(s, dim=-1), v), s

    o_ref, s = run()
    torch.cuda.synchronize()
    sp = si.score_matrix_bytes(w.B, w.Hq, w.N, 2)
    assert s.numel() * s.element_size() == sp, "S is not B*H*N^2 16-bit values"
    del s
    o_err = float((o_ref.float() - o_fused.float()).abs().max())
    ms = time_loop(lambda: run(), steps, stream)
    return {"ms": round(ms, 4), "tflops": round(w.fwd_flops() / ms / 1e9, 2),
            "s_and_p_bytes": 2 * sp, "fused_speedup": round(ms / fused_ms, 3),
            "o_max_abs_diff_vs_fused": round(o_err, 5)}


def cpu_baseline(w, inputs, budget_s):
    """Time the fp64 oracle on whole heads of the same workload (rank 0 only).

    Heads (b, h) are taken in order, each with its KV head, until about
    `budget_s` seconds of CPU work have been spent (at least one head).
    """
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    heads, secs = 0, 0.0
    for b in range(w.B):
        for h in range(w.Hq):
            hk = h // w.G
            q = si.to_f64(inputs["q"][b:b + 1, h:h + 1])
            k = si.to_f64(inputs["k"][b:b + 1, hk:hk + 1])
            v = si.to_f64(inputs["v"][b:b + 1, hk:hk + 1])
            t0 = time.perf_counter()
            # one-head arrays: the dropout stream of head (b, h) is head 0 of
            # a stream whose seed is unchanged, so the timing leg uses the
            # same amount of work, not the same mask
            if w.Nq is not None:
                oracle.ref_decode(q, k, v, w.scale, w.causal, window=w.window)
            else:
                oracle.ref_fwd(q, k, v, w.scale, w.causal, window=w.window, dropout=w.dropout)
            if w.backward:
                do = si.to_f64(inputs["do"][b:b + 1, h:h + 1])
                oracle.ref_bwd(q, k, v, do, w.scale, w.causal, window=w.window, dropout=w.dropout)
            secs += time.perf_counter() - t0
            heads += 1
            if secs * (heads + 1) / heads > budget_s:
                break
        else:
            continue
        break
    per_head = (w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)) / (w.B * w.Hq)
    value = per_head * heads / secs / 1e12
    return {
        "value": round(value, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "host_usable_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{heads} of {w.B * w.Hq} heads of the same workload "
                   f"({'Nq=' + str(w.Nq) + ' against a cache of ' if w.Nq else ''}N={w.N}, d={w.d}, "
                   f"{w.mask}, {'fwd+bwd' if w.backward else 'fwd'}), "
                   f"numpy float64 with S and P materialised, {secs:.1f} s; value credits the "
                   f"same algorithmic flops per head as the GPU line"),
        "seconds": round(secs, 2),
    }


def parity_sample(w, inputs, o, lse):
    """O and LSE error of sampled rows of the timed run against the oracle."""
    import numpy as np

    import oracle
    from oracle import philox
    b, h = w.B - 1, w.Hq - 1
    hk = h // w.G
    if w.Nq is not None:  # decoding: every query head of the last sequence
        O, L = oracle.ref_decode(si.to_f64(inputs["q"][b:b + 1]), si.to_f64(inputs["k"][b:b + 1]),
                                 si.to_f64(inputs["v"][b:b + 1]), w.scale, w.causal, window=w.window)
        eo = float(np.abs(si.to_f64(o[b]) - O[0]).max())
        el = float(np.abs(lse[b].double().cpu().numpy() - L[0]).max())
        return {"sequence": int(b), "rows": int(w.Hq * w.Nq), "o_max_abs_err": eo, "lse_max_abs_err": el}
    rows = np.unique(np.linspace(0, w.N - 1, 48).astype(int))
    q = si.to_f64(inputs["q"][b, h])
    k = si.to_f64(inputs["k"][b, hk])
    v = si.to_f64(inputs["v"][b, hk])
    og = si.to_f64(o[b, h])
    lg = lse[b, h].double().cpu().numpy()
    eo, el = 0.0, 0.0
    for r in rows:
        keep, p = None, 0.0
        if w.dropout is not None:
            keep = philox.dropout_keep(b * w.Hq + h, [int(r)], np.arange(w.N), *w.dropout)
            p = w.dropout[0]
        O, L = oracle.ref_fwd_head(q[r:r + 1], k, v, w.scale, w.causal, row0=int(r), window=w.window,
                                   keep=keep, p_drop=p)
        eo = max(eo, float(np.abs(og[r] - O[0]).max()))
        el = max(el, float(abs(lg[r] - L[0])))
    return {"head": [int(b), int(h)], "rows": int(len(rows)), "o_max_abs_err": eo, "lse_max_abs_err": el}


def summarize_trace(trace_dir, bench_json, out_md, workload):
    """Markdown table of a kernel-trace stats CSV next to the bench's own
    HIP-event timings of the same build."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    w = si.WORKLOADS[workload]
    b = json.loads(open(bench_json).read().strip().splitlines()[-1])
    out = [f"# Kernel trace: {workload} (B={w.B}, Hq={w.Hq}, Hkv={w.Hkv}, N={w.N}, d={w.d}, "
           f"{w.mask}, {'fwd+bwd' if w.backward else 'fwd'})", "",
           "Commands (repository root on the MI355X box):", "",
           f"    cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d <trace_dir> -o trace -- "
           f"python <repo>/bench.py --workload {workload} --steps 20 --no-cpu-baseline",
           f"    python bench.py --workload {workload} > <bench_json>",
           f"    python bench.py --workload {workload} --summarize-trace <trace_dir> <bench_json> <this file>",
           "", "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(files[0])):
        name = r["Name"]
        short = name.split("(")[0].replace("void ", "")
        if CALIBRATION_KERNEL in name:
            short = "calibration copy (torch neg, float32)"
        elif "attn::" not in name:
            short = short[:60]
        out.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    out += ["", f"HIP-event timings of the same build (bench run, {b['steps']} timed steps):", "",
            "| kernel | avg ms | median ms | min ms | credited TFLOP/s | % of 2.5 PFLOP/s | GB/s (algorithmic bytes) |",
            "|---|---|---|---|---|---|---|"]
    for name, v in b["kernels"].items():
        gbs = f"{v['bytes'] / v['ms'] / 1e6:.0f}" if v.get("bytes") else "-"
        out.append(f"| {name} | {v['ms']} | {v.get('ms_median', '-')} | {v.get('ms_min', '-')} | "
                   f"{v['tflops']} | {v['pct_of_bf16_peak']} | {gbs} |")
    out += ["", f"Step: {b['ms_per_step']} ms mean (median {b.get('ms_per_step_median', '-')}, min "
                f"{b.get('ms_per_step_min', '-')}) = {b['value']} TFLOP/s algorithmic "
                f"({b['pct_of_bf16_peak']}% of the bf16 peak); roofline kernel "
                f"{b['roofline']['kernel']} at {b['roofline']['achieved']} {b['roofline']['unit']} "
                f"(frac {b['roofline']['frac']})."]
    if b.get("cold_cache"):
        c = b["cold_cache"]
        out += ["", f"Cold caches ({c['scratch_mib']} MiB scratch overwritten before each call, each "
                    f"call bracketed by its own events): forward {c['fwd_ms']} ms."]
    if b.get("unfused_baseline"):
        u = b["unfused_baseline"]
        out += ["", f"Unfused torch eager baseline (S = Q K^T * scale, softmax, P V; S and P "
                    f"materialised, {u['s_and_p_bytes'] / 2**20:.0f} MiB): {u['ms']} ms = {u['tflops']} "
                    f"TFLOP/s; the fused forward is {u['fused_speedup']}x faster; outputs differ by at "
                    f"most {u['o_max_abs_diff_vs_fused']}."]
    if b.get("cpu_baseline"):
        c = b["cpu_baseline"]
        out += ["", f"CPU oracle: {c['value']} TFLOP/s on {c['cores']} threads ({c.get('cpu_model', '?')}); "
                    f"sample: {c['sample']}."]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print(out_md)


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.workload)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload)
        return
    if args.summarize_waves:
        summarize_waves(*args.summarize_waves, args.workload)
        return
    if args.summarize_busy:
        summarize_busy(*args.summarize_busy, args.workload)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.workload, args.calibration_copy_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported. Attention shards by (batch, KV-head group) with no exchange; run one "
              "process per GPU instead.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_12_amd as ea
    if not os.path.exists(ea.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mfma_ceiling:
        mfma_ceiling(args.steps)
        return

    w = si.WORKLOADS[args.workload]
    inputs = si.workload_inputs(w)
    g = {key: si.in_layout(t.cuda(), w.layout) for key, t in inputs.items()}
    stream = torch.cuda.current_stream()
    o = torch.empty_like(g["q"])
    rows_per_head = w.Nq if w.Nq is not None else w.N
    lse = torch.empty((w.B, w.Hq, rows_per_head), dtype=torch.float32, device="cuda")
    if w.Nq is not None:
        dws_bytes = ea.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.N, w.d, w.causal, w.window,
                                              ea.DTYPE_FP16 if w.dtype == "fp16" else ea.DTYPE_BF16)
        dws = torch.empty(max(dws_bytes, 256), dtype=torch.uint8, device="cuda")
    if w.backward:
        dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
        ws = torch.empty(ea.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8,
                         device="cuda")

    drop_kw = {}
    if w.dropout is not None:
        drop_kw = dict(dropout_p=w.dropout[0], seed=w.dropout[1], offset=w.dropout[2])

    def run_fwd():
        if w.Nq is not None:
            ea.decode(g["q"], g["k"], g["v"], scale=w.scale, causal=w.causal, window=w.window,
                      layout=w.layout, out=o, lse=lse, workspace=dws)
            return
        ea.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=w.causal, window=w.window,
               layout=w.layout, out=o, lse=lse, **drop_kw)

    def run_bwd():
        ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=w.scale, causal=w.causal,
               window=w.window, layout=w.layout, workspace=ws, dq=dq, dk=dk, dv=dv, **drop_kw)

    def bwd_pass(name):
        return lambda: ea.bwd_passes(g["q"], g["k"], g["v"], o, lse, g["do"], dq, dk, dv, ws,
                                     scale=w.scale, causal=w.causal, window=w.window,
                                     layout=w.layout, passes=(name,), **drop_kw)

    # One step = the forward, then the backward's three passes through their
    # own entry points (the kernels attn_bwd launches, in its order). A HIP
    # event on the launch stream sits between consecutive kernels, so the
    # timed steps also give each kernel's average launch duration.
    names, launches = [DECODE_UNIT if w.Nq is not None else "fwd_kernel"], [run_fwd]
    if w.backward:
        names += ["bwd_pre_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"]
        launches += [bwd_pass("pre"), bwd_pass("dkdv"), bwd_pass("dq")]

    warmup = warm_up(launches, args.warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ev in ev:
        s_ev[0].record(stream)
        for i, f in enumerate(launches):
            f()
            s_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev[0][0].elapsed_time(ev[-1][-1]) / args.steps
    step_ms = sorted(s_ev[0].elapsed_time(s_ev[-1]) for s_ev in ev)
    print(f"[bench] {args.steps} steps of {w.name}: {ms_step:.3f} ms/step (wall {wall:.2f} s)",
          file=sys.stderr, flush=True)

    credit = kernel_flop_credit(w)
    rows = w.B * w.Hq * w.N
    work = {"fwd_kernel": (credit["fwd"], w.fwd_bytes()),
            DECODE_UNIT: (credit["fwd"], w.fwd_bytes()),
            "bwd_pre_kernel": (0.0, 2 * rows * w.d * 2 + 12 * rows),  # O, dO, LSE in; -D, LSE2 out
            "bwd_dkdv_kernel": (credit["bwd_dkdv"], None),
            "bwd_dq_kernel": (credit["bwd_dq"], None)}
    kernels = {}
    for i, name in enumerate(names):
        per_step = sorted(s_ev[i].elapsed_time(s_ev[i + 1]) for s_ev in ev)
        ms = sum(per_step) / args.steps
        flops, nbytes = work[name]
        kernels[name] = {"ms": ms, "flops": flops, "ms_median": round(median(per_step), 4),
                         "ms_min": round(per_step[0], 4)}
        if nbytes is not None:
            kernels[name]["bytes"] = nbytes
    for k in kernels.values():
        k["tflops"] = round(k["flops"] / k["ms"] / 1e9, 2)
        k["pct_of_bf16_peak"] = round(100.0 * k["tflops"] / PEAK_BF16_TFLOPS, 2)
        k["ms"] = round(k["ms"], 4)
    print(f"[bench] kernels: {kernels}", file=sys.stderr, flush=True)
    passes = {"fwd": {"ms": kernels[names[0]]["ms"], "tflops": kernels[names[0]]["tflops"],
                      "pct_of_bf16_peak": kernels[names[0]]["pct_of_bf16_peak"]}}
    if w.backward:
        ms_bwd = sum(kernels[n]["ms"] for n in names[1:])
        tf = w.bwd_flops() / ms_bwd / 1e9
        passes["bwd"] = {"ms": round(ms_bwd, 4), "tflops": round(tf, 2),
                         "pct_of_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2)}
        # The fused attn_bwd call (same kernels, no events between them).
        passes["bwd"]["fused_call_ms"] = round(time_loop(run_bwd, args.steps, stream), 4)

    step_flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)
    value = step_flops / (ms_step * 1e-3) / 1e12

    # Roofline of the kernel that takes the most time per step.
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm_bound = dom == "bwd_pre_kernel" or (dom in ("fwd_kernel", DECODE_UNIT) and
                                             w.fwd_flops() / w.fwd_bytes() < ridge)
    if hbm_bound:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(kd["bytes"] / kd["ms"] / 1e6, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"kernel": dom, "bound": "mfma", "achieved": kd["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["avg_launch_ms"] = kd["ms"]
    roof["traffic"] = read_traffic(dom, w.name)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    run_fwd()
    torch.cuda.synchronize()
    par = parity_sample(w, inputs, o.transpose(1, 2) if w.layout == "bshd" else o, lse)
    print(f"[bench] parity sample: {par}", file=sys.stderr, flush=True)

    cold = None
    if not w.backward and w.Nq is None and w.N <= 1024:
        cold = {"fwd_ms": round(cold_time(run_fwd, args.steps, stream), 4), "scratch_mib": 512}
        print(f"[bench] cold-cache forward: {cold}", file=sys.stderr, flush=True)

    unfused = None
    if (not w.backward and not w.causal and w.window is None and w.Nq is None and w.dropout is None
            and w.Hq == w.Hkv and w.layout == "bhsd"):
        unfused = unfused_baseline(w, g, o, args.steps, stream, kernels[names[0]]["ms"])
        print(f"[bench] unfused torch baseline: {unfused}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inputs, args.cpu_seconds)
        print(f"[bench] cpu baseline: {cpu}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(median(step_ms), 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "window": w.window, "layout": w.layout, "Nq": w.Nq,
                   "dropout_p": w.dropout_p,
                   "passes": "fwd+bwd" if w.backward else "fwd",
                   "seed": w.seed, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "passes": passes,
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_sample": par,
    }
    if cold is not None:
        line["cold_cache"] = cold
    if unfused is not None:
        line["unfused_baseline"] = unfused
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
