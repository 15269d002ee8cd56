"""Throughput of the fused attention path on one MI355X, next to the CPU oracle.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward (O and LSE) and the recompute backward (row-term preprocess,
dK/dV pass, dQ pass) for the fwd+bwd workload; the forward alone for the
forward-only workloads. Inputs are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line. `value` is algorithmic TFLOP/s of a step (4*d flops per
allowed (query, key) pair forward, 2.5x that backward; masked pairs and the
backward's recomputed products are not credited).
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(si.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="rough CPU budget for the oracle leg (it times whole heads)")
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
            oracle.ref_fwd(q, k, v, w.scale, w.causal)
            if w.backward:
                do = si.to_f64(inputs["do"][b:b + 1, h:h + 1])
                oracle.ref_bwd(q, k, v, do, w.scale, w.causal)
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
        "kind": "oracle",
        "sample": (f"{heads} of {w.B * w.Hq} heads of the same workload (N={w.N}, d={w.d}, "
                   f"{'causal' if w.causal else 'no mask'}, {'fwd+bwd' if w.backward else 'fwd'}), "
                   f"numpy float64 with S and P materialised, {secs:.1f} s; value credits the "
                   f"same algorithmic flops per head as the GPU line"),
        "seconds": round(secs, 2),
    }


def parity_sample(w, inputs, o, lse):
    """O and LSE error of sampled rows of the timed run against the oracle."""
    import numpy as np

    import oracle
    b, h = w.B - 1, w.Hq - 1
    hk = h // w.G
    rows = np.unique(np.linspace(0, w.N - 1, 48).astype(int))
    q = si.to_f64(inputs["q"][b, h])
    k = si.to_f64(inputs["k"][b, hk])
    v = si.to_f64(inputs["v"][b, hk])
    og = si.to_f64(o[b, h])
    lg = lse[b, h].double().cpu().numpy()
    eo, el = 0.0, 0.0
    for r in rows:
        O, L = oracle.ref_fwd_head(q[r:r + 1], k, v, w.scale, w.causal, row0=int(r))
        eo = max(eo, float(np.abs(og[r] - O[0]).max()))
        el = max(el, float(abs(lg[r] - L[0])))
    return {"head": [int(b), int(h)], "rows": int(len(rows)), "o_max_abs_err": eo, "lse_max_abs_err": el}


def main():
    args = parse()
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

    w = si.WORKLOADS[args.workload]
    inputs = si.workload_inputs(w)
    g = {key: t.cuda() for key, t in inputs.items()}
    stream = torch.cuda.current_stream()
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    if w.backward:
        dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
        ws = torch.empty(ea.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8,
                         device="cuda")

    def run_fwd():
        ea.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=w.causal, out=o, lse=lse)

    def run_bwd():
        ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=w.scale, causal=w.causal,
               workspace=ws, dq=dq, dk=dk, dv=dv)

    def step():
        run_fwd()
        if w.backward:
            run_bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = time_loop(step, args.steps, stream)
    wall = time.perf_counter() - t0
    print(f"[bench] {args.steps} steps of {w.name}: {ms_step:.3f} ms/step (wall {wall:.2f} s)",
          file=sys.stderr, flush=True)

    # Per-pass timings (same stream, HIP events) for the roofline and the breakdown.
    credit = kernel_flop_credit(w)
    ms_fwd = time_loop(run_fwd, args.steps, stream)
    passes = {"fwd": {"ms": ms_fwd, "tflops": credit["fwd"] / ms_fwd / 1e9}}
    if w.backward:
        ms_bwd = time_loop(run_bwd, args.steps, stream)
        passes["bwd"] = {"ms": ms_bwd, "tflops": w.bwd_flops() / ms_bwd / 1e9}
    for p in passes.values():
        p["pct_of_bf16_peak"] = 100.0 * p["tflops"] / PEAK_BF16_TFLOPS
        p["ms"] = round(p["ms"], 4)
        p["tflops"] = round(p["tflops"], 2)
        p["pct_of_bf16_peak"] = round(p["pct_of_bf16_peak"], 2)
    print(f"[bench] passes: {passes}", file=sys.stderr, flush=True)

    step_flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0.0)
    value = step_flops / (ms_step * 1e-3) / 1e12

    # Roofline of the forward kernel (one kernel per attn_fwd call, timed with
    # HIP events on the stream it runs on).
    if w.fwd_flops() / w.fwd_bytes() >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"kernel": "fwd_kernel", "bound": "mfma", "achieved": round(credit["fwd"] / ms_fwd / 1e9, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": "fwd_kernel", "bound": "hbm", "achieved": round(w.fwd_bytes() / ms_fwd / 1e6, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None

    run_fwd()
    torch.cuda.synchronize()
    par = parity_sample(w, inputs, o, lse)
    print(f"[bench] parity sample: {par}", file=sys.stderr, flush=True)

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
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "passes": "fwd+bwd" if w.backward else "fwd",
                   "seed": w.seed, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "passes": passes,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_sample": par,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
