#!/usr/bin/env python3
"""Throughput of the fused GEMM-epilogue path on one MI355X.

One step = one ``gemm_epilogue_run`` (a single fused kernel launch) over the
workload's seeded synthetic inputs, already resident in HBM.  The default
workload is the batched one (batch 16 x 1024^3, alpha 1.25, column bias, ReLU,
AMAX over all outputs, bf16 output); ``--config c1..c5`` selects another.

Prints ONE JSON line:
  value      whole-job TFLOP/s = 2*M*N*K*batch (x2 pairwise) / (timed wall time / steps)
  roofline   the fused kernel's achieved TFLOP/s from per-launch HIP events on its
             stream, against the MI355X dense bf16 MFMA peak (2.5 PFLOP/s)
  cpu_baseline  the float64 oracle on this host's cores over a bounded sample
  epilogue_overhead_pct  fused kernel time over the same kernel instance with the
             chain reduced to a plain bf16 store (pairwise: the bare product g*u)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "fused GEMM-epilogue TFLOP/s (% of MI355X bf16 MFMA peak) per config"

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of this kernel at this workload,
# scaled by the copy-kernel calibration factor; None until counters are taken for the current kernel.
MEASURED_TRAFFIC = {}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle timing sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bare", action="store_true", help="skip the bare-GEMM comparison")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark: run a plain device copy of MIB MiB ten times (the "
                         "reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n * 4, "copy_bytes_written_per_launch": n * 4, "launches": 10}))


def time_launches(prob, steps, warmup):
    """(ms per step over the bracketed region, mean per-launch ms from event pairs)."""
    import torch

    for _ in range(warmup):
        prob.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    region0.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        prob.run(stream.cuda_stream)
        ends[i].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    total_ms = region0.elapsed_time(region1)
    per_launch = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    per_launch.sort()
    mean_ms = sum(per_launch) / len(per_launch)
    return total_ms / steps, mean_ms, per_launch[len(per_launch) // 2]


def bare_chain(w):
    return (("pairwise", "none"),) if w.pairwise else ()


def cpu_baseline(w, inputs, seconds):
    """The oracle as it stands, on this host's cores, over a bounded sample of the workload."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    # sample: whole batches for the batched workload, else a block of rows (all columns, full K)
    if w.batch > 1:
        sample_desc = "1 of %d batches (M=N=K=%d), repeated" % (w.batch, w.M)
        sub = {k: (v[:1] if k in ("A", "B", "B2", "R") else v) for k, v in inputs.items()}
        w_s = w.with_shape(batch=1)
        rows = None
    else:
        nrows = min(w.M, max(64, int(256 * 4096 * 4096 / max(1, w.N * w.K))))
        rows = np.arange(nrows)
        sample_desc = "rows 0..%d of %d (all %d columns, K=%d), repeated" % (nrows - 1, w.M, w.N, w.K)
        sub, w_s = inputs, w.with_shape(M=nrows)
    flops_per = w_s.flops()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run_workload(w_s if rows is None else w, sub, rows=rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": round(flops_per * reps / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "sample": sample_desc + f" x{reps} in {el:.1f} s (float64 GEMM + unfused epilogue + encode)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the fused GEMM-epilogue path has no multi-GPU leg "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import workloads
    from gemm_epilogue_transformer_tiled_amd import runner

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = workloads.WORKLOADS[args.config]
    inputs = workloads.generate(w)
    prob = runner.prepare(w, inputs)
    ms_step, launch_ms, launch_med = time_launches(prob, args.steps, args.warmup)
    flops = w.flops()
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "batch": w.batch, "M": w.M, "N": w.N, "K": w.K,
            "chain": [list(op) for op in w.chain],
            "output": w.out,
            "kernel": prob.plan.describe(),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": MEASURED_TRAFFIC.get(w.name),
            "kernel": "fused_gemm_epilogue",
            "launch_ms_mean": round(launch_ms, 6),
            "launch_ms_median": round(launch_med, 6),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes(),
            "hbm_gbs_at_algorithmic_bytes": round(w.algorithmic_bytes() / (launch_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(w.algorithmic_bytes() / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        },
    }
    if not args.no_bare:
        wb = w.__class__(**{**w.__dict__, "chain": bare_chain(w), "out": "bf16", "name": w.name + "-bare"})
        bare = runner.prepare(wb, inputs)
        _, bare_ms, _ = time_launches(bare, args.steps, args.warmup)
        result["bare_gemm_ms"] = round(bare_ms, 6)
        result["epilogue_overhead_pct"] = round((launch_ms / bare_ms - 1.0) * 100.0, 2)
        del bare
    del prob
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
