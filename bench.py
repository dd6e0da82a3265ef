#!/usr/bin/env python3
"""Throughput of the fused GEMM-epilogue path on one MI355X.

One step = one ``gemm_epilogue_run`` (a single fused kernel launch) over a
workload's seeded synthetic inputs, already resident in HBM.

Without ``--config`` the benchmark runs the whole suite: the SwiGLU
up-projection c3 (8192x4096 -> 2x11008, the largest configuration, and the
headline), then c1, c2, c4, c5 and the three further workloads f1 (RMSNorm-MLP),
f2 (MLP backward) and f3 (fp8 operands).  Each configuration runs in a child
process of its own (``--config X``); this parent process never touches the GPU.
A configuration that fails is recorded with its status and the suite carries
on; one that ends abnormally (a signal, an abort, a time limit) stops the suite,
and the remaining configurations are recorded as skipped.

The K timed steps run back to back on one stream, issued either eagerly or as one
replay of a HIP graph holding the K launches (``--launch``; by default the faster
on an untimed probe, named in the output).

Prints ONE JSON line (the headline configuration's fields, plus ``per_config``):
  value      whole-job TFLOP/s = 2*M*N*K*batch (x2 pairwise) / (timed wall time / steps)
  roofline   the fused kernel's achieved rate over its average launch duration (HIP
             events on its stream around the back-to-back steps) against the MI355X peak
             of its bound: dense bf16 MFMA 2.5 PFLOP/s (fp8 operands: 5.0) when the
             workload's ideal time at that peak exceeds its ideal time at 8 TB/s of HBM,
             else HBM; traffic = HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE
             counters, when they were taken on this kernel source
  cpu_baseline  the float64 oracle on this host's cores over a bounded sample
  epilogue_overhead_pct  fused kernel time over the same kernel instance with the
             chain reduced to a plain bf16 store (pairwise: the bare product g*u)
  cold       median single launch with L2/MALL flushed before each launch
  unfused    the same chain run unfused (GEMM writes bf16 C, one kernel per operation):
             its time, kernels and algorithmic HBM bytes, and the bytes the fusion saves
  measured_peaks  what the MFMA (three instruction forms), streaming-copy, L2->LDS and
             LDS-read probes sustain on this GPU; roofline.frac_of_measured_mfma_peak is
             achieved over the probe of the instruction the mainloop runs
  per_config  for every configuration of the suite: status, TFLOP/s, GB/s, roofline
             fractions, epilogue overhead, unfused bytes saved and a short oracle baseline
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
GRAPH_PROBE_BELOW_MS = 0.1     # eager steps at least this long are not probed as a graph
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published (the fp8-operand workload)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "fused GEMM-epilogue TFLOP/s (% of MI355X bf16 MFMA peak) per config"
# The suite, headline first: c3 is the largest configuration (1.48 TFLOP per step).
SUITE = ["c3", "c1", "c2", "c4", "c5", "f1", "f2", "f3"]
# Exit statuses of a child that ended abnormally (signal, abort, segmentation fault, time
# limit): after one of these nothing more is started on the GPU.
ABNORMAL_RC = {-6, -9, -11, -15, 124, 134, 137, 139}

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE (x2.0) + WRITE_SIZE (x1.0) of the fused
# kernel at each workload; the factors scale the counters to the bytes of a plain 1 GiB device
# copy.  Valid only for the device code they were taken on (sha256 prefix of the library's
# .hip_fatbin section, below): any change to any kernel instance changes it.
MEASURED_TRAFFIC_CODE = "04daa6e50266fff0"
MEASURED_TRAFFIC = {"c1": 1066177, "c2": 101051631, "c3": 2402031871, "c4": 537792963, "c5": 1695033449,
                    "f1": 2391858012, "f2": 1852936119, "f3": 877316544}


def kernel_code_hash(lib_path=None):
    """sha256 prefix of the device code in libgemm_epilogue.so (its .hip_fatbin ELF section)."""
    import struct
    path = lib_path or os.path.join(ROOT, "gemm_epilogue_transformer_tiled_amd", "libgemm_epilogue.so")
    with open(path, "rb") as f:
        data = f.read()
    if data[:4] != b"\x7fELF" or data[4] != 2:
        raise ValueError(f"{path}: not a 64-bit ELF file")
    e_shoff, = struct.unpack_from("<Q", data, 0x28)
    e_shentsize, e_shnum, e_shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    def section(i):
        name, _type, _flags, _addr, off, size = struct.unpack_from("<IIQQQQ", data, e_shoff + i * e_shentsize)
        return name, off, size
    _, str_off, _ = section(e_shstrndx)
    for i in range(e_shnum):
        name, off, size = section(i)
        end = data.index(b"\0", str_off + name)
        if data[str_off + name:end] == b".hip_fatbin":
            return hashlib.sha256(data[off:off + size]).hexdigest()[:16]
    raise ValueError(f"{path}: no .hip_fatbin section")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None, choices=SUITE,
                    help="run one workload in this process (default: the whole suite, each configuration in "
                         "a child process).  c1..c5: the five configurations; f1: the RMSNorm-MLP (row RMS + "
                         "pairwise product); f2: the MLP backward step (activation gradient + column sums, B as "
                         "[N][K]); f3: fp8-e4m3 operands (delayed scaling) into the c5 epilogue")
    ap.add_argument("--suite", default=",".join(SUITE),
                    help="comma-separated configurations of the suite, the headline first")
    ap.add_argument("--suite-cpu-seconds", type=float, default=2.5,
                    help="oracle sample budget of each non-headline configuration of the suite")
    ap.add_argument("--child-timeout", type=float, default=300.0,
                    help="seconds one configuration of the suite may take before it is stopped")
    ap.add_argument("--launch", default="auto", choices=["auto", "eager", "graph"],
                    help="issue the timed steps eagerly or as one HIP-graph replay (auto: the faster on a probe)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle timing sample")
    ap.add_argument("--tile-cache", default=None, metavar="JSON",
                    help="tile-config cache: plan the workload with the instance it holds (and, with --tune, "
                         "record the sweep there)")
    ap.add_argument("--tune", action="store_true",
                    help="time every admissible kernel instance on the workload first (untimed), then run "
                         "the fastest")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bare", action="store_true", help="skip the bare-GEMM comparison")
    ap.add_argument("--breakdown", action="store_true",
                    help="also time the chain with each epilogue op left out, in turn (per-op cost)")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the workload's bare GEMM through torch.matmul (hipBLASLt), same layout")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache single-launch timing")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused-sequence comparison")
    ap.add_argument("--no-probes", action="store_true", help="skip the MFMA / copy calibration probes")
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


def _region_ms(fn, stream):
    """Elapsed ms of fn() between two HIP events on `stream`, device synchronised both sides."""
    import torch

    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record(stream)
    fn()
    r1.record(stream)
    torch.cuda.synchronize()
    return r0.elapsed_time(r1)


def _graph_of(prob, steps):
    import torch

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            prob.run()
    graph.replay()                       # untimed first replay
    torch.cuda.synchronize()
    return graph


def time_launches(prob, steps, warmup, launch="auto"):
    """Times `steps` back-to-back launches with inputs resident in HBM.

    Two ways to issue the steps: eagerly (one Python call, one hipLaunchKernel per step) or
    as one replay of a HIP graph holding the `steps` launches.  "auto" times 10 eager steps
    and, only when a step is short enough for the host's launch cost to matter (under
    GRAPH_PROBE_BELOW_MS), 10 graph steps, and takes the faster.  Longer kernels stay eager
    without a graph probe: on this GPU a graph replay leaves the eager launches after it
    slower for tens of milliseconds (a 256x256-tile kernel of ~220 us measured 6-20 % slower
    for the next 70 launches), which would be timed as the kernel's own cost.  The timed
    steps follow a fresh warm-up of at least 0.25 s in the chosen mode.  Returns (ms per
    step, mode, probe {mode: ms per step}).
    """
    import torch

    stream = torch.cuda.current_stream()

    def eager(n):
        for _ in range(n):
            prob.run(stream.cuda_stream)

    def warm(fn, per_call):
        # `warmup` steps, continued until 0.25 s have passed when warmup > 0 (the clocks take
        # that long to settle under load)
        t0 = time.perf_counter()
        done = 0
        while done < warmup or (warmup > 0 and time.perf_counter() - t0 < 0.25):
            fn()
            done += per_call
            torch.cuda.synchronize()

    warm(lambda: eager(8), 8)
    probe = {}
    if launch == "auto":
        n = min(steps, 10)
        probe["eager"] = _region_ms(lambda: eager(n), stream) / n
        launch = "eager"
        if probe["eager"] < GRAPH_PROBE_BELOW_MS:
            g = _graph_of(prob, n)
            probe["graph"] = _region_ms(g.replay, stream) / n
            del g
            launch = min(probe, key=probe.get)
    if launch == "graph":
        g = _graph_of(prob, steps)
        warm(g.replay, steps)
        ms = _region_ms(g.replay, stream) / steps
        del g
    else:
        warm(lambda: eager(8), 8)
        ms = _region_ms(lambda: eager(steps), stream) / steps
    return ms, launch, {k: round(v, 6) for k, v in probe.items()}


def cold_launches(prob, n, flops):
    """Median single-launch time with L2 and MALL flushed before each launch (a 1 GiB write
    between launches, outside the events)."""
    import torch

    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(n):
        scrub.fill_(1.0)
        times.append(_region_ms(lambda: prob.run(stream.cuda_stream), stream))
    del scrub
    times.sort()
    med = times[len(times) // 2]
    return {"launches": n, "ms_median": round(med, 6), "tflops": round(flops / (med * 1e-3) / 1e12, 3)}


def bare_chain(w):
    return (("pairwise", "none"),) if w.pairwise else ()


class _VendorGemm:
    """The workload's product alone through torch.matmul (hipBLASLt on ROCm), bf16 in and out,
    on the same device tensors ([batch, rows, cols]): B [K][N] as is, B [N][K] (batch 1 only)
    as a transposed view of a 2-D matrix (the library's K-contiguous kernel), the pairwise
    product as one GEMM over [B | B2]."""

    def __init__(self, w, prob):
        import torch

        A, B = prob.tensors["A"], prob.tensors["B"]
        nk = getattr(w, "b_layout", "kn") == "nk"
        if w.pairwise:
            B = torch.cat([B, prob.tensors["B2"]], dim=1 if nk else 2)
        if nk:
            # 2-D only: a batched bf16 product with a transposed right operand is avoided
            assert A.shape[0] == 1 and B.shape[0] == 1
            A, B = A[0], B[0].t()
        self.A, self.B = A, B
        self.Y = torch.empty(*A.shape[:-1], B.shape[-1], dtype=torch.bfloat16, device=A.device)

    def run(self, stream=None):
        import torch

        torch.matmul(self.A, self.B, out=self.Y)


def vendor_bare_gemm(w, prob, args, mode):
    """ms per step and TFLOP/s of the vendor library's bare GEMM on the workload (bf16 operands
    only; None for fp8 operands)."""
    if getattr(w, "in_dtype", "bf16") != "bf16" or (getattr(w, "b_layout", "kn") == "nk" and w.batch != 1):
        return None
    v = _VendorGemm(w, prob)
    ms, vmode, _ = time_launches(v, args.steps, args.warmup, mode)
    del v
    return {"library": "torch.matmul (hipBLASLt)", "ms_per_step": round(ms, 6),
            "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 3), "launch_mode": vmode}


# ops that define the kind of output rather than a step of the epilogue; never left out
STRUCTURAL_OPS = ("pairwise", "quant_fp8")


def chain_breakdown(w, inputs, prob, args, mode):
    """ms per step of the full chain, of the bare store, and of the chain with each epilogue op
    left out in turn (same instance rule, same inputs): full - without_op is that op's cost."""
    from gemm_epilogue_transformer_tiled_amd import runner

    out = {"full_ms": round(time_launches(prob, args.steps, args.warmup, mode)[0], 6)}
    variants = [("bare", w.__class__(**{**w.__dict__, "chain": bare_chain(w), "out": "bf16", "name": w.name + "-bare"}))]
    for op in w.chain:
        if op[0] in STRUCTURAL_OPS:
            continue
        chain = tuple(o for o in w.chain if o is not op)
        variants.append((f"without_{op[0]}", w.__class__(**{**w.__dict__, "chain": chain, "name": w.name + "-" + op[0]})))
    for name, wv in variants:
        pv = runner.prepare(wv, inputs)
        out[name + "_ms"] = round(time_launches(pv, args.steps, args.warmup, mode)[0], 6)
        del pv
    out["full_again_ms"] = round(time_launches(prob, args.steps, 0, mode)[0], 6)
    return out


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
    # the split: the oracle's GEMM step alone on the same sample (operands decoded untimed)
    from oracle.chain import decode_operand
    a = decode_operand(sub["A"] if rows is None else sub["A"][:, rows, :])
    bs = [decode_operand(sub[k]) for k in ("B", "B2") if k in sub and (k == "B" or w.pairwise)]
    if w.b_layout == "nk":
        bs = [np.swapaxes(b, -1, -2) for b in bs]
    t1 = time.perf_counter()
    for b in bs:
        oracle.gemm(a, b)
    gemm_s = time.perf_counter() - t1
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flops_per * reps / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "sample": sample_desc + f" x{reps} in {el:.1f} s (float64 GEMM + unfused epilogue + encode)",
            "gemm_s_per_sample": round(gemm_s, 6), "rest_s_per_sample": round(el / reps - gemm_s, 6),
            "cpu_model": cpu_model}


def roofline_bound(w, peak_tflops):
    """("mfma" | "hbm", ideal µs at the MFMA peak, ideal µs at the HBM peak): the bound is the
    larger of the two ideal times (flops at the matrix-core peak of the operand type, the
    algorithmic bytes at 8 TB/s)."""
    t_mfma = w.flops() / (peak_tflops * 1e12) * 1e6
    t_hbm = w.algorithmic_bytes() / (PEAK_HBM_GBS * 1e9) * 1e6
    return ("mfma" if t_mfma >= t_hbm else "hbm"), t_mfma, t_hbm


def run_one(args):
    """Measures one workload in this process and prints its JSON line."""
    import torch

    import workloads
    from gemm_epilogue_transformer_tiled_amd import runner

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = workloads.WORKLOADS[args.config]
    inputs = workloads.generate(w)
    from gemm_epilogue_transformer_tiled_amd import tuning

    cache = tuning.TileCache.load(args.tile_cache) if args.tile_cache else None
    prob = runner.prepare(w, inputs, cache=cache)
    tuned = None
    if args.tune:
        default_kernel = prob.plan.describe()
        cache = cache or tuning.TileCache(path="")
        best, timings = runner.tune(prob, cache, steps=min(args.steps, 20))
        if args.tile_cache:
            cache.save()
        prob = prob.with_tile(best)
        tuned = {"ms_per_launch": {str(t): round(v, 6) for t, v in timings.items()}, "chosen": best,
                 "default_kernel": default_kernel}
    ms_step, mode, probe = time_launches(prob, args.steps, args.warmup, args.launch)
    flops = w.flops()
    value = flops / (ms_step * 1e-3) / 1e12
    # The steps run back to back, so the kernel's average launch duration is the step time.
    launch_ms = ms_step
    achieved = value
    # a contraction is priced against the matrix-core peak of its own operand type; a workload
    # whose ideal time at 8 TB/s exceeds its ideal time at that peak is priced against HBM
    fp8_in = w.in_dtype == "fp8_e4m3"
    peak = PEAK_FP8_TFLOPS if fp8_in else PEAK_BF16_TFLOPS
    bound, t_mfma_us, t_hbm_us = roofline_bound(w, peak)
    gbs = w.algorithmic_bytes() / (launch_ms * 1e-3) / 1e9
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
        "dtype": "fp8_e4m3" if fp8_in else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "batch": w.batch, "M": w.M, "N": w.N, "K": w.K,
            "chain": [list(op) for op in w.chain],
            "output": w.out,
            "kernel": prob.plan.describe(),
        },
        "launch": {"mode": mode, "probe_ms_per_step": probe},
        "tile_sweep": tuned,
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 3) if bound == "mfma" else round(gbs, 1),
            "peak": peak if bound == "mfma" else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
            "frac": round(achieved / peak, 4) if bound == "mfma" else round(gbs / PEAK_HBM_GBS, 4),
            "frac_mfma": round(achieved / peak, 4),
            "ideal_us_at_mfma_peak": round(t_mfma_us, 3),
            "ideal_us_at_hbm_peak": round(t_hbm_us, 3),
            "traffic": MEASURED_TRAFFIC.get(w.name) if kernel_code_hash() == MEASURED_TRAFFIC_CODE else None,
            "kernel": "fused_gemm_epilogue",
            "launch_ms_mean": round(launch_ms, 6),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes(),
            "hbm_gbs_at_algorithmic_bytes": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        },
    }
    if max(t_mfma_us, t_hbm_us) < 1.0:
        result["roofline"]["note"] = ("launch-latency bound: the ideal time at either peak is under 1 us, "
                                      "so the fraction measures launch and synchronisation cost")
    if not args.no_bare:
        # fused, bare, fused again: the overhead compares the bare kernel with the mean of the
        # fused runs on either side of it, so slow clock drift cancels
        wb = w.__class__(**{**w.__dict__, "chain": bare_chain(w), "out": "bf16", "name": w.name + "-bare"})
        bare = runner.prepare(wb, inputs)
        bare_ms, _, _ = time_launches(bare, args.steps, args.warmup, mode)
        again_ms, _, _ = time_launches(prob, args.steps, 0, mode)
        result["bare_gemm_ms"] = round(bare_ms, 6)
        result["epilogue_overhead_pct"] = round(((launch_ms + again_ms) / 2 / bare_ms - 1.0) * 100.0, 2)
        del bare
    if args.breakdown:
        result["breakdown"] = chain_breakdown(w, inputs, prob, args, mode)
    if args.vendor:
        result["vendor_bare_gemm"] = vendor_bare_gemm(w, prob, args, mode)
    if not args.no_cold:
        result["cold"] = cold_launches(prob, min(args.steps, 20), flops)
    if not args.no_unfused:
        from gemm_epilogue_transformer_tiled_amd import baselines
        unf = baselines.Unfused(w, inputs)
        unf_ms, _, _ = time_launches(unf, args.steps, args.warmup, mode)
        ub = unf.algorithmic_bytes()
        result["unfused"] = {
            "kernels": unf.kernels(),
            "ms_per_step": round(unf_ms, 6),
            "fused_speedup": round(unf_ms / launch_ms, 3),
            "algorithmic_bytes": ub,
            "bytes_saved": ub - w.algorithmic_bytes(),
            "bytes_ratio": round(ub / w.algorithmic_bytes(), 3),
        }
        del unf
    del prob
    torch.cuda.synchronize()
    if not args.no_probes:
        from gemm_epilogue_transformer_tiled_amd import baselines
        mf = baselines.probe_mfma()
        mf16 = baselines.probe_mfma(form="bf16_16x16x32")
        mf8 = baselines.probe_mfma(form="fp8_32x32x64")
        cp = baselines.probe_copy()
        ll = baselines.probe_lds_load()
        lr = baselines.probe_lds_read()
        result["measured_peaks"] = {"mfma_bf16_tflops": mf["tflops"], "mfma_implied_clock_ghz": mf["implied_clock_ghz"],
                                    "mfma_bf16_16x16x32_tflops": mf16["tflops"],
                                    "mfma_fp8_tflops": mf8["tflops"], "mfma_fp8_implied_clock_ghz": mf8["implied_clock_ghz"],
                                    "copy_gbs": cp["gbs"], "l2_to_lds_gbs": ll["gbs"],
                                    "lds_read_gbs": lr["gbs"], "lds_read_bytes_per_clk_cu": lr["bytes_per_clk_cu"],
                                    "lds_read_implied_clock_ghz": lr["implied_clock_ghz"]}
        # against the probe of the instruction the mainloop runs: fp8 operands 32x32x64, the
        # two-wave bf16 instances (512 threads) 16x16x32, the one-wave bf16 instances 32x32x16
        two_wave = "threads=512" in result["config"]["kernel"]
        ref = mf8 if fp8_in else (mf16 if two_wave else mf)
        result["roofline"]["frac_of_measured_mfma_peak"] = round(achieved / ref["tflops"], 4)
        result["roofline"]["measured_mfma_probe"] = ref.get("form")
        result["roofline"]["frac_of_measured_copy_gbs"] = round(gbs / cp["gbs"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _summary(d):
    """The per-configuration record of a child's JSON line."""
    rf = d.get("roofline", {})
    out = {
        "status": "ok",
        "workload": d["config"]["workload"],
        "kernel": d["config"].get("kernel"),
        "dtype": d.get("dtype"),
        "value": d["value"],
        "unit": d["unit"],
        "ms_per_step": d["ms_per_step"],
        "launch_mode": d.get("launch", {}).get("mode"),
        "bound": rf.get("bound"),
        "frac": rf.get("frac"),
        "frac_mfma": rf.get("frac_mfma"),
        "gbs": rf.get("hbm_gbs_at_algorithmic_bytes"),
        "frac_hbm": rf.get("hbm_frac"),
        "traffic": rf.get("traffic"),
        "algorithmic_bytes_per_launch": rf.get("algorithmic_bytes_per_launch"),
        "epilogue_overhead_pct": d.get("epilogue_overhead_pct"),
        "bare_gemm_ms": d.get("bare_gemm_ms"),
    }
    if "note" in rf:
        out["note"] = rf["note"]
    if "unfused" in d:
        u = d["unfused"]
        out["unfused"] = {k: u[k] for k in ("ms_per_step", "fused_speedup", "algorithmic_bytes", "bytes_saved",
                                            "bytes_ratio") if k in u}
    if "cold" in d:
        out["cold_ms_median"] = d["cold"]["ms_median"]
    if "cpu_baseline" in d:
        out["cpu_baseline"] = d["cpu_baseline"]
    return out


def run_suite(args):
    """Runs every configuration of the suite in a child process (this process never touches
    the GPU) and prints one JSON line: the headline configuration's fields plus per_config."""
    names = [n for n in args.suite.split(",") if n]
    for n in names:
        if n not in SUITE:
            print(f"unknown configuration {n!r} in --suite", file=sys.stderr)
            sys.exit(2)
    headline = names[0]
    per, lines, stop = {}, {}, None
    t_suite = time.perf_counter()
    for n in names:
        if stop is not None:
            per[n] = {"status": "skipped", "reason": f"{stop} ended abnormally; nothing more was started on the GPU"}
            continue
        cmd = [sys.executable, "-u", os.path.abspath(__file__), "--config", n, "--steps", str(args.steps),
               "--warmup", str(args.warmup), "--launch", args.launch,
               "--cpu-seconds", str(args.cpu_seconds if n == headline else args.suite_cpu_seconds)]
        for flag in ("no_cpu_baseline", "no_bare", "no_cold", "no_unfused", "no_probes"):
            if getattr(args, flag):
                cmd.append("--" + flag.replace("_", "-"))
        print(f"[bench] {n}: start", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=args.child_timeout)
            rc, out, err = r.returncode, r.stdout, r.stderr
        except subprocess.TimeoutExpired as e:
            rc, out, err = 124, (e.stdout or b""), (e.stderr or b"")
            out = out.decode(errors="replace") if isinstance(out, bytes) else out
            err = err.decode(errors="replace") if isinstance(err, bytes) else err
        el = time.perf_counter() - t0
        line = next((l for l in reversed(out.splitlines()) if l.startswith("{")), None)
        if rc == 0 and line is not None:
            d = json.loads(line)
            lines[n] = d
            per[n] = _summary(d)
            per[n]["wall_s"] = round(el, 1)
            print(f"[bench] {n}: ok, {d['value']} TFLOP/s, {d['ms_per_step'] * 1e3:.2f} us/step ({el:.1f} s)",
                  file=sys.stderr, flush=True)
        else:
            per[n] = {"status": "failed", "rc": rc, "wall_s": round(el, 1),
                      "stderr_tail": "\n".join(err.strip().splitlines()[-6:])}
            print(f"[bench] {n}: FAILED rc={rc} ({el:.1f} s)\n{per[n]['stderr_tail']}", file=sys.stderr, flush=True)
            if rc in ABNORMAL_RC:
                stop = n
    if headline in lines:
        result = dict(lines[headline])
    else:
        result = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                  "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
                  "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                  "config": {"workload": headline}, "status": per[headline]}
    result["per_config"] = per
    result["suite_wall_s"] = round(time.perf_counter() - t_suite, 1)
    print(json.dumps(result), flush=True)
    if headline not in lines:
        sys.exit(1)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the fused GEMM-epilogue path has no multi-GPU leg "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.config is None:
        run_suite(args)
    else:
        run_one(args)


if __name__ == "__main__":
    main()
