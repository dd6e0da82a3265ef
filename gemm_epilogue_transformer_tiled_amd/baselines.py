"""Binding of libge_baselines.so: the unfused comparator sequence and the calibration probes.

Measurement infrastructure, not the fused path.  `Unfused` runs a workload the way the pages
describe it before fusion -- the GEMM (libgemm_epilogue.so with an empty chain) writes bf16 C,
then every epilogue operation is its own kernel reading and writing a whole bf16 array -- so that
the fused kernel's HBM bytes saved and speed-up are measured.  Argument marshalling only: all the
arithmetic runs in the kernels declared in ``include/ge_baselines.h``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

from . import GE_DT_BF16, GE_DT_FP8_E4M3, GE_LAYOUT_KN, GE_LAYOUT_NK, Plan, make_args, make_desc, make_ops
from .runner import to_device

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libge_baselines.so")

EXPORTED = ("ge_unfused_scale", "ge_unfused_bias_col", "ge_unfused_act", "ge_unfused_act_mul",
            "ge_unfused_row_rms", "ge_unfused_row_scale", "ge_unfused_add", "ge_unfused_amax",
            "ge_unfused_quant_fp8", "ge_unfused_act_grad", "ge_unfused_col_sum", "ge_probe_mfma",
            "ge_probe_mfma_variant", "ge_probe_mfma_f8", "ge_probe_lds_load", "ge_probe_lds_read",
            "ge_probe_copy")
ACTS = {"none": 0, "relu": 1, "gelu_tanh": 2, "silu": 3}

_p, _i64, _i, _f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
_SIGS = {
    "ge_unfused_scale": [_p, _p, _i64, _f, _p],
    "ge_unfused_bias_col": [_p, _p, _p, _i64, _i64, _p],
    "ge_unfused_act": [_p, _p, _i64, _i, _p],
    "ge_unfused_act_mul": [_p, _p, _p, _i64, _i, _p],
    "ge_unfused_row_rms": [_p, _p, _i64, _i64, _f, _p],
    "ge_unfused_row_scale": [_p, _p, _p, _i64, _i64, _p],
    "ge_unfused_add": [_p, _p, _p, _i64, _p],
    "ge_unfused_amax": [_p, _i64, _p, _p],
    "ge_unfused_quant_fp8": [_p, _p, _i64, _f, _p],
    "ge_unfused_act_grad": [_p, _p, _p, _i64, _i, _p],
    "ge_unfused_col_sum": [_p, _p, _i64, _i64, _p],
    "ge_probe_mfma": [_p, _i, _i, _p],
    "ge_probe_mfma_variant": [_p, _i, _i, _i, _p],
    "ge_probe_mfma_f8": [_p, _p, _p, _p, _i, _p],
    "ge_probe_lds_load": [_p, _i, _p, _i, _i, _p],
    "ge_probe_lds_read": [_p, _p, _i, _i, _p],
    "ge_probe_copy": [_p, _p, _i64, _p],
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python gemm_epilogue_transformer_tiled_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    return lib


lib = _load()


def call(name: str, *args) -> None:
    st = getattr(lib, name)(*args)
    if st != 0:
        raise RuntimeError(f"{name} failed with status {st}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class Unfused:
    """The unfused sequence for workload `w` on uploaded inputs.

    steps: list of (name, callable, bytes read, bytes written) -- the bytes are the algorithmic
    HBM traffic of that kernel (each input read once, each output written once)."""

    def __init__(self, w, inputs: Dict, device="cuda"):
        self.w = w
        t = {k: to_device(v, device) for k, v in inputs.items() if k in ("A", "B", "B2", "bias", "R", "Z")}
        if "row_scale" in inputs:
            import numpy as np
            t["row_scale"] = torch.from_numpy(np.ascontiguousarray(inputs["row_scale"], dtype=np.float32)).to(device)
        self.t = t
        rows, n_out = w.batch * w.M, w.batch * w.M * w.N
        bf = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=device)
        self.amax = torch.zeros(1, dtype=torch.float32, device=device) if w.has("amax") else None
        self.col_sum = torch.zeros(w.N, dtype=torch.float32, device=device) if w.has("col_sum") else None
        self.plans: List[Plan] = []
        steps: List[Tuple[str, object, int, int]] = []
        A = t["A"]
        a_bytes = A.numel() * A.element_size()      # fp8 operands: one byte per element
        # RMS: statistic kernel, normalisation kernel, then the GEMM on the normalised rows
        if w.has("row_rms"):
            S = torch.empty(rows, dtype=torch.float32, device=device)
            Xn = bf(A.shape)
            eps = float(w.op("row_rms")[1])
            steps.append(("row_rms", lambda A=A, S=S, eps=eps: call(
                "ge_unfused_row_rms", A.data_ptr(), S.data_ptr(), rows, w.K, eps, _stream()), a_bytes, rows * 4))
            steps.append(("row_normalise", lambda A=A, S=S, Xn=Xn: call(
                "ge_unfused_row_scale", A.data_ptr(), S.data_ptr(), Xn.data_ptr(), rows, w.K, _stream()),
                a_bytes + rows * 4, a_bytes))
            A = Xn
        C = bf(w.batch, w.M, w.N)
        nb = lambda x: x.numel() * x.element_size()
        steps.append(("gemm", self._gemm(A, t["B"], C), nb(A) + nb(t["B"]), n_out * 2))
        cur = C
        if w.pairwise:
            U = bf(w.batch, w.M, w.N)
            steps.append(("gemm_up", self._gemm(A, t["B2"], U), nb(A) + nb(t["B2"]), n_out * 2))
            Y = bf(w.batch, w.M, w.N)
            act = ACTS[w.op("pairwise")[1]]
            steps.append(("act_mul", lambda g=cur, u=U, y=Y, act=act: call(
                "ge_unfused_act_mul", g.data_ptr(), u.data_ptr(), y.data_ptr(), n_out, act, _stream()),
                2 * n_out * 2, n_out * 2))
            cur = Y
        for op in w.chain:
            kind = op[0]
            if kind in ("pairwise", "row_rms"):
                continue
            if kind == "col_sum":
                steps.append(("col_sum", lambda x=cur: call(
                    "ge_unfused_col_sum", x.data_ptr(), self.col_sum.data_ptr(), rows, w.N, _stream()),
                    n_out * 2, w.N * 4))
                continue
            if kind == "amax":
                steps.append(("amax", lambda x=cur: call(
                    "ge_unfused_amax", x.data_ptr(), n_out, self.amax.data_ptr(), _stream()), n_out * 2, 4))
                continue
            if kind == "quant_fp8":
                Y8 = torch.empty(w.batch, w.M, w.N, dtype=torch.uint8, device=device)
                steps.append(("quant_fp8", lambda x=cur, y=Y8: call(
                    "ge_unfused_quant_fp8", x.data_ptr(), y.data_ptr(), n_out, float(w.quant_scale), _stream()),
                    n_out * 2, n_out))
                cur = Y8
                continue
            Y = bf(w.batch, w.M, w.N)
            if kind == "scale":
                fn = lambda x=cur, y=Y: call("ge_unfused_scale", x.data_ptr(), y.data_ptr(), n_out,
                                             float(w.alpha), _stream())
                rd = n_out * 2
            elif kind == "row_scale":
                s = t["row_scale"]
                fn = lambda x=cur, y=Y, s=s: call("ge_unfused_row_scale", x.data_ptr(), s.data_ptr(), y.data_ptr(),
                                                  rows, w.N, _stream())
                rd = n_out * 2 + rows * 4
            elif kind == "bias":
                fn = lambda x=cur, y=Y: call("ge_unfused_bias_col", x.data_ptr(), t["bias"].data_ptr(), y.data_ptr(),
                                             rows, w.N, _stream())
                rd = n_out * 2 + w.N * 2
            elif kind == "act":
                act = ACTS[op[1]]
                fn = lambda x=cur, y=Y, act=act: call("ge_unfused_act", x.data_ptr(), y.data_ptr(), n_out, act,
                                                      _stream())
                rd = n_out * 2
            elif kind == "act_grad":
                act = ACTS[op[1]]
                fn = lambda x=cur, y=Y, act=act: call("ge_unfused_act_grad", x.data_ptr(), t["Z"].data_ptr(),
                                                      y.data_ptr(), n_out, act, _stream())
                rd = 2 * n_out * 2
            elif kind == "residual":
                fn = lambda x=cur, y=Y: call("ge_unfused_add", x.data_ptr(), t["R"].data_ptr(), y.data_ptr(), n_out,
                                             _stream())
                rd = 2 * n_out * 2
            else:
                raise ValueError(f"no unfused kernel for {kind}")
            steps.append((kind, fn, rd, n_out * 2))
            cur = Y
        self.steps = steps
        self.Y = cur

    def _gemm(self, A, B, C):
        w = self.w
        in_t = GE_DT_FP8_E4M3 if A.dtype == torch.uint8 else GE_DT_BF16
        plan = Plan(make_desc(w.batch, w.M, w.N, w.K, make_ops([]), y_type=GE_DT_BF16, a_type=in_t, b_type=in_t,
                              b_layout=GE_LAYOUT_NK if w.b_layout == "nk" else GE_LAYOUT_KN))
        self.plans.append(plan)
        args = make_args(A=A, B=B, Y=C)
        return lambda: plan.run(args)

    def run(self, stream: Optional[int] = None) -> None:
        for _, fn, _, _ in self.steps:
            fn()

    def algorithmic_bytes(self) -> int:
        return sum(r + wr for _, _, r, wr in self.steps)

    def kernels(self) -> List[str]:
        return [s[0] for s in self.steps]

    def col_sum_host(self):
        return None if self.col_sum is None else self.col_sum.cpu().numpy().astype("float64")

    def amax_host(self) -> Optional[float]:
        return None if self.amax is None else float(self.amax.item())

    def y_host_bits(self):
        y = self.Y.cpu()
        if self.w.out == "fp8_e4m3":
            return y.view(torch.uint8).numpy()
        import numpy as np
        return y.view(torch.int16).numpy().view(np.uint16)


# matrix-core probe forms: variant -> (chains per wave, flop per instruction)
PROBE_FORMS = {"bf16_32x32x16": (0, 16, 32768.0), "bf16_16x16x32": (1, 16, 16384.0), "fp8_32x32x64": (2, 8, 131072.0)}


def probe_mfma(workgroups: int = 1024, iters: int = 4096, form: str = "bf16_32x32x16") -> Dict:
    """Sustained matrix-core TFLOP/s of one instruction form (``PROBE_FORMS``; default
    v_mfma_f32_32x32x16_bf16) on random register operands that change from one instruction to
    the next."""
    variant, chains, per_inst = PROBE_FORMS[form]
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    call("ge_probe_mfma_variant", sink.data_ptr(), workgroups, 16, variant, _stream())     # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(3):
        e0.record()
        call("ge_probe_mfma_variant", sink.data_ptr(), workgroups, iters, variant, _stream())
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    flops = workgroups * 4 * chains * iters * per_inst
    # implied clock: a CU's matrix cores do 4096 bf16 (8192 fp8) flop per cycle, 256 CUs
    per_cu_cycle = 8192 if form.startswith("fp8") else 4096
    return {"form": form, "tflops": round(flops / best / 1e9, 1), "ms": round(best, 4),
            "implied_clock_ghz": round(flops / (best * 1e-3) / (256 * per_cu_cycle) / 1e9, 3)}


def probe_lds_load(src_kb: int = 2048, workgroups: int = 512, iters: int = 2048) -> Dict:
    """Sustained rate of direct global->LDS loads from an L2-resident buffer (the fused
    kernels' operand path with nothing else running), GB/s over all CUs."""
    src = torch.zeros(src_kb * 1024, dtype=torch.uint8, device="cuda")
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    call("ge_probe_lds_load", src.data_ptr(), src_kb, sink.data_ptr(), workgroups, 16, _stream())   # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(3):
        e0.record()
        call("ge_probe_lds_load", src.data_ptr(), src_kb, sink.data_ptr(), workgroups, iters, _stream())
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    nbytes = workgroups * iters * 32768.0
    return {"gbs": round(nbytes / best / 1e6, 1), "ms": round(best, 4), "src_kb": src_kb, "workgroups": workgroups}


def probe_lds_read(workgroups: int = 256, iters: int = 16384) -> Dict:
    """Sustained LDS read rate (the fused kernels' fragment reads with nothing else running):
    one 8-wave workgroup per CU reading 16 bytes per lane without bank conflicts.  Returns the
    aggregate GB/s (host events), the shader clock implied by the workgroups' s_memtime cycles
    over the kernel's time, and bytes per clock per CU (bytes of one workgroup over its median
    s_memtime cycles)."""
    sink = torch.empty(workgroups * 512, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2 * workgroups, dtype=torch.int64, device="cuda")
    call("ge_probe_lds_read", sink.data_ptr(), clocks.data_ptr(), workgroups, 64, _stream())   # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(3):
        e0.record()
        call("ge_probe_lds_read", sink.data_ptr(), clocks.data_ptr(), workgroups, iters, _stream())
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if best is None or ms < best[0]:
            best = (ms, clocks.cpu().numpy().reshape(workgroups, 2).copy())
    ms, ck = best
    wg_bytes = iters * 65536.0
    cycles = float(np.median(ck[:, 0]))
    ticks = float(np.median(ck[:, 1]))
    return {"gbs": round(workgroups * wg_bytes / ms / 1e6, 1), "ms": round(ms, 4), "workgroups": workgroups,
            "bytes_per_clk_cu": round(wg_bytes / cycles, 1) if cycles > 0 else None,
            "implied_clock_ghz": round(cycles / (ms * 1e6), 3),
            "memtime_per_realtime_tick": round(cycles / ticks, 2) if ticks > 0 else None}


def mfma_f8(src0: np.ndarray, src1: np.ndarray, c: np.ndarray) -> np.ndarray:
    """One v_mfma_f32_32x32x64_f8f6f4 per wave: src0, src1 uint8 e4m3 codes [waves, 64, 32]
    (lane, register byte), c float32 [waves, 64, 16] (lane, accumulator register); returns the
    float32 result registers [waves, 64, 16]."""
    waves = src0.shape[0]
    assert src0.shape == (waves, 64, 32) and src1.shape == (waves, 64, 32) and c.shape == (waves, 64, 16)
    dev = "cuda"
    t0 = torch.from_numpy(np.ascontiguousarray(src0, dtype=np.uint8)).to(dev)
    t1 = torch.from_numpy(np.ascontiguousarray(src1, dtype=np.uint8)).to(dev)
    tc = torch.from_numpy(np.ascontiguousarray(c, dtype=np.float32)).to(dev)
    td = torch.empty_like(tc)
    call("ge_probe_mfma_f8", t0.data_ptr(), t1.data_ptr(), tc.data_ptr(), td.data_ptr(), waves, _stream())
    torch.cuda.synchronize()
    return td.cpu().numpy()


def probe_copy(mib: int = 1024) -> Dict:
    """Sustained device copy GB/s (bytes read + bytes written per second)."""
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    call("ge_probe_copy", src.data_ptr(), dst.data_ptr(), n, _stream())
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(5):
        e0.record()
        call("ge_probe_copy", src.data_ptr(), dst.data_ptr(), n, _stream())
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return {"gbs": round(2 * n / (best * 1e-3) / 1e9, 1), "ms": round(best, 4), "bytes_each_way": n}
