"""Marshalling between seeded workloads and the C-ABI (no arithmetic here).

Turns a workload's host bit arrays into device tensors, builds the descriptor
for its epilogue chain, and enqueues ``gemm_epilogue_run`` on the current
torch stream.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np
import torch

from . import (GE_DT_BF16, GE_DT_FP8_E4M3, GE_LAYOUT_KN, GE_LAYOUT_NK, Plan, ge_args_t, ge_desc_t, make_args,
               make_desc, make_ops, tuning)


def to_device_bf16(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit array -> torch.bfloat16 tensor on ``device``."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_device(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bits -> torch.bfloat16; uint8 e4m3 codes -> torch.uint8 (same bytes)."""
    if bits.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device)
    return to_device_bf16(bits, device)


@dataclasses.dataclass
class DeviceProblem:
    workload: object
    plan: Plan
    tensors: Dict[str, torch.Tensor]
    Y: torch.Tensor
    amax: Optional[torch.Tensor]
    args: object
    col_sum: Optional[torch.Tensor] = None

    def run(self, stream: Optional[int] = None) -> None:
        self.plan.run(self.args, stream)

    def y_host_bits(self) -> np.ndarray:
        y = self.Y.cpu()
        if self.workload.out == "fp8_e4m3":
            return y.view(torch.uint8).numpy()
        return y.view(torch.int16).numpy().view(np.uint16)

    def amax_host(self) -> Optional[float]:
        return None if self.amax is None else float(self.amax.item())

    def col_sum_host(self):
        return None if self.col_sum is None else self.col_sum.cpu().numpy().astype(np.float64)

    def with_tile(self, tile: int, library=None) -> "DeviceProblem":
        """The same problem (same device tensors and outputs) planned on kernel instance `tile`
        (of `library`, a library loaded by the binding; default: the fused path's)."""
        desc = ge_desc_t.from_buffer_copy(self.plan.desc)
        desc.tile = tile + 1
        args = ge_args_t.from_buffer_copy(self.args)
        args.workspace, args.workspace_bytes = None, 0        # the new plan brings its own
        return dataclasses.replace(self, plan=Plan(desc, library=library), args=args)


def descriptor(w) -> ge_desc_t:
    """The descriptor of workload `w` (dense operands and output, no tile requested)."""
    in_t = GE_DT_FP8_E4M3 if getattr(w, "in_dtype", "bf16") == "fp8_e4m3" else GE_DT_BF16
    return make_desc(w.batch, w.M, w.N, w.K, make_ops(w.chain),
                     y_type=GE_DT_FP8_E4M3 if w.out == "fp8_e4m3" else GE_DT_BF16, a_type=in_t, b_type=in_t,
                     b_layout=GE_LAYOUT_NK if getattr(w, "b_layout", "kn") == "nk" else GE_LAYOUT_KN)


def prepare(w, inputs: Dict[str, np.ndarray], device="cuda", y_fill: Optional[int] = None,
            tile: Optional[int] = None, cache: Optional[tuning.TileCache] = None) -> DeviceProblem:
    """Uploads inputs, allocates Y (and AMAX), creates the plan for workload ``w``.  The kernel
    instance is `tile` if given, else the one `cache` holds for this problem, else create's
    own choice."""
    t = {k: to_device(v, device) for k, v in inputs.items()
         if k in ("A", "B", "B2", "bias", "R", "Z")}
    if "row_scale" in inputs:
        t["row_scale"] = torch.from_numpy(np.ascontiguousarray(inputs["row_scale"], dtype=np.float32)).to(device)
    fp8 = w.out == "fp8_e4m3"
    shape = (w.batch, w.M, w.N)
    if fp8:
        Y = torch.empty(shape, dtype=torch.uint8, device=device)
    else:
        Y = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if y_fill is not None:
        Y.view(torch.uint8).fill_(y_fill)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=device) if w.has("amax") else None
    col = torch.full((w.N,), float("nan"), dtype=torch.float32, device=device) if w.has("col_sum") else None
    desc = descriptor(w)
    if tile is None and cache is not None:
        tile = cache.lookup(desc)
    if tile is not None:
        desc.tile = tile + 1
    plan = Plan(desc)
    args = make_args(A=t.get("A"), B=t.get("B"), B2=t.get("B2"), bias=t.get("bias"), residual=t.get("R"),
                     row_scale=t.get("row_scale"), Y=Y, amax=amax, alpha=w.alpha, quant_scale=w.quant_scale,
                     aux=t.get("Z"), col_sum=col)
    return DeviceProblem(w, plan, t, Y, amax, args, col)


def tune(prob: DeviceProblem, cache: tuning.TileCache, steps: int = 20) -> Tuple[int, Dict[int, float]]:
    """Sweeps every admissible kernel instance on `prob`'s tensors, records the fastest in
    `cache` (not saved) and returns (best tile, {tile: ms per launch})."""
    def make_run(t):
        p = prob.with_tile(t)
        return lambda: p.run()
    timings = tuning.sweep(prob.plan.desc, make_run, steps=steps)
    return cache.record(prob.plan.desc, timings), timings
