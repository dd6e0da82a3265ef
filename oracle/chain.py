"""Literal, unfused evaluation of an epilogue chain after a float64 GEMM.

Test infrastructure only (see the package docstring).

The fused kernel reaches, up to rounding order, the result of running the
GEMM and then each epilogue op as its own pass over the whole array (CODA news
item, "How CODA works": the ops are re-expressed to run on the still-on-chip
output tile; cuDNN tutorial, batched-matmul paragraph: the gain comes from
removing the epilogue's memory traffic, not from a different result).  So the
oracle is that sequence, in the canonical order

    t = alpha * acc -> t = s[m] * t -> t = t + bias[n]
      -> y = act(t)   (or y = act(t_gate) * t_up for the pairwise op,
                       or y = t * act'(Z[m, n]) for the backward activation gradient)
      -> y = y + R[m, n] -> colsum[n] = sum_m y -> amax = max|y|
      -> encode (bf16, or fp8 of y * scale)

AMAX is taken on the unrounded value ``y`` (before the fp8 scale), the value
whose maximum sets the next quantisation scale.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

from . import ops
from .codecs import decode_bf16, decode_e4m3, encode_bf16


@dataclasses.dataclass
class OracleResult:
    y: np.ndarray                 # float64 final value before output encoding
    codes: np.ndarray             # uint16 bf16 bits or uint8 e4m3 codes
    amax: Optional[float]         # None when the chain has no AMAX op
    out: str                      # "bf16" or "fp8_e4m3"
    col_sum: Optional[np.ndarray] = None   # [N] float64, when the chain has COL_SUM


def decode_operand(x: np.ndarray) -> np.ndarray:
    """GEMM operand bits -> float64, exactly: uint16 arrays are bf16 bit patterns, uint8
    arrays OCP e4m3 codes (the fp8 operands of delayed scaling; the cuDNN tutorial's
    batched-matmul paragraph feeds fp8 scaling from AMAX)."""
    if x.dtype == np.uint8:
        return decode_e4m3(x)
    return decode_bf16(x)


def run_chain(chain: Sequence[tuple], A: np.ndarray, B: np.ndarray,
              B2: Optional[np.ndarray] = None, bias: Optional[np.ndarray] = None,
              R: Optional[np.ndarray] = None, row_scale_vec: Optional[np.ndarray] = None,
              alpha: float = 1.0, quant_scale: float = 1.0, out: str = "bf16",
              rows: Optional[np.ndarray] = None, b_layout: str = "kn",
              Z: Optional[np.ndarray] = None) -> OracleResult:
    """Evaluate ``chain`` on bf16-bit inputs.

    A: uint16 [batch, M, K] (or uint8 e4m3 codes, then B and B2 too); B, B2: uint16 [batch, K, N], or [batch, N, K] with
    ``b_layout="nk"`` -- then the product is A @ B^T, the backward-pass form dY @ W^T
    (CODA news item, "How CODA works": forward and backward); bias: uint16 [N];
    R, Z: uint16 [batch, M, N] (Z: the saved pre-activation of ACT_GRAD); row_scale_vec:
    float32 [batch, M].
    ``rows`` (optional) restricts the evaluation to those rows of every batch
    (the result then has M = len(rows)); AMAX is then over those rows only.
    """
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        A = A[:, rows, :]
        if R is not None:
            R = R[:, rows, :]
        if Z is not None:
            Z = Z[:, rows, :]
        if row_scale_vec is not None:
            row_scale_vec = np.asarray(row_scale_vec)[:, rows]
    kinds = [op[0] for op in chain]
    Af = decode_operand(A)

    def as_kn(W: np.ndarray) -> np.ndarray:
        W = decode_operand(W)
        return np.swapaxes(W, -1, -2) if b_layout == "nk" else W

    acc = ops.gemm(Af, as_kn(B))
    acc2 = ops.gemm(Af, as_kn(B2)) if "pairwise" in kinds else None

    def linear_part(t: np.ndarray) -> np.ndarray:
        for op in chain:
            if op[0] == "scale":
                t = ops.scale(t, alpha)
            elif op[0] == "row_rms":
                t = ops.row_scale(t, ops.row_rms_scale(Af, op[1]))
            elif op[0] == "row_scale":
                t = ops.row_scale(t, np.asarray(row_scale_vec, dtype=np.float64))
        return t

    t = linear_part(acc)
    t2 = linear_part(acc2) if acc2 is not None else None
    result_amax = None
    result_col = None
    y = t
    for op in chain:
        kind = op[0]
        if kind in ("scale", "row_rms", "row_scale"):
            continue
        if kind == "bias":
            y = ops.bias_col(y, decode_bf16(bias))
        elif kind == "act":
            y = ops.act(y, op[1])
        elif kind == "pairwise":
            y = ops.pairwise_act_mul(y, t2, op[1])
        elif kind == "act_grad":
            y = ops.act_grad(y, decode_bf16(Z), op[1])
        elif kind == "col_sum":
            result_col = ops.col_sum(y)
        elif kind == "residual":
            y = ops.residual(y, decode_bf16(R))
        elif kind == "amax":
            result_amax = ops.amax(y)
        elif kind == "quant_fp8":
            pass                                   # applied at encoding below
        else:
            raise ValueError(f"unknown epilogue op {kind!r}")
    if out == "fp8_e4m3":
        codes = ops.quant_fp8(y, quant_scale)
    else:
        codes = encode_bf16(y)
    return OracleResult(y=y, codes=codes, amax=result_amax, out=out, col_sum=result_col)


def run_workload(w, inputs: Dict[str, np.ndarray], rows=None) -> OracleResult:
    """Run a ``workloads.Workload`` on its generated inputs."""
    return run_chain(w.chain, inputs["A"], inputs["B"], inputs.get("B2"), inputs.get("bias"),
                     inputs.get("R"), inputs.get("row_scale"), alpha=w.alpha,
                     quant_scale=w.quant_scale, out=w.out, rows=rows,
                     b_layout=getattr(w, "b_layout", "kn"), Z=inputs.get("Z"))
