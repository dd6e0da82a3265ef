"""Seeded synthetic inputs for the fused GEMM-epilogue workloads.

This module is shared by the HIP path's tests/bench and by the CPU oracle.  It
holds the workload *definitions* (shapes, host scalars, the epilogue chain as
plain data) and the random-number recipe, and nothing of the method's
arithmetic: no GEMM, no epilogue op, no encoder.  Every tensor is returned as
raw bits (bf16 as ``uint16``) or ``float32`` so both sides read identical
bytes.

Recipe (one independent stream per tensor):
  ``numpy.random.Generator(PCG64(SeedSequence([config_id, tensor_id])))``,
  tensor ids A=0, B=1, B2=2, bias=3, R=4, g=5, base W (RMS fold)=6.
  ``N(0, v)`` means variance ``v``; normals are drawn as float32 standard
  normals, multiplied by ``sqrt(v)`` in float32 and cast to bf16 with
  round-to-nearest-even (torch's float32 -> bfloat16 cast).

fp8 operands (``in_dtype="fp8_e4m3"``): the same float32 draws are multiplied by the
operand's quantisation scale, clamped to +-448 and cast to OCP e4m3 ("e4m3fn") codes with
round-to-nearest-even (torch's float32 -> float8_e4m3fn cast); the codes are the inputs.
The dequantisation factor 1 / (scale_A * scale_B) is the workload's alpha.

The RMS workload folds a per-channel gain ``g[k]`` into the weight before
anything runs: ``W'[k, n] = bf16(g[k] * W[k, n])`` with the product taken in
float32 (a row scaling over the contraction axis, the only fold for which
``rmsnorm(X) * g @ W == s * (X @ W')``).  That is input preparation: both sides
receive ``W'``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

# Tensor ids of the seeded streams.
T_A, T_B, T_B2, T_BIAS, T_R, T_G, T_W, T_Z = 0, 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    """One fused GEMM-epilogue problem.

    ``chain`` lists the epilogue ops in their canonical order as plain tuples:
    ``("scale",)``, ``("row_rms", eps)``, ``("bias",)``, ``("act", name)``,
    ``("pairwise", act_name)``, ``("act_grad", act_name)``, ``("residual",)``,
    ``("col_sum",)``, ``("amax",)``, ``("quant_fp8",)``.  Activation names: ``none``,
    ``relu``, ``gelu_tanh``, ``silu``.
    """

    name: str
    config_id: int
    batch: int
    M: int
    N: int
    K: int
    chain: Tuple[tuple, ...]
    alpha: float = 1.0
    quant_scale: float = 1.0
    a_var: str = "1/K"          # "1/K" or "1"
    b_var: str = "1/K"
    bias_var: float = 1.0
    out: str = "bf16"           # "bf16" or "fp8_e4m3"
    description: str = ""
    b_layout: str = "kn"        # "kn": B stored [K][N]; "nk": B stored [N][K] (product A @ B^T)
    in_dtype: str = "bf16"      # operand type: "bf16" or "fp8_e4m3" (codes, B stored [N][K])
    a_qscale: float = 1.0       # fp8 operands: quantisation scales of A and B
    b_qscale: float = 1.0

    @property
    def pairwise(self) -> bool:
        return any(op[0] == "pairwise" for op in self.chain)

    def has(self, kind: str) -> bool:
        return any(op[0] == kind for op in self.chain)

    def op(self, kind: str) -> Optional[tuple]:
        for op in self.chain:
            if op[0] == kind:
                return op
        return None

    def flops(self) -> float:
        """2*M*N*K per GEMM, times batch, times two for the pairwise (gate, up) pair."""
        return 2.0 * self.batch * self.M * self.N * self.K * (2 if self.pairwise else 1)

    @property
    def operand_bytes(self) -> int:
        """Bytes per A / B element."""
        return 1 if self.in_dtype == "fp8_e4m3" else 2

    def algorithmic_bytes(self) -> int:
        """Each operand read once, the output written once, plus the 4-byte AMAX."""
        b = self.batch
        ob = self.operand_bytes
        nbytes = ob * b * self.M * self.K + ob * b * self.K * self.N
        if self.pairwise:
            nbytes += ob * b * self.K * self.N
        if self.has("bias"):
            nbytes += 2 * self.N
        if self.has("residual"):
            nbytes += 2 * b * self.M * self.N
        if self.has("act_grad"):
            nbytes += 2 * b * self.M * self.N
        if self.has("col_sum"):
            nbytes += 4 * self.N
        nbytes += (1 if self.out == "fp8_e4m3" else 2) * b * self.M * self.N
        if self.has("amax"):
            nbytes += 4
        return nbytes

    def with_shape(self, batch=None, M=None, N=None, K=None) -> "Workload":
        return dataclasses.replace(
            self,
            batch=self.batch if batch is None else batch,
            M=self.M if M is None else M,
            N=self.N if N is None else N,
            K=self.K if K is None else K,
        )


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload(
        name="c1", config_id=1, batch=1, M=256, N=256, K=256,
        chain=(("scale",), ("bias",), ("act", "gelu_tanh"), ("amax",)),
        alpha=0.5, bias_var=1.0,
        description="Y = GELU_tanh(0.5*A@B + bias), AMAX=max|Y|; M=N=K=256; A,B N(0,1/K); bias N(0,1)"),
    "c2": Workload(
        name="c2", config_id=2, batch=16, M=1024, N=1024, K=1024,
        chain=(("scale",), ("bias",), ("act", "relu"), ("amax",)),
        alpha=1.25, bias_var=0.1,
        description="batch 16 x 1024^3, alpha=1.25, per-column bias N(0,0.1), ReLU, AMAX over all outputs"),
    "c3": Workload(
        name="c3", config_id=3, batch=1, M=8192, N=11008, K=4096,
        chain=(("pairwise", "silu"),),
        a_var="1", b_var="1/K",
        description="SwiGLU up-projection: SiLU(X@Wg)*(X@Wu), X[8192x4096] N(0,1), W[4096x11008] N(0,1/4096)"),
    "c4": Workload(
        name="c4", config_id=4, batch=1, M=8192, N=4096, K=4096,
        chain=(("row_rms", 1e-6), ("residual",)),
        a_var="1", b_var="1/K",
        description="RMS row scale of X[8192x4096] (gain U(0.5,1.5) folded into W), plus residual R N(0,1)"),
    "c5": Workload(
        name="c5", config_id=5, batch=1, M=8192, N=8192, K=8192,
        chain=(("bias",), ("act", "gelu_tanh"), ("amax",), ("quant_fp8",)),
        quant_scale=448.0 / 4.0, bias_var=0.1, out="fp8_e4m3",
        description="M=N=K=8192, bias N(0,0.1), GELU_tanh, fp8 e4m3 output with scale 112 and fp32 AMAX"),
}

# Beyond the five configurations: the RMSNorm-MLP of the superoptimizer write-up (section 10),
# the row RMS statistic feeding the pairwise product with no activation, out = up * gate, at
# the SwiGLU shapes.
WORKLOADS["f1"] = Workload(
    name="f1", config_id=6, batch=1, M=8192, N=11008, K=4096,
    chain=(("row_rms", 1e-6), ("pairwise", "none")),
    a_var="1", b_var="1/K",
    description="RMSNorm-MLP: (S*X@Wg')*(S*X@Wu'), S = 1/rms(X), gain U(0.5,1.5) folded into Wg and Wu, "
                "X[8192x4096] N(0,1), W[4096x11008] N(0,1/4096), no activation")

# The backward-pass epilogue (CODA news item, "How CODA works": forward and backward): for a
# GELU MLP layer H = GELU(Z1), Y = H @ W2 with W2 stored [hidden][d], the gradient step
# dZ1 = (dY @ W2^T) * GELU'(Z1) with the bias gradient db1 = sum over rows of dZ1, in one
# kernel: A = dY [8192 x 4096], B = W2 stored [N = 11008][K = 4096] (the [N][K] layout),
# Z = Z1 [8192 x 11008].
WORKLOADS["f2"] = Workload(
    name="f2", config_id=7, batch=1, M=8192, N=11008, K=4096,
    chain=(("act_grad", "gelu_tanh"), ("col_sum",)),
    a_var="1", b_var="1/K", b_layout="nk",
    description="MLP backward: dZ1 = (dY@W2^T)*GELU'(Z1), db1 = colsum(dZ1); dY[8192x4096] N(0,1), "
                "W2 stored [11008x4096] N(0,1/4096), Z1 N(0,1)")

# fp8 operands with delayed scaling (cuDNN tutorial, batched-matmul paragraph: the AMAX of
# one pass sets the fp8 scale of the next): the large fp8-output GEMM of c5 fed with fp8
# operands, X ~ N(0, 1) quantised with the scale 448/4 = 112 that c5's output uses, W ~
# N(0, 1/K) stored [N][K] and quantised with 4096; alpha = 1/(112*4096) dequantises the
# accumulator, then bias, GELU-tanh, AMAX and the fp8 output with scale 112.
WORKLOADS["f3"] = Workload(
    name="f3", config_id=8, batch=1, M=8192, N=8192, K=8192,
    chain=(("scale",), ("bias",), ("act", "gelu_tanh"), ("amax",), ("quant_fp8",)),
    alpha=1.0 / (112.0 * 4096.0), quant_scale=448.0 / 4.0, bias_var=0.1, out="fp8_e4m3",
    a_var="1", b_var="1/K", b_layout="nk", in_dtype="fp8_e4m3", a_qscale=112.0, b_qscale=4096.0,
    description="fp8 operands: X[8192x8192] N(0,1) as e4m3 with scale 112, W stored [8192x8192] "
                "N(0,1/8192) as e4m3 with scale 4096; alpha=1/(112*4096), bias N(0,0.1), GELU_tanh, "
                "fp8 e4m3 output with scale 112 and fp32 AMAX")

CONFIG_ORDER: List[str] = ["c1", "c2", "c3", "c4", "c5"]


def _rng(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, tensor_id])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round-to-nearest-even (torch's cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_codes(x: np.ndarray, qscale: float) -> np.ndarray:
    """OCP e4m3 codes of clamp(x * qscale, -448, 448), round-to-nearest-even (torch's
    float32 -> float8_e4m3fn cast; the clamp keeps the cast away from its NaN overflow)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) * float(qscale)
    return t.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _normal_e4m3(config_id: int, tensor_id: int, shape, var: float, qscale: float) -> np.ndarray:
    z = _rng(config_id, tensor_id).standard_normal(size=shape, dtype=np.float32)
    z *= np.float32(math.sqrt(var))
    return f32_to_e4m3_codes(z, qscale)


def _fold(w_bits: np.ndarray, g: np.ndarray, layout: str = "kn") -> np.ndarray:
    """bf16(fp32(W[k, n]) * g[k]) for W stored [batch, K, N] ("kn") or [batch, N, K] ("nk")."""
    w_f32 = (w_bits.astype(np.uint32) << 16).view(np.float32)
    gk = g[None, :, None] if layout == "kn" else g[None, None, :]
    return f32_to_bf16_bits(w_f32 * gk)


def _normal_bf16(config_id: int, tensor_id: int, shape, var: float) -> np.ndarray:
    z = _rng(config_id, tensor_id).standard_normal(size=shape, dtype=np.float32)
    z *= np.float32(math.sqrt(var))
    return f32_to_bf16_bits(z)


def _var(spec: str, K: int) -> float:
    return 1.0 / max(K, 1) if spec == "1/K" else float(spec)


def generate(w: Workload, sensitive: bool = False, seed_offset: int = 0) -> Dict[str, np.ndarray]:
    """Seeded inputs for workload ``w``.

    Returns bf16 tensors as uint16 bit arrays, fp8 operands as uint8 e4m3 codes (A: [batch, M, K]; B, B2:
    [batch, K, N], or [batch, N, K] for b_layout "nk"; bias: [N]; R: [batch, M, N]) and float32 arrays for the
    gain ``g`` (RMS workload only).  ``sensitive=True`` draws A from N(0, 1)
    and sets the bias to zero, so the GEMM term dominates the output.
    ``seed_offset`` shifts the config id of every stream (extra seeds for the
    parity sweeps).
    """
    cid = w.config_id + 100 * seed_offset
    b, M, N, K = w.batch, w.M, w.N, w.K
    lay = w.b_layout
    bshape = (b, K, N) if lay == "kn" else (b, N, K)
    out: Dict[str, np.ndarray] = {}
    a_var = 1.0 if sensitive else _var(w.a_var, K)
    if w.in_dtype == "fp8_e4m3":
        # fp8 operands: uint8 codes; no gain fold, no pairwise (not defined for these workloads)
        out["A"] = _normal_e4m3(cid, T_A, (b, M, K), a_var, w.a_qscale)
        out["B"] = _normal_e4m3(cid, T_B, bshape, _var(w.b_var, K), w.b_qscale)
        if w.pairwise:
            out["B2"] = _normal_e4m3(cid, T_B2, bshape, _var(w.b_var, K), w.b_qscale)
        if w.has("bias"):
            out["bias"] = (np.zeros(N, dtype=np.uint16) if sensitive
                           else _normal_bf16(cid, T_BIAS, (N,), w.bias_var))
        if w.has("residual"):
            out["R"] = _normal_bf16(cid, T_R, (b, M, N), 1.0)
        return out
    out["A"] = _normal_bf16(cid, T_A, (b, M, K), a_var)
    g = None
    if w.has("row_rms"):
        # gain g[k] ~ U(0.5, 1.5) folded into the base weight(s) along the contraction axis
        g = _rng(cid, T_G).uniform(0.5, 1.5, size=K).astype(np.float32)
        w_base = _normal_bf16(cid, T_W, bshape, _var(w.b_var, K))
        out["g"] = g
        out["W_base"] = w_base
        out["B"] = _fold(w_base, g, lay)
    else:
        out["B"] = _normal_bf16(cid, T_B, bshape, _var(w.b_var, K))
    if w.pairwise:
        out["B2"] = _normal_bf16(cid, T_B2, bshape, _var(w.b_var, K))
        if g is not None:            # RMSNorm-MLP: the same gain scales X before both products
            out["W2_base"] = out["B2"]
            out["B2"] = _fold(out["B2"], g, lay)
    if w.has("bias"):
        if sensitive:
            out["bias"] = np.zeros(N, dtype=np.uint16)
        else:
            out["bias"] = _normal_bf16(cid, T_BIAS, (N,), w.bias_var)
    if w.has("residual"):
        out["R"] = _normal_bf16(cid, T_R, (b, M, N), 1.0)
    if w.has("act_grad"):
        # the saved pre-activation of the forward pass, N(0, 1)
        out["Z"] = _normal_bf16(cid, T_Z, (b, M, N), 1.0)
    return out
