"""The oracle's GEMM and epilogue primitives, each a plain full-array float64 pass.

Test infrastructure only (see the package docstring).  Inputs are float64
arrays; nothing here is blocked, fused or reordered.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import E4M3_MAX, encode_e4m3

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
_GELU_CUBIC = 0.044715


def gemm(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """acc[b, m, n] = sum_k A[b, m, k] * B[b, k, n] in float64.

    The product the superoptimizer write-up's section 8 (Matmul) computes,
    ``O = X @ W`` with W laid out [d, N] (the tile copy indexes W by
    ``[k*block_d, gx*block_n]``), and the batched matmul of the cuDNN
    tutorial.  numpy's float64 matmul is the library step; every bf16 product
    is exact in float64, so the only rounding is float64 summation.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if A.shape[-1] != B.shape[-2]:
        raise ValueError(f"contraction mismatch: A {A.shape} B {B.shape}")
    return np.matmul(A, B)


def scale(t: np.ndarray, alpha: float) -> np.ndarray:
    """Host-scalar alpha times the GEMM result (cuDNN tutorial, batched-matmul
    paragraph; the CODA 'scaling' primitive)."""
    return float(alpha) * t


def row_rms_scale(X: np.ndarray, eps: float) -> np.ndarray:
    """s[b, m] = 1 / sqrt(mean_k X[b, m, k]^2 + eps).

    Superoptimizer write-up, section 9 (RMSNorm): the per-row scale is the
    reciprocal square root of the mean of squares along the reduced axis d
    plus eps; its first generated kernel forms it as the row's running sum of
    squares divided by d.
    """
    X = np.asarray(X, dtype=np.float64)
    K = X.shape[-1]
    if K == 0:
        raise ValueError("RMS scale needs at least one element per row")
    ms = np.sum(X * X, axis=-1) / K
    return 1.0 / np.sqrt(ms + float(eps))


def row_scale(t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """t[b, m, n] * s[b, m]: the row-broadcast scale that the section-9 rewrite
    ``(X * S) @ W == (X @ W) * S`` moves behind the GEMM."""
    return t * np.asarray(s, dtype=np.float64)[..., :, None]


def bias_col(t: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """t + bias[n], the bias broadcast over rows and batches (TileLang tutorial's
    fused bias + GELU epilogue; cuDNN tutorial's per-column bias)."""
    return t + np.asarray(bias, dtype=np.float64)


def relu(t: np.ndarray) -> np.ndarray:
    """max(t, 0)."""
    return np.maximum(t, 0.0)


def gelu_tanh(t: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))).

    The pages name GELU without a formula (TileLang tutorial, fused epilogue
    paragraph); the workload names the tanh form, whose constants are the
    textbook ones of Hendrycks & Gimpel.
    """
    t = np.asarray(t, dtype=np.float64)
    return 0.5 * t * (1.0 + np.tanh(_SQRT_2_OVER_PI * (t + _GELU_CUBIC * t * t * t)))


def silu(t: np.ndarray) -> np.ndarray:
    """silu(x) = x * sigmoid(x) = x / (1 + e^-x) (superoptimizer write-up, section 7)."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def silu_exp2_form(t: np.ndarray, log2e: float = 1.44269504) -> np.ndarray:
    """The section-7 kernel's form of SiLU: x / (1 + 2^(-x * log2(e))), with the
    page's printed constant for log2(e).  Used only to pin ``silu``."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp2(-t * log2e))


_ACTS = {"none": lambda t: t, "relu": relu, "gelu_tanh": gelu_tanh, "silu": silu}


def act(t: np.ndarray, name: str) -> np.ndarray:
    """Apply the named activation (none, relu, gelu_tanh, silu)."""
    return _ACTS[name](t)


def relu_grad(z: np.ndarray) -> np.ndarray:
    """d relu / dz: 1 where z > 0, else 0 (0 at z = 0)."""
    return (np.asarray(z, dtype=np.float64) > 0.0).astype(np.float64)


def gelu_tanh_grad(z: np.ndarray) -> np.ndarray:
    """d/dz of 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3):
    0.5 (1 + tanh u) + 0.5 z (1 - tanh^2 u) sqrt(2/pi) (1 + 3 * 0.044715 z^2)."""
    z = np.asarray(z, dtype=np.float64)
    th = np.tanh(_SQRT_2_OVER_PI * (z + _GELU_CUBIC * z * z * z))
    return 0.5 * (1.0 + th) + 0.5 * z * (1.0 - th * th) * _SQRT_2_OVER_PI * (1.0 + 3.0 * _GELU_CUBIC * z * z)


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz of z sigmoid(z): sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


_ACT_GRADS = {"none": lambda z: np.ones_like(np.asarray(z, dtype=np.float64)), "relu": relu_grad,
              "gelu_tanh": gelu_tanh_grad, "silu": silu_grad}


def act_grad(t: np.ndarray, z: np.ndarray, name: str) -> np.ndarray:
    """Backward epilogue: t * act'(z), z the saved pre-activation -- the activation-gradient
    step of a backward pass (CODA news item, "How CODA works": epilogues for the forward
    and the backward pass), dZ = (dY @ W^T) * act'(Z)."""
    return np.asarray(t, dtype=np.float64) * _ACT_GRADS[name](z)


def col_sum(y: np.ndarray) -> np.ndarray:
    """s[n] = sum over batches and rows of y[b, m, n] -- the column reduction that gives a
    bias gradient (CODA news item, "How CODA works": the reductions primitive)."""
    y = np.asarray(y, dtype=np.float64)
    return y.reshape(-1, y.shape[-1]).sum(axis=0) if y.size else np.zeros(y.shape[-1])


def pairwise_act_mul(t_gate: np.ndarray, t_up: np.ndarray, name: str) -> np.ndarray:
    """out = act(gate) * up: the SwiGLU graph of section 7 (out = up * silu(gate))
    and, with no activation, the RMSNorm-MLP product of section 10."""
    return act(t_gate, name) * t_up


def residual(y: np.ndarray, R: np.ndarray) -> np.ndarray:
    """y + R (the CODA 'accumulation' primitive: a residual update)."""
    return y + np.asarray(R, dtype=np.float64)


def amax(y: np.ndarray) -> float:
    """max |y| over every output of every batch (cuDNN tutorial: the AMAX
    reduction on the result that sets the next fp8 scale).  0 for no outputs."""
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y))) if y.size else 0.0


def quant_fp8(y: np.ndarray, qscale: float) -> np.ndarray:
    """E4M3 codes of clamp(y * qscale, -448, 448), rounded to nearest even."""
    z = np.asarray(y, dtype=np.float64) * float(qscale)
    return encode_e4m3(np.clip(z, -E4M3_MAX, E4M3_MAX))
