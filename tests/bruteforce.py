"""Pure-Python brute force for tiny fused GEMM-epilogue problems.

Written independently of ``oracle/``: the GEMM is summed in exact rationals
(``fractions.Fraction``), the activations use ``math.tanh`` / ``math.exp``
directly, and the chain is walked element by element with scalar code.  Only
for tiny shapes (it is very slow).
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Optional, Sequence


def bf16_value(bits: int) -> float:
    """Value of a bf16 bit pattern, from its fields."""
    s = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return s * m * 2.0 ** -133
    if e == 0xFF:
        return s * math.inf if m == 0 else math.nan
    return s * (1.0 + m / 128.0) * 2.0 ** (e - 127)


def e4m3_value(code: int) -> float:
    """Value of an OCP e4m3 ("e4m3fn") code from its fields: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (step 2^-9); S.1111.111 is NaN, no infinities."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        return s * m * 2.0 ** -9
    if e == 0xF and m == 0x7:
        return math.nan
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def exact_gemm(A: Sequence[Sequence[float]], B: Sequence[Sequence[float]]) -> List[List[Fraction]]:
    M, K, N = len(A), len(A[0]) if A else 0, len(B[0]) if B else 0
    return [[sum((Fraction(A[m][k]) * Fraction(B[k][n]) for k in range(K)), Fraction(0))
             for n in range(N)] for m in range(M)]


def exact_gemm_nt(A: Sequence[Sequence[float]], Bt: Sequence[Sequence[float]]) -> List[List[Fraction]]:
    """acc[m][n] = sum_k A[m][k] * Bt[n][k] (B given transposed, [N][K])."""
    M, K, N = len(A), len(A[0]) if A else 0, len(Bt)
    return [[sum((Fraction(A[m][k]) * Fraction(Bt[n][k]) for k in range(K)), Fraction(0))
             for n in range(N)] for m in range(M)]


def act(x: float, name: str) -> float:
    if name == "none":
        return x
    if name == "relu":
        return x if x > 0 else 0.0
    if name == "gelu_tanh":
        return 0.5 * x * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))
    if name == "silu":
        return x * (1.0 / (1.0 + math.exp(-x))) if x > -700 else 0.0
    raise ValueError(name)


def act_derivative(z: float, name: str) -> float:
    """Derivative of ``act`` at z, each written from its textbook closed form."""
    if name == "none":
        return 1.0
    if name == "relu":
        return 1.0 if z > 0 else 0.0
    if name == "gelu_tanh":
        c = math.sqrt(2.0 / math.pi)
        u = c * (z + 0.044715 * z ** 3)
        return 0.5 * (1.0 + math.tanh(u)) + 0.5 * z * (1.0 / math.cosh(u)) ** 2 * c * (1.0 + 0.134145 * z * z)
    if name == "silu":
        sg = 1.0 / (1.0 + math.exp(-z))
        return sg + z * sg * (1.0 - sg)
    raise ValueError(name)


def run_chain_scalar(chain, A, B, B2=None, bias=None, R=None, alpha=1.0, b_layout="kn", Z=None) -> dict:
    """A: [batch][M][K] floats, B/B2: [batch][K][N] ([batch][N][K] for b_layout "nk");
    bias: [N]; R: [batch][M][N].

    Z: [batch][M][N] (ACT_GRAD).  Returns {"y": [batch][M][N] floats (before output
    encoding), "amax": float|None, "col_sum": [N] floats|None}.
    """
    kinds = [op[0] for op in chain]
    ys = []
    amax = 0.0
    for b in range(len(A)):
        mm = exact_gemm_nt if b_layout == "nk" else exact_gemm
        acc = mm(A[b], B[b])
        acc2 = mm(A[b], B2[b]) if "pairwise" in kinds else None
        M = len(A[b])
        N = len(acc[0]) if acc else 0
        K = len(A[b][0]) if M else 0
        rows = []
        for m in range(M):
            s = None
            for op in chain:
                if op[0] == "row_rms":
                    ss = sum(Fraction(a) * Fraction(a) for a in A[b][m])
                    s = 1.0 / math.sqrt(float(ss / K) + op[1])
            row = []
            for n in range(N):
                vals = [float(acc[m][n])] + ([float(acc2[m][n])] if acc2 is not None else [])
                out = None
                for op in chain:
                    if op[0] == "scale":
                        vals = [alpha * v for v in vals]
                    elif op[0] == "row_rms":
                        vals = [s * v for v in vals]
                    elif op[0] == "bias":
                        vals = [vals[0] + bias[n]] + vals[1:]
                    elif op[0] == "act":
                        vals = [act(vals[0], op[1])]
                    elif op[0] == "pairwise":
                        vals = [act(vals[0], op[1]) * vals[1]]
                    elif op[0] == "act_grad":
                        vals = [vals[0] * act_derivative(Z[b][m][n], op[1])]
                    elif op[0] == "residual":
                        vals = [vals[0] + R[b][m][n]]
                out = vals[0]
                amax = max(amax, abs(out))
                row.append(out)
            rows.append(row)
        ys.append(rows)
    col = None
    if "col_sum" in kinds:
        N = len(ys[0][0]) if ys and ys[0] else 0
        col = [math.fsum(ys[b][m][n] for b in range(len(ys)) for m in range(len(ys[b]))) for n in range(N)]
    return {"y": ys, "amax": amax if "amax" in kinds else None, "col_sum": col}
