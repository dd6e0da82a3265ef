"""Number formats of the oracle: bf16 and OCP FP8 E4M3 (the "fn" variant).

Test infrastructure only (see the package docstring).

Both encoders round a float64 value *directly* to the target format with
round-to-nearest, ties-to-even, so there is no double rounding through
float32.  The method: for a finite ``|x|`` pick the quantum ``q`` of the
target format at that magnitude (``2**(floor(log2|x|) - p)`` with ``p`` the
stored mantissa bits, never below the subnormal quantum), then
``round_half_even(|x| / q) * q``.  Scaling by a power of two is exact in
float64, and ``numpy.rint`` rounds half to even, so the result is the
correctly rounded value.  When rounding carries into the next binade the
product is exactly that power of two, which is representable.

bf16: 8 exponent bits (bias 127), 7 stored mantissa bits; overflow -> inf.
E4M3 (OCP 8-bit float spec, e4m3fn): 4 exponent bits (bias 7), 3 stored
mantissa bits, largest finite 448, subnormal quantum 2**-9, no infinities,
NaN = S.1111.111.  The fp8 writer of the cuDNN tutorial's "FP8-style
epilogues" saturates: ``encode_e4m3`` clamps to +-448 before rounding.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")          # (2 - 2**-7) * 2**127
E4M3_MAX = 448.0                                 # 1.75 * 2**8
_BF16_MANT = 7
_BF16_MIN_QEXP = -133                            # subnormal quantum 2**-133
_E4M3_MANT = 3
_E4M3_MIN_QEXP = -9                              # subnormal quantum 2**-9
_E4M3_MIN_NORMAL_EXP = -6


def _round_to_format(ax: np.ndarray, mant_bits: int, min_qexp: int) -> np.ndarray:
    """Round non-negative finite float64 values to the format's grid (RNE)."""
    _, e = np.frexp(ax)                  # ax = f * 2**e with f in [0.5, 1): floor(log2 ax) = e - 1
    qexp = np.maximum(e - 1 - mant_bits, min_qexp)
    return np.ldexp(np.rint(np.ldexp(ax, -qexp)), qexp)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact: bf16 is the top half of float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):             # NaN payloads widen to NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round-to-nearest-even; overflow -> +-inf."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(ax)
    with np.errstate(invalid="ignore", over="ignore"):
        r = _round_to_format(np.where(finite, ax, 0.0), _BF16_MANT, _BF16_MIN_QEXP)
        r = np.where(r > BF16_MAX, np.inf, r)
        r = np.where(finite, r, ax)                      # inf stays inf, NaN stays NaN
        r = np.copysign(r, x)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    # canonical quiet NaN
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def _e4m3_table() -> np.ndarray:
    """Value of every E4M3 code, from the format's definition (NaN for S.1111.111)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** _E4M3_MIN_QEXP
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_VALUES = _e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float64 -> E4M3 codes: clamp to +-448, then round-to-nearest-even.

    NaN maps to 0x7F.  -0.0 maps to 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    ax = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    r = _round_to_format(ax, _E4M3_MANT, _E4M3_MIN_QEXP)
    # code fields from the rounded magnitude
    _, e = np.frexp(r)
    ex = e - 1                                            # floor(log2 r) for r > 0
    normal = (r > 0) & (ex >= _E4M3_MIN_NORMAL_EXP)
    mant_norm = np.where(normal, np.ldexp(r, -np.where(normal, ex, 0) + _E4M3_MANT), 0).astype(np.int64) - 8
    code_norm = ((ex + 7) << 3) + mant_norm
    code_sub = np.ldexp(r, -_E4M3_MIN_QEXP).astype(np.int64)   # 0..7 (0 for zero)
    mag = np.where(normal, code_norm, code_sub)
    sign = np.signbit(x).astype(np.int64) << 7
    codes = (sign | mag).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), codes).astype(np.uint8)
