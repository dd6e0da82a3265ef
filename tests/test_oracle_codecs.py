"""Pins for the oracle's number formats (bf16, OCP E4M3), independent of the oracle.

Each check compares against something other than the oracle's own formula:
torch's float32 -> bf16 / float8_e4m3fn casts (library special cases, both
round-to-nearest-even on float32 inputs), brute-force nearest-value search
over the 256-entry code table, and directed float64 cases whose correct
rounding is fixed by arithmetic.
"""
import numpy as np
import pytest
import torch

from oracle import BF16_MAX, decode_bf16, decode_e4m3, encode_bf16, encode_e4m3


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_decode_bf16_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("low_kind", ["fixed", "random"])
def test_encode_bf16_matches_torch_on_float32_inputs(low_kind):
    """Every float32 high half with low halves at the rounding boundaries (and random ones)."""
    hi = np.arange(1 << 16, dtype=np.uint32)
    if low_kind == "fixed":
        lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    else:
        lows = np.random.default_rng(7).integers(0, 1 << 16, size=24, dtype=np.uint32)
    pat = ((hi[:, None] << 16) | lows[None, :]).ravel()
    x32 = pat.view(np.float32)
    finite = np.isfinite(x32)
    with np.errstate(invalid="ignore"):
        ours = encode_bf16(x32.astype(np.float64))
    ref = _torch_bf16_bits(x32)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.all(np.isnan(decode_bf16(ours[np.isnan(x32)])))


def test_encode_bf16_directed_float64_cases():
    one = 1.0
    cases = [
        (one + 2.0 ** -8, one),                          # exact tie -> even (1.0)
        (one + 3 * 2.0 ** -8, one + 2.0 ** -6),          # exact tie -> even (mantissa 2)
        (one + 2.0 ** -8 + 2.0 ** -40, one + 2.0 ** -7),  # just above the tie: a float32 detour would tie to 1.0
        (one + 2.0 ** -8 - 2.0 ** -40, one),
        (BF16_MAX, BF16_MAX),
        (BF16_MAX + 2.0 ** 119, np.inf),                 # max + half ulp: tie to even overflows
        (BF16_MAX + 2.0 ** 119 - 2.0 ** 80, BF16_MAX),
        (2.0 ** -133, 2.0 ** -133),                      # smallest subnormal
        (2.0 ** -134, 0.0),                              # half of it: tie -> even (0)
        (0.75 * 2.0 ** -133, 2.0 ** -133),
        (1.5 * 2.0 ** -133, 2.0 ** -132),                # tie between 1 and 2 quanta -> 2
        (-0.0, -0.0),
        (-(one + 2.0 ** -7), -(one + 2.0 ** -7)),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    got = decode_bf16(encode_bf16(x))
    assert np.array_equal(got, want), list(zip(x, got, want))
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_bf16_round_trip_every_finite_code():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = decode_bf16(bits)
    fin = np.isfinite(v)
    assert np.array_equal(encode_bf16(v[fin]), bits[fin])


def test_decode_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0 and ours[0x01] == 2.0 ** -9


def _brute_force_e4m3(x: float) -> int:
    """Nearest finite code by exhaustive search; ties to the even code; |x| > 448 saturates."""
    vals = decode_e4m3(np.arange(256, dtype=np.uint8))
    x = min(max(x, -448.0), 448.0)
    best, best_d = None, None
    for c in range(256):
        v = vals[c]
        if np.isnan(v):
            continue
        if v == 0.0 and (c == 0x80) != bool(np.signbit(x)):
            continue                                      # keep the sign of zero
        d = abs(v - x)
        if best is None or d < best_d or (d == best_d and (c & 1) == 0 and (best & 1) == 1):
            best, best_d = c, d
    return best


def test_encode_e4m3_brute_force_nearest():
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        rng.normal(0, 60, 400), rng.normal(0, 0.01, 200), rng.uniform(-600, 600, 200),
        np.array([0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 465.0, 1e9, -1e9, 2.0 ** -10, 2.0 ** -9 * 0.5,
                  2.0 ** -9 * 1.5, 2.0 ** -9 * 2.5, 240.0, 248.0, 232.0]),
    ])
    got = encode_e4m3(xs)
    want = np.array([_brute_force_e4m3(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want), [(x, g, w) for x, g, w in zip(xs, got, want) if g != w][:10]


def test_encode_e4m3_midpoints_tie_to_even():
    vals = decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))   # non-negative finite codes, increasing
    mids = (vals[:-1] + vals[1:]) / 2
    got = encode_e4m3(mids)
    lo = np.arange(0, 0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(encode_e4m3(-mids), want | 0x80)


def test_encode_e4m3_matches_torch_after_clamp():
    rng = np.random.default_rng(3)
    grid = np.concatenate([np.linspace(-512, 512, 200001), rng.normal(0, 30, 100000)]).astype(np.float32)
    clamped = np.clip(grid, -448, 448)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = encode_e4m3(grid.astype(np.float64))
    # torch keeps the sign of a zero result; so do we
    assert np.array_equal(ours, ref)


def test_encode_e4m3_saturates_and_round_trips():
    assert encode_e4m3(np.array([1e6]))[0] == 0x7E
    assert encode_e4m3(np.array([-1e6]))[0] == 0xFE
    assert encode_e4m3(np.array([np.nan]))[0] == 0x7F
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)
