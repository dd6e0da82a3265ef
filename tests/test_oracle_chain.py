"""Pins for the oracle's chain evaluation, plus planted-mistake checks.

* Every workload's chain, on tiny shapes drawn by the real generator, is
  compared with the pure-Python brute force of ``tests/bruteforce.py``
  (exact-rational GEMM, scalar math-module epilogue).
* Degenerate cases whose answers are fixed: zero A, zero residual, K = 1.
* Planted mistakes: plausible bugs are patched into the oracle (on the CPU)
  and at least one pin must then fail.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
import workloads
from oracle import chain as oracle_chain
from oracle import ops
from tests.bruteforce import e4m3_value, run_chain_scalar

TINY = dict(batch=2, M=3, N=5, K=16)


def _tiny(name, **kw):
    shape = dict(TINY)
    shape.update(kw)
    w = workloads.WORKLOADS[name].with_shape(**shape)
    return w, workloads.generate(w)


def _as_lists(inp, key):
    if key not in inp:
        return None
    if inp[key].dtype == np.uint8:          # fp8 operands: decoded from the code fields
        return np.vectorize(e4m3_value, otypes=[np.float64])(inp[key]).tolist()
    return oracle.decode_bf16(inp[key]).tolist()


def _check_against_bruteforce(w, inp):
    res = oracle.run_workload(w, inp)
    bias = oracle.decode_bf16(inp["bias"]).tolist() if "bias" in inp else None
    ref = run_chain_scalar(w.chain, _as_lists(inp, "A"), _as_lists(inp, "B"), _as_lists(inp, "B2"),
                           bias, _as_lists(inp, "R"), alpha=w.alpha, b_layout=w.b_layout,
                           Z=_as_lists(inp, "Z"))
    y_ref = np.array(ref["y"], dtype=np.float64)
    assert res.y.shape == y_ref.shape
    assert np.allclose(res.y, y_ref, rtol=1e-12, atol=1e-13), np.abs(res.y - y_ref).max()
    if w.has("amax"):
        assert math.isclose(res.amax, ref["amax"], rel_tol=1e-12)
        assert res.amax == np.abs(res.y).max()
    if w.has("col_sum"):
        assert np.allclose(res.col_sum, np.array(ref["col_sum"]), rtol=1e-12, atol=1e-12)
    else:
        assert res.col_sum is None
    if w.out == "fp8_e4m3":
        assert res.codes.dtype == np.uint8
        want = oracle.encode_e4m3(np.clip(y_ref * w.quant_scale, -448, 448))
        assert np.array_equal(res.codes, want)
    else:
        assert np.array_equal(res.codes, oracle.encode_bf16(y_ref))


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_chain_matches_bruteforce(name):
    w, inp = _tiny(name)
    _check_against_bruteforce(w, inp)


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER + ["f1"])
def test_nk_layout_matches_bruteforce(name):
    """B stored [N][K]: the product is A @ B^T (brute force indexes B[n][k] directly)."""
    w = dataclasses.replace(workloads.WORKLOADS[name], b_layout="nk").with_shape(**TINY)
    inp = workloads.generate(w)
    assert inp["B"].shape == (w.batch, w.N, w.K)
    _check_against_bruteforce(w, inp)


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_chain_sensitive_inputs_match_bruteforce(name):
    w = workloads.WORKLOADS[name].with_shape(**TINY)
    inp = workloads.generate(w, sensitive=True)
    assert not inp["bias"].any()
    _check_against_bruteforce(w, inp)


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_zero_A_gives_activation_of_bias(name):
    w, inp = _tiny(name)
    inp["A"] = np.zeros_like(inp["A"])
    res = oracle.run_workload(w, inp)
    act_name = w.op("act")[1]
    fb = ops.act(oracle.decode_bf16(inp["bias"]), act_name)
    assert np.array_equal(res.y, np.broadcast_to(fb, res.y.shape))
    assert res.amax == np.abs(fb).max()


def test_residual_reductions():
    w, inp = _tiny("c4")
    with_r = oracle.run_workload(w, inp)
    inp0 = dict(inp)
    inp0["R"] = np.zeros_like(inp["R"])
    no_r = oracle.run_workload(w, inp0)
    assert np.allclose(with_r.y - oracle.decode_bf16(inp["R"]), no_r.y, rtol=0, atol=1e-14)
    A = oracle.decode_bf16(inp["A"])
    s = ops.row_rms_scale(A, 1e-6)
    assert np.allclose(no_r.y, s[..., None] * oracle.gemm(A, oracle.decode_bf16(inp["B"])), rtol=1e-14)


def test_row_subset_matches_full():
    w, inp = _tiny("c4", M=9)
    full = oracle.run_workload(w, inp)
    rows = np.array([0, 4, 8])
    part = oracle.run_workload(w, inp, rows=rows)
    assert np.array_equal(part.y, full.y[:, rows, :])
    assert np.array_equal(part.codes, full.codes[:, rows, :])


def test_k_equals_one_outer_product():
    w, inp = _tiny("c2", K=1)
    _check_against_bruteforce(w, inp)


# ----------------------------------------------------------------------------------------------
# Planted mistakes: each patch is a plausible bug; the brute-force pins must notice it.
# ----------------------------------------------------------------------------------------------

def _gemm_transposed_b(A, B):
    return np.matmul(np.asarray(A, np.float64), np.swapaxes(np.asarray(B, np.float64), -1, -2))


def _gelu_wrong_cubic_sign(t):
    t = np.asarray(t, dtype=np.float64)
    return 0.5 * t * (1.0 + np.tanh(math.sqrt(2 / math.pi) * (t - 0.044715 * t ** 3)))


def _silu_wrong_sign(t):
    return np.asarray(t, np.float64) / (1.0 + np.exp(np.asarray(t, np.float64)))


def _rms_sum_not_mean(X, eps):
    X = np.asarray(X, dtype=np.float64)
    return 1.0 / np.sqrt(np.sum(X * X, axis=-1) + eps)


def _bias_dropped(t, bias):
    return t


def _amax_signed(y):
    return float(np.max(y))


MUTANTS = [
    ("gemm", _gemm_transposed_b, "c1", dict(M=5, N=5, K=5)),
    ("gelu_tanh", _gelu_wrong_cubic_sign, "c1", {}),
    ("silu", _silu_wrong_sign, "c3", {}),
    ("row_rms_scale", _rms_sum_not_mean, "c4", {}),
    ("bias_col", _bias_dropped, "c2", {}),
    ("amax", _amax_signed, "c5", {}),
]


@pytest.mark.parametrize("attr,mutant,name,shape", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, attr, mutant, name, shape):
    w, inp = _tiny(name, **shape)
    if attr == "amax":
        inp["B"] = np.where(inp["B"] < 0x8000, inp["B"] | 0x8000, inp["B"] & 0x7FFF).astype(np.uint16)
    monkeypatch.setattr(ops, attr, mutant)
    if attr in ("silu", "gelu_tanh"):
        monkeypatch.setitem(ops._ACTS, attr, mutant)
    monkeypatch.setattr(oracle_chain, "ops", ops)
    with pytest.raises(AssertionError):
        _check_against_bruteforce(w, inp)


def test_planted_e4m3_truncation_is_caught(monkeypatch):
    from oracle import codecs

    def trunc_round(ax, mant_bits, min_qexp):
        _, e = np.frexp(ax)
        qexp = np.maximum(e - 1 - mant_bits, min_qexp)
        return np.ldexp(np.floor(np.ldexp(ax, -qexp)), qexp)

    monkeypatch.setattr(codecs, "_round_to_format", trunc_round)
    w, inp = _tiny("c5", M=8, N=16)
    with pytest.raises(AssertionError):
        res = oracle.run_workload(w, inp)
        from tests.test_oracle_codecs import _brute_force_e4m3
        y = res.y * w.quant_scale
        want = np.array([_brute_force_e4m3(float(v)) for v in y.ravel()], dtype=np.uint8)
        assert np.array_equal(res.codes.ravel(), want)


BACKWARD_CHAINS = [
    (("act_grad", "gelu_tanh"), ("col_sum",)),
    (("act_grad", "silu"), ("col_sum",)),
    (("act_grad", "relu"), ("residual",), ("col_sum",), ("amax",)),
    (("scale",), ("bias",), ("act_grad", "gelu_tanh"), ("col_sum",)),
    (("act", "relu"), ("col_sum",)),
]


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("chain", BACKWARD_CHAINS, ids=lambda c: "-".join(op[0] for op in c))
def test_backward_chains_match_bruteforce(chain, layout):
    w = dataclasses.replace(workloads.WORKLOADS["f2"], chain=chain, b_layout=layout, alpha=0.75,
                            bias_var=0.3).with_shape(batch=2, M=3, N=5, K=16)
    inp = workloads.generate(w)
    assert ("Z" in inp) == w.has("act_grad")
    _check_against_bruteforce(w, inp)


# ---- fp8 operands (delayed scaling) ----

FP8_TINY = dict(batch=2, M=3, N=5, K=32)


@pytest.mark.parametrize("out", ["fp8_e4m3", "bf16"])
def test_fp8_operands_match_bruteforce(out):
    """e4m3 operand codes decoded from their fields by the brute force; the chain of the
    fp8-operand workload (alpha dequantises, then bias, GELU, AMAX, output)."""
    w = dataclasses.replace(workloads.WORKLOADS["f3"], out=out,
                            chain=tuple(op for op in workloads.WORKLOADS["f3"].chain
                                        if out == "fp8_e4m3" or op[0] != "quant_fp8")).with_shape(**FP8_TINY)
    inp = workloads.generate(w)
    assert inp["A"].dtype == np.uint8 and inp["B"].dtype == np.uint8
    assert inp["B"].shape == (w.batch, w.N, w.K)
    _check_against_bruteforce(w, inp)


def test_fp8_operands_pairwise_and_residual_match_bruteforce():
    base = workloads.WORKLOADS["f3"]
    for chain in ((("scale",), ("pairwise", "silu")), (("scale",), ("act", "relu"), ("residual",), ("amax",))):
        w = dataclasses.replace(base, chain=chain, out="bf16").with_shape(**FP8_TINY)
        _check_against_bruteforce(w, workloads.generate(w))


def test_fp8_operand_generator_codes():
    """Codes are finite e4m3 values (no NaN code) and decode to the clamped, scaled draws
    within half an e4m3 step (relative 2^-4, or the subnormal step 2^-10 absolute)."""
    w = workloads.WORKLOADS["f3"].with_shape(batch=1, M=64, N=48, K=256)
    inp = workloads.generate(w)
    for key, var, qs, shape in (("A", 1.0, w.a_qscale, (1, 64, 256)), ("B", 1.0 / 256, w.b_qscale, (1, 48, 256))):
        codes = inp[key]
        assert codes.dtype == np.uint8 and codes.shape == shape
        assert not np.any((codes & 0x7F) == 0x7F)
        tid = workloads.T_A if key == "A" else workloads.T_B
        z = workloads._rng(w.config_id, tid).standard_normal(size=shape, dtype=np.float32)
        x = np.clip((z * np.float32(math.sqrt(var))).astype(np.float64) * qs, -448, 448)
        got = np.vectorize(e4m3_value, otypes=[np.float64])(codes)
        assert np.all(np.abs(got - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def test_planted_fp8_operand_misdecode_is_caught(monkeypatch):
    """Reading fp8 operand codes as if they were the high byte of a bf16 value must fail."""
    w = dataclasses.replace(workloads.WORKLOADS["f3"], out="bf16",
                            chain=(("scale",), ("bias",), ("act", "gelu_tanh"), ("amax",))).with_shape(**FP8_TINY)
    inp = workloads.generate(w)
    monkeypatch.setattr(oracle_chain, "decode_operand",
                        lambda x: oracle.decode_bf16(x.astype(np.uint16) << 8) if x.dtype == np.uint8
                        else oracle.decode_bf16(x))
    with pytest.raises(AssertionError):
        _check_against_bruteforce(w, inp)
