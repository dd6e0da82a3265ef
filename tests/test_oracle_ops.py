"""Pins for the oracle's GEMM and epilogue primitives.

Every check compares the oracle with something other than itself: exact
rational brute force, closed forms and invariants fixed by the mathematics,
the superoptimizer write-up's exp2 form of SiLU with its printed constant,
and library special cases (torch's float64 gelu/silu/rms_norm/baddbmm).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ops
from tests.bruteforce import bf16_value, exact_gemm


def _bf16_array(rng, shape, scale=1.0):
    """Random bf16-representable float64 values (including powers of two and large magnitudes)."""
    x = rng.normal(0, scale, size=shape).astype(np.float32)
    bits = oracle.encode_bf16(x.astype(np.float64))
    return oracle.decode_bf16(bits)


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (4, 2, 64), (1, 1, 1), (5, 3, 33)])
def test_gemm_matches_exact_rationals(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = _bf16_array(rng, (M, K))
    B = _bf16_array(rng, (K, N))
    A[0, 0] = 2.0 ** 20
    B[0, 0] = -(2.0 ** -20)
    if K > 1:
        A[-1, -1] = 1.5 * 2.0 ** 60
    got = oracle.gemm(A[None], B[None])[0]
    ex = exact_gemm(A.tolist(), B.tolist())
    bound = K * 2.0 ** -53 * (np.abs(A) @ np.abs(B))
    for m in range(M):
        for n in range(N):
            assert abs(got[m, n] - float(ex[m][n])) <= bound[m, n] + 1e-300


def test_gemm_identity_zero_and_outer_product():
    rng = np.random.default_rng(1)
    B = _bf16_array(rng, (1, 6, 9))
    eye = np.eye(6)[None]
    assert np.array_equal(oracle.gemm(eye, B), B)
    assert np.array_equal(oracle.gemm(np.zeros((1, 4, 6)), B), np.zeros((1, 4, 9)))
    a = _bf16_array(rng, (1, 5, 1))
    b = _bf16_array(rng, (1, 1, 7))
    assert np.array_equal(oracle.gemm(a, b)[0], np.outer(a[0, :, 0], b[0, 0, :]))


def test_gemm_is_not_transposed_and_batches_are_independent():
    rng = np.random.default_rng(2)
    A = _bf16_array(rng, (3, 4, 5))
    B = _bf16_array(rng, (3, 5, 6))
    got = oracle.gemm(A, B)
    assert got.shape == (3, 4, 6)
    for b in range(3):
        ex = exact_gemm(A[b].tolist(), B[b].tolist())
        assert np.allclose(got[b], np.array(ex, dtype=np.float64), rtol=1e-14, atol=1e-14)
    # torch's baddbmm with beta=0, alpha=1 in float64 (the cuDNN tutorial's comparison chain)
    tb = torch.baddbmm(torch.zeros(3, 4, 6, dtype=torch.float64), torch.from_numpy(A),
                       torch.from_numpy(B).contiguous(), beta=0.0, alpha=1.0).numpy()
    assert np.allclose(got, tb, rtol=1e-14, atol=1e-14)


def test_scaling_by_half_is_exact():
    rng = np.random.default_rng(3)
    A = _bf16_array(rng, (1, 8, 16))
    B = _bf16_array(rng, (1, 16, 8))
    assert np.array_equal(oracle.gemm(0.5 * A, B), ops.scale(oracle.gemm(A, B), 0.5))


def test_gelu_tanh_closed_forms_and_torch():
    x = np.concatenate([np.linspace(-12, 12, 4801), np.array([0.0, 1e-8, -1e-8, 40.0, -40.0])])
    g = ops.gelu_tanh(x)
    assert ops.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(g - ops.gelu_tanh(-x), x, rtol=0, atol=1e-14)          # odd part is x
    assert abs(ops.gelu_tanh(np.array([40.0]))[0] - 40.0) < 1e-12               # -> x for large x
    assert abs(ops.gelu_tanh(np.array([-40.0]))[0]) < 1e-12                     # -> 0 for very negative x
    # tanh form equals the sigmoid form t * sigmoid(2u)
    u = math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)
    with np.errstate(over="ignore"):
        sig_form = x / (1 + np.exp(-2 * u))
    # 1 + tanh(u) cancels for very negative x, so the two forms agree absolutely there
    assert np.allclose(g, sig_form, rtol=1e-13, atol=1e-14)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-15)


def test_silu_closed_forms_page_exp2_form_and_torch():
    x = np.linspace(-30, 30, 6001)
    s = ops.silu(x)
    assert ops.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - ops.silu(-x), x, rtol=0, atol=1e-13)
    # the exp2 rewrite printed in the SwiGLU section, with its 9-digit log2(e)
    assert np.allclose(s, ops.silu_exp2_form(x), rtol=5e-8, atol=1e-12)
    assert abs(1.44269504 - 1 / math.log(2)) < 1e-8
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(s, ref, rtol=1e-14, atol=1e-15)


def test_relu_exact():
    x = np.array([-2.0, -0.0, 0.0, 1e-30, 3.5])
    assert np.array_equal(ops.relu(x), np.array([0.0, 0.0, 0.0, 1e-30, 3.5]))


def test_row_rms_constant_row_and_torch_rms_norm():
    c = 0.37
    X = np.full((1, 3, 64), c)
    s = ops.row_rms_scale(X, 1e-6)
    assert np.allclose(s, 1 / math.sqrt(c * c + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(4)
    X = _bf16_array(rng, (2, 5, 48))
    s = ops.row_rms_scale(X, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(X), (48,), eps=1e-6).numpy()
    assert np.allclose(X * s[..., None], ref, rtol=1e-13, atol=1e-15)
    with pytest.raises(ValueError):
        ops.row_rms_scale(np.zeros((1, 2, 0)), 1e-6)


def test_row_scale_rewrite_invariant():
    """(X * S) @ W == (X @ W) * S for a row-broadcast S (RMSNorm section's rewrite)."""
    rng = np.random.default_rng(5)
    X = _bf16_array(rng, (1, 7, 32))
    W = _bf16_array(rng, (1, 32, 9), 0.2)
    s = ops.row_rms_scale(X, 1e-6)
    lhs = oracle.gemm(X * s[..., None], W)
    rhs = ops.row_scale(oracle.gemm(X, W), s)
    assert np.allclose(lhs, rhs, rtol=1e-13, atol=1e-13)


def test_rms_fold_of_gain_matches_unfolded_norm():
    """rmsnorm(X)*g @ W  ==  s * (X @ (diag(g) W)) (up to W' rounding)."""
    rng = np.random.default_rng(6)
    K = 64
    X = _bf16_array(rng, (1, 6, K))
    W = _bf16_array(rng, (1, K, 10), 1 / 8)
    g = rng.uniform(0.5, 1.5, K)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(X), (K,), weight=torch.from_numpy(g), eps=1e-6)
    ref = (ref @ torch.from_numpy(W)).numpy()
    folded = ops.row_scale(oracle.gemm(X, g[None, :, None] * W), ops.row_rms_scale(X, 1e-6))
    assert np.allclose(folded, ref, rtol=1e-12, atol=1e-12)


def test_amax_and_permutation_invariance():
    rng = np.random.default_rng(8)
    y = rng.normal(size=(3, 5, 7))
    assert ops.amax(y) == np.abs(y).max()
    perm = rng.permutation(5)
    assert ops.amax(y[:, perm, :][::-1]) == ops.amax(y)
    assert ops.amax(np.zeros((0, 3))) == 0.0
    y[1, 2, 3] = -100.0
    assert ops.amax(y) == 100.0


def test_pairwise_and_residual():
    rng = np.random.default_rng(9)
    g = rng.normal(size=(2, 3))
    u = rng.normal(size=(2, 3))
    assert np.array_equal(ops.pairwise_act_mul(g, u, "none"), g * u)
    assert np.allclose(ops.pairwise_act_mul(g, u, "silu"), torch.nn.functional.silu(
        torch.from_numpy(g)).numpy() * u, rtol=1e-14)
    R = rng.normal(size=(2, 3))
    assert np.array_equal(ops.residual(np.zeros((2, 3)), R), R)


def test_quant_fp8_scales_then_clamps():
    y = np.array([0.0, 1.0, -1.0, 4.0, 5.0, -100.0, 1.0 / 112])
    codes = ops.quant_fp8(y, 112.0)
    vals = oracle.decode_e4m3(codes)
    assert list(vals[:6]) == [0.0, 112.0, -112.0, 448.0, 448.0, -448.0]
    assert vals[6] == 1.0


def test_bruteforce_bf16_decoder_agrees_with_field_definition():
    for bits in [0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4049, 0x0080]:
        assert bf16_value(bits) == oracle.decode_bf16(np.array([bits], dtype=np.uint16))[0]


@pytest.mark.parametrize("name", ["none", "relu", "gelu_tanh", "silu"])
def test_act_grad_matches_central_differences_of_the_activation(name):
    """act'(z) against (act(z+h) - act(z-h)) / 2h of the oracle's own activation (away from
    ReLU's kink): a dropped term or a wrong sign in the derivative shows up here."""
    z = np.concatenate([np.linspace(-6.0, -0.05, 60), np.linspace(0.05, 6.0, 60)])
    h = 1e-5
    fd = (ops.act(z + h, name) - ops.act(z - h, name)) / (2 * h)
    got = ops.act_grad(np.ones_like(z), z, name)
    assert np.allclose(got, fd, rtol=1e-6, atol=1e-9), np.abs(got - fd).max()


def test_act_grad_special_values_and_torch_autograd():
    assert ops.gelu_tanh_grad(np.array([0.0]))[0] == 0.5
    assert ops.silu_grad(np.array([0.0]))[0] == 0.5
    assert list(ops.relu_grad(np.array([-1.0, 0.0, 2.0]))) == [0.0, 0.0, 1.0]
    assert abs(ops.gelu_tanh_grad(np.array([12.0]))[0] - 1.0) < 1e-12
    assert abs(ops.gelu_tanh_grad(np.array([-12.0]))[0]) < 1e-12
    assert abs(ops.silu_grad(np.array([40.0]))[0] - 1.0) < 1e-12
    # torch's float64 autograd of its own GELU (tanh approximation) and SiLU
    z = torch.linspace(-5, 5, 101, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(z, approximate="tanh").sum().backward()
    assert np.allclose(ops.gelu_tanh_grad(z.detach().numpy()), z.grad.numpy(), rtol=1e-12, atol=1e-14)
    z.grad = None
    torch.nn.functional.silu(z).sum().backward()
    assert np.allclose(ops.silu_grad(z.detach().numpy()), z.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_act_grad_multiplies_the_incoming_gradient():
    t = np.array([[[2.0, -3.0, 0.5]]])
    z = np.array([[[1.0, -1.0, 0.0]]])
    assert np.array_equal(ops.act_grad(t, z, "relu"), np.array([[[2.0, -0.0, 0.0]]]))
    assert np.array_equal(ops.act_grad(t, z, "none"), t)


def test_col_sum_over_rows_and_batches():
    y = np.arange(2 * 3 * 4, dtype=np.float64).reshape(2, 3, 4)
    want = [sum(y[b, m, n] for b in range(2) for m in range(3)) for n in range(4)]
    assert list(ops.col_sum(y)) == want
    assert list(ops.col_sum(np.zeros((1, 0, 5)))) == [0.0] * 5
    # a column of ones over M rows and B batches sums to M*B
    assert ops.col_sum(np.ones((3, 7, 2)))[1] == 21.0
