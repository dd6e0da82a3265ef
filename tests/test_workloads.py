"""The seeded input generator: determinism, shapes and the distributions the workloads state."""
import numpy as np
import pytest

import oracle
import workloads


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_shapes_and_determinism(name):
    w = workloads.WORKLOADS[name].with_shape(batch=min(workloads.WORKLOADS[name].batch, 2), M=64, N=48, K=32)
    a = workloads.generate(w)
    b = workloads.generate(w)
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["A"].shape == (w.batch, 64, 32) and a["A"].dtype == np.uint16
    assert a["B"].shape == (w.batch, 32, 48)
    if w.pairwise:
        assert a["B2"].shape == a["B"].shape and not np.array_equal(a["B2"], a["B"])
    if w.has("bias"):
        assert a["bias"].shape == (48,)
    if w.has("residual"):
        assert a["R"].shape == (w.batch, 64, 48)
    c = workloads.generate(w, seed_offset=1)
    assert not np.array_equal(c["A"], a["A"])


def test_variances_follow_the_workload_text():
    w = workloads.WORKLOADS["c2"].with_shape(batch=2, M=256, N=256, K=1024)
    inp = workloads.generate(w)
    A = oracle.decode_bf16(inp["A"])
    assert abs(A.var() - 1 / 1024) < 0.05 / 1024
    assert abs(oracle.decode_bf16(inp["bias"]).var() - 0.1) < 0.03
    w3 = workloads.WORKLOADS["c3"].with_shape(M=256, N=512, K=512)
    inp3 = workloads.generate(w3)
    assert abs(oracle.decode_bf16(inp3["A"]).var() - 1.0) < 0.02
    assert abs(oracle.decode_bf16(inp3["B"]).var() * 512 - 1.0) < 0.02


def test_rms_fold_is_row_scaling_over_k():
    w = workloads.WORKLOADS["c4"].with_shape(M=8, N=16, K=32)
    inp = workloads.generate(w)
    g = inp["g"]
    assert g.min() >= 0.5 and g.max() < 1.5
    base = oracle.decode_bf16(inp["W_base"])[0]
    folded = oracle.decode_bf16(inp["B"])[0]
    ratio = folded / np.where(base == 0, 1, base)
    # every row k of W' is W's row k times g[k] (to bf16 rounding)
    assert np.allclose(ratio[base != 0], np.broadcast_to(g[:, None], base.shape)[base != 0], rtol=2 ** -7)


def test_rmsnorm_mlp_folds_the_gain_into_both_weights():
    w = workloads.WORKLOADS["f1"].with_shape(M=8, N=16, K=32)
    inp = workloads.generate(w)
    g = inp["g"]
    for base_key, key in (("W_base", "B"), ("W2_base", "B2")):
        base = oracle.decode_bf16(inp[base_key])[0]
        folded = oracle.decode_bf16(inp[key])[0]
        ratio = folded / np.where(base == 0, 1, base)
        assert np.allclose(ratio[base != 0], np.broadcast_to(g[:, None], base.shape)[base != 0], rtol=2 ** -7)
    assert not np.array_equal(inp["W_base"], inp["W2_base"])
    assert w.pairwise and w.op("pairwise")[1] == "none" and w.has("row_rms")


def test_flops_and_bytes_of_the_full_workloads():
    W = workloads.WORKLOADS
    assert W["c1"].flops() == 2 * 256 ** 3
    assert W["c3"].flops() == 2 * 2 * 8192 * 11008 * 4096
    assert W["c2"].algorithmic_bytes() == 100_665_348
    assert W["c3"].algorithmic_bytes() == 427_819_008
    assert W["c4"].algorithmic_bytes() == 234_881_024
    assert W["c5"].algorithmic_bytes() == 335_560_708
