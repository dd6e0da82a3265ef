"""GPU parity of the fp8-operand mainloop (e4m3 A and B, B given [N][K]) against the oracle.

The oracle decodes the same e4m3 codes exactly and runs the float64 GEMM and the literal
epilogue; the kernel multiplies the codes on the fp8 matrix cores with fp32 accumulation.
Covered: every tile shape with ragged M, N and K (K not a multiple of the 128-value LDS
slot takes the masked loads), the K edges, the pairwise tiles, a residual chain, padded
leading dimensions and the full-size workload in the benchmark's launch configuration.

Tolerance: bf16 outputs as everywhere (floored relative error 1e-2), fp8 outputs one code,
both widened per output by the allowance E of ``tests.parity.fp8_acc_bound``: the fp8
instruction does not sum its products exactly, and the model of it in
``tests/fp8_mfma_model.py`` (pinned to the instruction by ``test_fp8_mfma_model_gpu.py``)
gives how far its accumulator may stand from the exact dot product for these operands.  Each
test reports how many outputs needed the allowance; ``test_accumulator_follows_the_model``
checks the kernel's accumulator itself against the model, by cancellation.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import fp8_mfma_model
from tests.parity import (check_amax, check_bf16, check_fp8_interval, count_needing_allowance,
                          fp8_acc_bound)

pytestmark = pytest.mark.gpu

ge = pytest.importorskip("gemm_epilogue_transformer_tiled_amd")
from gemm_epilogue_transformer_tiled_amd import runner  # noqa: E402
from tests.test_parity_gpu import PAIR_TILES, SINGLE_TILES, TILE_NAMES, gpu_run  # noqa: E402

F3 = workloads.WORKLOADS["f3"]
# bf16-output variant of the same chain (no output quantisation)
F3_BF16 = dataclasses.replace(F3, out="bf16", chain=tuple(op for op in F3.chain if op[0] != "quant_fp8"))
RAGGED8 = dict(batch=2, M=300, N=264, K=208)


def acc_bound(w, inp, rows=None):
    """E[b, m, n] = |alpha| * (|T - X| + env) from the model of the fp8 instruction (float64)."""
    return fp8_acc_bound(inp["A"], inp["B"], w.alpha, rows=rows)


SLOPE = {"none": 1.0, "relu": 1.0, "gelu_tanh": 1.2, "silu": 1.2}   # >= max |act'|


def compare(w, inp, prob, what, rows=None):
    """Every output (or the outputs of `rows`) against the oracle, with the allowance."""
    ref = oracle.run_workload(w, inp, rows=rows)
    y = prob.y_host_bits()
    if rows is not None:
        y = y[:, rows, :]
    act = w.op("act")[1] if w.has("act") else ("none" if not w.pairwise else w.op("pairwise")[1])
    if w.out == "fp8_e4m3":
        # y = act(alpha * acc + bias): an accumulator error e moves y by at most slope * e
        assert [op[0] for op in w.chain if op[0] not in ("amax", "quant_fp8")] in (
            ["scale", "bias", "act"], ["scale", "act"], ["scale"]), w.chain
        e = SLOPE[act] * acc_bound(w, inp, rows)
        check_fp8_interval(y, ref.y - e, ref.y + e, w.quant_scale, what)
        needed = count_needing_allowance(y, ref.y, True, ref.codes)
    elif w.pairwise:
        check_bf16(y, ref.y, what)          # (passes without an allowance at these sizes)
        needed = 0
    else:
        # y = act(alpha * acc + bias) [+ R]: an accumulator error e moves y by at most slope * e
        check_bf16(y, ref.y, what, allow=SLOPE[act] * acc_bound(w, inp, rows))
        needed = count_needing_allowance(y, ref.y, False)
    print(f"\n{what}: {needed} of {y.size} outputs needed the fp8-accumulation allowance", flush=True)
    if w.has("amax") and rows is None:
        check_amax(prob.amax_host(), ref.amax, what)
    return ref


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("tile", SINGLE_TILES, ids=[TILE_NAMES[t] for t in SINGLE_TILES])
@pytest.mark.parametrize("w0", [F3, F3_BF16], ids=["fp8out", "bf16out"])
def test_ragged_every_tile(w0, tile):
    w = w0.with_shape(**RAGGED8)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp, tile)
    assert "in=fp8" in prob.plan.describe()
    compare(w, inp, prob, f"fp8 operands {w.out} tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("K", [0, 16, 112, 128, 144, 256, 1040])
@pytest.mark.parametrize("tile", [0, 3], ids=["256x256", "64x64"])
def test_k_edges(K, tile):
    w = F3_BF16.with_shape(batch=1, M=136, N=264, K=K)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp, tile), f"fp8 operands K={K} tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("tile", PAIR_TILES, ids=[TILE_NAMES[t] for t in PAIR_TILES])
def test_pairwise_tiles(tile):
    w = dataclasses.replace(F3, out="bf16", chain=(("scale",), ("pairwise", "silu"))).with_shape(**RAGGED8)
    inp = workloads.generate(w)
    assert inp["B2"].dtype == np.uint8
    compare(w, inp, gpu_run(w, inp, tile), f"fp8 operands pairwise tile {TILE_NAMES[tile]}")


def test_residual_chain():
    w = dataclasses.replace(F3, out="bf16",
                            chain=(("scale",), ("act", "relu"), ("residual",), ("amax",))).with_shape(**RAGGED8)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp), "fp8 operands relu + residual")


def test_padded_leading_dimensions():
    w = F3.with_shape(batch=1, M=256, N=264, K=400)
    inp = workloads.generate(w)
    lda, ldb = w.K + 48, w.K + 16
    Ap = np.zeros((1, w.M, lda), dtype=np.uint8)
    Ap[:, :, :w.K] = inp["A"]
    Bp = np.zeros((1, w.N, ldb), dtype=np.uint8)
    Bp[:, :, :w.K] = inp["B"]
    prob = runner.prepare(w, {**inp, "A": Ap, "B": Bp})
    desc = ge.make_desc(1, w.M, w.N, w.K, ge.make_ops(w.chain), y_type=ge.GE_DT_FP8_E4M3,
                        a_type=ge.GE_DT_FP8_E4M3, b_type=ge.GE_DT_FP8_E4M3, b_layout=ge.GE_LAYOUT_NK,
                        lda=lda, ldb=ldb)
    plan = ge.Plan(desc)
    args = ge.make_args(A=prob.tensors["A"], B=prob.tensors["B"], bias=prob.tensors["bias"], Y=prob.Y,
                        amax=prob.amax, alpha=w.alpha, quant_scale=w.quant_scale)
    plan.run(args)
    torch.cuda.synchronize()
    compare(w, inp, prob, "fp8 operands, padded lda/ldb")


# rows of the full-size check: both ends, and rows at every 32-row block position and several
# positions inside a block of the 256-row tile, spread over the tiles (and the eight XCDs)
FULL_ROWS = np.array([0, 1, 31, 32, 63, 100, 127, 128, 200, 255, 256, 777, 1023, 2047, 2200, 3001,
                      4095, 4100, 5000, 5555, 6143, 6200, 7000, 7424, 7680, 8000, 8064, 8128, 8190, 8191])


def test_full_workload():
    """M = N = K = 8192 in the benchmark's launch configuration: every output of 30 rows spread
    over the tiles against the oracle with the model's per-output allowance (the allowance
    costs ~0.4 s of host time per row), and AMAX over all outputs."""
    w = F3
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    print(f"\nf3: {prob.plan.describe()}", flush=True)
    assert "tile=256x256" in prob.plan.describe() and "in=fp8" in prob.plan.describe()
    compare(w, inp, prob, "f3 full, sampled rows", rows=FULL_ROWS)
    check_amax(prob.amax_host(), oracle.run_workload(w, inp).amax, "f3 full")


@pytest.mark.parametrize("K", [64, 1024, 8192])
def test_accumulator_follows_the_model(K):
    """The kernel's accumulator itself, by cancellation: chain (scale, residual) with the residual
    R = bf16(-alpha * X) from the oracle (X the exact dot product), so the output holds
    alpha * (acc_gpu - X) plus R's known rounding residue.  The model of the fp8 instruction
    predicts acc_gpu = T +- env (T the group-truncated sum): the output must lie within
    alpha * env (plus its own bf16 rounding) of alpha * T + R.  A kernel that drops, repeats or
    misplaces products, or accumulates in a different order of groups, lands outside; the
    error against the exact X is reported beside it."""
    M, N = (256, 1024) if K == 8192 else (512, 1024)
    w = dataclasses.replace(F3, chain=(("scale",), ("residual",)), out="bf16").with_shape(M=M, N=N, K=K)
    inp = workloads.generate(w)
    A = oracle.decode_e4m3(inp["A"])[0]
    B = oracle.decode_e4m3(inp["B"])[0]
    X = A @ B.T
    R = oracle.encode_bf16(-w.alpha * X)[None]
    r = oracle.decode_bf16(R)[0]
    prob = runner.prepare(w, {**inp, "R": R})
    prob.run()
    torch.cuda.synchronize()
    out = oracle.decode_bf16(prob.y_host_bits())[0]
    T, env = fp8_mfma_model.accumulation(A, B)
    model = w.alpha * T + r
    dev = np.abs(out - model)
    bound = w.alpha * env + 2.0 ** -24 * np.abs(w.alpha * T) + 2.0 ** -8 * np.abs(model) + 2.0 ** -133
    S = w.alpha * (np.abs(A) @ np.abs(B).T)
    print(f"\nK={K}: max |out - (alpha T + R)| / bound = {float((dev / bound).max()):.3f}; "
          f"max |alpha (acc - X)| / (alpha sum|ab|) = {float((np.abs(out - (w.alpha * X + r)) / S).max()):.3e}, "
          f"of which the model's truncation explains max {float((w.alpha * np.abs(T - X) / S).max()):.3e}",
          flush=True)
    assert np.all(dev <= bound), float((dev / bound).max())


def test_batched_with_broadcast_weight():
    """batch 3 with B's batch stride 0 (one weight for every batch), fp8 output and AMAX over
    all batches."""
    w = F3.with_shape(batch=3, M=200, N=136, K=272)
    inp = workloads.generate(w)
    inp = {**inp, "B": np.ascontiguousarray(np.broadcast_to(inp["B"][:1], inp["B"].shape))}
    prob = runner.prepare(w, {**inp, "B": inp["B"][:1]})
    desc = ge.make_desc(w.batch, w.M, w.N, w.K, ge.make_ops(w.chain), y_type=ge.GE_DT_FP8_E4M3,
                        a_type=ge.GE_DT_FP8_E4M3, b_type=ge.GE_DT_FP8_E4M3, b_layout=ge.GE_LAYOUT_NK,
                        stride_b=0)
    plan = ge.Plan(desc)
    args = ge.make_args(A=prob.tensors["A"], B=prob.tensors["B"], bias=prob.tensors["bias"], Y=prob.Y,
                        amax=prob.amax, alpha=w.alpha, quant_scale=w.quant_scale)
    plan.run(args)
    torch.cuda.synchronize()
    compare(w, inp, prob, "fp8 operands, broadcast B over 3 batches")


@pytest.mark.parametrize("shape", [dict(M=0), dict(N=0), dict(batch=0)], ids=["M0", "N0", "batch0"])
def test_empty_problem_zeroes_amax(shape):
    w = F3.with_shape(**{**dict(batch=1, M=64, N=64, K=128), **shape})
    inp = workloads.generate(w)
    prob = runner.prepare(w, inp)
    prob.run()
    torch.cuda.synchronize()
    assert prob.amax_host() == 0.0


@pytest.mark.parametrize("tile", [0, 2, 3], ids=["256x256", "128x128", "64x64"])
def test_requested_tile(tile):
    w = F3.with_shape(batch=1, M=264, N=200, K=336)
    inp = workloads.generate(w)
    prob = runner.prepare(w, inp, tile=tile)
    assert f"tile={TILE_NAMES[tile]}" in prob.plan.describe()
    prob.run()
    torch.cuda.synchronize()
    compare(w, inp, prob, f"fp8 operands requested tile {TILE_NAMES[tile]}")


def test_graph_replays_match_eager_runs():
    """fp8 operands replayed from a HIP graph (as the benchmark may): every replay, with eager
    work between replays, reproduces the eager output and AMAX bit for bit."""
    w = F3.with_shape(M=1024, N=2048, K=1024)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    compare(w, inp, prob, "f3 eager")
    y_eager, a_eager = prob.Y.clone(), prob.amax_host()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            prob.run()
    for rep in range(3):
        prob.Y.zero_()
        prob.amax.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(prob.Y, y_eager), f"replay {rep}"
        assert prob.amax_host() == a_eager, f"replay {rep}"
        prob.run()
        torch.cuda.synchronize()
        assert torch.equal(prob.Y, y_eager)


def test_fp8_output_feeds_the_next_layer():
    """Delayed scaling end to end: layer 1 (bf16 operands, c5's chain) writes e4m3 codes of
    y * 112 and its AMAX; layer 2 consumes such codes as its fp8 A operand, dequantised by
    alpha = 1 / (112 * scale_B).  Layer 1 is checked against the oracle; layer 2 runs on the
    oracle's layer-1 codes (oracle inputs never come from the kernel) and is checked against
    the oracle too, and the kernel's own layer-1 codes are the same codes within one step."""
    l1 = workloads.WORKLOADS["c5"].with_shape(batch=1, M=512, N=768, K=1024)
    in1 = workloads.generate(l1)
    p1 = gpu_run(l1, in1)
    ref1 = oracle.run_workload(l1, in1)
    from tests.parity import check_fp8
    check_fp8(p1.y_host_bits(), ref1.codes, "layer 1")
    check_amax(p1.amax_host(), ref1.amax, "layer 1")
    assert 448.0 / ref1.amax > 0                      # the next scale delayed scaling would use
    l2 = dataclasses.replace(F3, alpha=1.0 / (l1.quant_scale * F3.b_qscale)).with_shape(batch=1, M=512, N=640, K=768)
    in2 = workloads.generate(l2)
    in2 = {**in2, "A": ref1.codes}                    # layer 1's output, as the oracle encoded it
    assert in2["A"].shape == (1, l2.M, l2.K) and in2["A"].dtype == np.uint8
    p2 = gpu_run(l2, in2)
    compare(l2, in2, p2, "layer 2 on layer-1 codes")


# ---------------------------------------------------------------------------------------------
# Two-wave instances (8 waves, two per SIMD) with fp8 operands: K a multiple of 128 (one slot
# holds two 64-deep steps); K of 0, 1, 2, 3 and 5 slots covers whole and partial rings.
# ---------------------------------------------------------------------------------------------

TWO_WAVE8 = dict(batch=2, M=300, N=264, K=256)


def run_two_wave8(w, inp):
    prob = gpu_run(w, inp, 6 if w.pairwise else 5)
    assert "threads=512" in prob.plan.describe() and "in=fp8" in prob.plan.describe(), prob.plan.describe()
    return prob


@pytest.mark.parametrize("w0", [F3, F3_BF16], ids=["fp8out", "bf16out"])
def test_two_wave_ragged(w0):
    w = w0.with_shape(**TWO_WAVE8)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave8(w, inp), f"fp8 operands {w.out} two-wave")


@pytest.mark.parametrize("K", [0, 128, 256, 384, 640])
def test_two_wave_k_steps(K):
    w = F3_BF16.with_shape(batch=1, M=136, N=264, K=K)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave8(w, inp), f"fp8 operands two-wave K={K}")


def test_two_wave_pairwise_and_residual():
    w = dataclasses.replace(F3, out="bf16", chain=(("scale",), ("pairwise", "silu"))).with_shape(**TWO_WAVE8)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave8(w, inp), "fp8 operands pairwise two-wave")
    w = dataclasses.replace(F3, out="bf16",
                            chain=(("scale",), ("act", "relu"), ("residual",), ("amax",))).with_shape(**TWO_WAVE8)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave8(w, inp), "fp8 operands relu + residual two-wave")


def test_two_wave_refuses_k_not_a_multiple_of_128():
    ops = ge.make_ops((("scale",), ("act", "relu")))
    kw = dict(a_type=ge.GE_DT_FP8_E4M3, b_type=ge.GE_DT_FP8_E4M3, b_layout=ge.GE_LAYOUT_NK, tile=5)
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 256, ops, **kw)) == ge.GE_OK
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 192, ops, **kw)) == ge.GE_ERR_UNSUPPORTED


def test_two_wave_full_workload():
    w = F3
    inp = workloads.generate(w)
    prob = run_two_wave8(w, inp)
    compare(w, inp, prob, "f3 full two-wave, sampled rows", rows=FULL_ROWS)
    check_amax(prob.amax_host(), oracle.run_workload(w, inp).amax, "f3 full two-wave")
