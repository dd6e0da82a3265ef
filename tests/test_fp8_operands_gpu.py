"""GPU parity of the fp8-operand mainloop (e4m3 A and B, B given [N][K]) against the oracle.

The oracle decodes the same e4m3 codes exactly and runs the float64 GEMM and the literal
epilogue; the kernel multiplies the codes on the fp8 matrix cores with fp32 accumulation.
Covered: every tile shape with ragged M, N and K (K not a multiple of the 128-value LDS
slot takes the masked loads), the K edges, the pairwise tiles, a residual chain, padded
leading dimensions and the full-size workload in the benchmark's launch configuration.

Tolerance: bf16 outputs as everywhere (floored relative error 1e-2).  fp8 outputs use the
interval check of ``tests.parity.check_fp8_interval``: the fp8 instruction's accumulation is
less exact than fp32 (``test_accumulation_error_bound`` measures it by cancellation and holds
it to the bound E used there), so where the oracle's value sits within E of an e4m3 rounding
boundary -- outputs that nearly cancel against the bias -- the kernel's code may be one step
further away than the bf16-operand kernels' one-step rule allows.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import FP8_ACC_REL, check_amax, check_bf16, check_fp8_interval, fp8_acc_bound

pytestmark = pytest.mark.gpu

ge = pytest.importorskip("gemm_epilogue_transformer_tiled_amd")
from gemm_epilogue_transformer_tiled_amd import runner  # noqa: E402
from tests.test_parity_gpu import PAIR_TILES, SINGLE_TILES, TILE_NAMES, gpu_run  # noqa: E402

F3 = workloads.WORKLOADS["f3"]
# bf16-output variant of the same chain (no output quantisation)
F3_BF16 = dataclasses.replace(F3, out="bf16", chain=tuple(op for op in F3.chain if op[0] != "quant_fp8"))
RAGGED8 = dict(batch=2, M=300, N=264, K=208)


def acc_bound(w, inp):
    """E[b, m, n] = FP8_ACC_REL / sqrt(max(K, 64)) * alpha * sum_k |a_k b_k| (float64)."""
    return fp8_acc_bound(inp["A"], inp["B"], w.alpha, w.K)


SLOPE = {"none": 1.0, "relu": 1.0, "gelu_tanh": 1.2, "silu": 1.2}   # >= max |act'|


def compare(w, inp, prob, what):
    ref = oracle.run_workload(w, inp)
    y = prob.y_host_bits()
    if w.out == "fp8_e4m3":
        # y = act(alpha * acc + bias): an accumulator error e moves y by at most slope * e
        assert [op[0] for op in w.chain if op[0] not in ("amax", "quant_fp8")] in (
            ["scale", "bias", "act"], ["scale", "act"], ["scale"]), w.chain
        act = w.op("act")[1] if w.has("act") else "none"
        e = SLOPE[act] * acc_bound(w, inp)
        check_fp8_interval(y, ref.y - e, ref.y + e, w.quant_scale, what)
    elif w.pairwise:
        check_bf16(y, ref.y, what)          # (passes without an allowance at these sizes)
    else:
        # y = act(alpha * acc + bias) [+ R]: an accumulator error e moves y by at most slope * e
        act = w.op("act")[1] if w.has("act") else "none"
        check_bf16(y, ref.y, what, allow=SLOPE[act] * acc_bound(w, inp))
    if w.has("amax"):
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


def test_full_workload():
    """M = N = K = 8192 in the benchmark's launch configuration, every output checked."""
    w = F3
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    print(f"\nf3: {prob.plan.describe()}", flush=True)
    assert "tile=256x256" in prob.plan.describe() and "in=fp8" in prob.plan.describe()
    compare(w, inp, prob, "f3 full")


@pytest.mark.parametrize("K", [64, 1024, 8192])
def test_accumulation_error_bound(K):
    """The accumulator error itself, by cancellation: chain (scale, residual) with the residual
    R = bf16(-alpha * acc) from the oracle, so the bf16 output holds alpha * (acc_gpu - acc)
    plus R's known rounding residue.  Every |error| must stay within the bound E (the output's
    own bf16 rounding of the residue allowed for); the bf16-operand kernel on operands of the
    same distribution is measured alongside as the reference level."""
    w = dataclasses.replace(F3, chain=(("scale",), ("residual",)), out="bf16").with_shape(M=512, N=2048, K=K)
    inp = workloads.generate(w)
    A = oracle.decode_e4m3(inp["A"])
    B = oracle.decode_e4m3(inp["B"])
    y = w.alpha * np.matmul(A, np.swapaxes(B, -1, -2))
    R = oracle.encode_bf16(-y)
    exact = y + oracle.decode_bf16(R)                      # what an exact accumulator leaves
    prob = runner.prepare(w, {**inp, "R": R})
    prob.run()
    torch.cuda.synchronize()
    d = np.abs(oracle.decode_bf16(prob.y_host_bits()) - exact)
    E = acc_bound(w, inp)
    S = E / FP8_ACC_REL * np.sqrt(max(K, 64))
    print(f"\nK={K}: max |error| / (alpha sum|ab|) = {float((d / S).max()):.3e}, "
          f"bound {FP8_ACC_REL / np.sqrt(max(K, 64)):.3e}", flush=True)
    assert np.all(d <= (1 + 2.0 ** -8) * E + 2.0 ** -8 * np.abs(exact)), float((d / S).max())


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
