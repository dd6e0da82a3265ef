"""GPU parity: the HIP path (through the C-ABI) against the float64 oracle.

Small ragged shapes on every kernel instance, the K / empty / stride edge
cases, the fp8 writer over every bf16 value in range, and each of the five
workloads at full size in the launch configuration the benchmark uses.
"""
import contextlib
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import check_amax, check_bf16, check_col_sum, check_fp8, fp8_acc_bound

pytestmark = pytest.mark.gpu

ge = pytest.importorskip("gemm_epilogue_transformer_tiled_amd")
from gemm_epilogue_transformer_tiled_amd import runner  # noqa: E402

TILE_NAMES = {0: "256x256", 1: "256x128p", 2: "128x128", 3: "64x64", 4: "128x128p", 5: "256x256", 6: "256x128p"}
SINGLE_TILES = [0, 2, 3]
PAIR_TILES = [1, 4]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    yield
    torch.cuda.synchronize()


@contextlib.contextmanager
def forced_tile(kind):
    old = os.environ.get("GE_FORCE_TILE")
    if kind is not None:
        os.environ["GE_FORCE_TILE"] = str(kind)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("GE_FORCE_TILE", None)
        else:
            os.environ["GE_FORCE_TILE"] = old


def gpu_run(w, inp, tile=None, y_fill=None):
    with forced_tile(tile):
        prob = runner.prepare(w, inp, y_fill=y_fill)
    prob.run()
    torch.cuda.synchronize()
    return prob


def compare(w, inp, prob, what, rows=None):
    ref = oracle.run_workload(w, inp, rows=rows)
    y = prob.y_host_bits()
    if rows is not None:
        y = y[:, rows, :]
    if w.out == "fp8_e4m3":
        check_fp8(y, ref.codes, what)
    else:
        check_bf16(y, ref.y, what)
    if w.has("amax") and rows is None:
        check_amax(prob.amax_host(), ref.amax, what)
    if w.has("col_sum") and rows is None:
        check_col_sum(prob.col_sum_host(), ref.col_sum, what)
    return ref


RAGGED = dict(batch=2, M=300, N=264, K=200)


def plan_tile(prob):
    """(rows, columns) of the kernel instance the plan chose, from its description."""
    bm, bn = prob.plan.describe().split("tile=")[1].split("x")[:2]
    return int(bm), int(bn)


def shares_row_statistic(w, prob):
    """Two-wave RMS plans with several tile columns share the row statistic along a tile row."""
    bm, bn = plan_tile(prob)
    return w.has("row_rms") and "threads=512" in prob.plan.describe() and -(-w.N // bn) > 1


def workspace_words(w, prob):
    """Word offsets of the plan's workspace, from the tile the plan actually chose: AMAX --
    nine ticket counters in words [0, 1024) and one slot per workgroup from word 1024; COL_SUM
    -- one ticket counter per column tile (16 words apart) from `cs_ctr`; a shared row
    statistic -- a flag and a counter per tile row (16 words apart) from `rs_ctr`; then the
    COL_SUM partials."""
    bm, bn = plan_tile(prob)
    tiles_m, tiles_n = -(-w.M // bm), -(-w.N // bn)
    wgs = tiles_m * tiles_n * w.batch
    round64 = lambda x: (x + 63) // 64 * 64
    cs_ctr = round64(1024 + wgs) if w.has("amax") else 0
    rs_ctr = round64(cs_ctr + tiles_n * 16) if w.has("col_sum") else cs_ctr
    rows = w.batch * tiles_m
    cs_part = round64(rs_ctr + rows * 16) if shares_row_statistic(w, prob) else rs_ctr
    return {"wgs": wgs, "tiles_m": tiles_m, "tiles_n": tiles_n, "cs_ctr": cs_ctr, "rs_ctr": rs_ctr,
            "rows": rows, "cs_part": cs_part}


def assert_counters_zero(w, prob, what=""):
    """Every ticket counter and flag the plan uses is back at zero (partials and slots may stay)."""
    if not (w.has("amax") or w.has("col_sum") or shares_row_statistic(w, prob)):
        assert prob.plan.workspace is None, f"{what}: a workspace without AMAX, COL_SUM or a shared statistic"
        return
    ws = prob.plan.workspace.view(torch.int32)
    lay = workspace_words(w, prob)
    if w.has("amax"):
        assert int(ws[:1024].count_nonzero()) == 0, f"{what}: AMAX counters"
    if w.has("col_sum"):
        ctr = ws[lay["cs_ctr"]: lay["cs_ctr"] + lay["tiles_n"] * 16]
        assert ctr.numel() == lay["tiles_n"] * 16
        assert int(ctr.count_nonzero()) == 0, f"{what}: column-tile counters"
    if shares_row_statistic(w, prob):
        ctr = ws[lay["rs_ctr"]: lay["rs_ctr"] + lay["rows"] * 16]
        assert ctr.numel() == lay["rows"] * 16
        assert int(ctr.count_nonzero()) == 0, f"{what}: tile-row flags and counters"


@pytest.mark.parametrize("tile", SINGLE_TILES, ids=[TILE_NAMES[t] for t in SINGLE_TILES])
@pytest.mark.parametrize("name", ["c1", "c2", "c4", "c5"])
def test_ragged_nk_every_tile(name, tile):
    """B given as [N][K] (the product A @ B^T), ragged in every dimension."""
    w = dataclasses.replace(workloads.WORKLOADS[name], b_layout="nk").with_shape(**RAGGED)
    inp = workloads.generate(w)
    assert inp["B"].shape == (w.batch, w.N, w.K)
    compare(w, inp, gpu_run(w, inp, tile), f"{name} nk tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("tile", PAIR_TILES, ids=[TILE_NAMES[t] for t in PAIR_TILES])
def test_ragged_nk_pairwise_tiles(tile):
    w = dataclasses.replace(workloads.WORKLOADS["c3"], b_layout="nk").with_shape(**RAGGED)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp, tile), f"c3 nk tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("K", [0, 8, 56, 64, 72, 136, 1032])
@pytest.mark.parametrize("tile", [0, 1, 3], ids=["256x256", "256x128p", "64x64"])
def test_k_edges_nk(K, tile):
    name = "c3" if tile == 1 else "c2"
    w = dataclasses.replace(workloads.WORKLOADS[name], b_layout="nk").with_shape(batch=1, M=136, N=264, K=K)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp, tile), f"{name} nk K={K} tile {TILE_NAMES[tile]}")


def test_nk_padded_leading_dimension_and_sensitive_inputs():
    w = dataclasses.replace(workloads.WORKLOADS["c5"], b_layout="nk").with_shape(batch=1, M=512, N=520, K=1000)
    inp = workloads.generate(w, sensitive=True)
    ldb = w.K + 24
    Bp = np.zeros((1, w.N, ldb), dtype=np.uint16)
    Bp[:, :, :w.K] = inp["B"]
    prob = runner.prepare(w, {**inp, "B": Bp})
    desc = ge.make_desc(1, w.M, w.N, w.K, ge.make_ops(w.chain), y_type=ge.GE_DT_FP8_E4M3,
                        b_layout=ge.GE_LAYOUT_NK, ldb=ldb)
    plan = ge.Plan(desc)
    args = ge.make_args(A=prob.tensors["A"], B=prob.tensors["B"], bias=prob.tensors["bias"], Y=prob.Y,
                        amax=prob.amax, quant_scale=w.quant_scale)
    plan.run(args)
    torch.cuda.synchronize()
    ref = oracle.run_workload(w, inp)
    check_fp8(prob.y_host_bits(), ref.codes, "nk padded ldb")
    check_amax(prob.amax_host(), ref.amax, "nk padded ldb")


@pytest.mark.parametrize("tile", SINGLE_TILES, ids=[TILE_NAMES[t] for t in SINGLE_TILES])
@pytest.mark.parametrize("name", ["c1", "c2", "c4", "c5"])
def test_ragged_every_tile(name, tile):
    w = workloads.WORKLOADS[name].with_shape(**RAGGED)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp, tile)
    bm, bn = TILE_NAMES[tile].rstrip("p").split("x")
    assert f"tile={bm}x{bn}x64" in prob.plan.describe()
    compare(w, inp, prob, f"{name} ragged tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("tile", PAIR_TILES, ids=[TILE_NAMES[t] for t in PAIR_TILES])
def test_ragged_pairwise_tiles(tile):
    w = workloads.WORKLOADS["c3"].with_shape(**RAGGED)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp, tile), f"c3 ragged tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("tile", SINGLE_TILES, ids=[TILE_NAMES[t] for t in SINGLE_TILES])
@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_sensitive_inputs_every_tile(name, tile):
    """bias = 0 and A ~ N(0, 1): the GEMM term dominates, so a wrong GEMM cannot hide behind the bias."""
    w = workloads.WORKLOADS[name].with_shape(batch=2, M=264, N=136, K=520)
    inp = workloads.generate(w, sensitive=True)
    compare(w, inp, gpu_run(w, inp, tile), f"{name} sensitive tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("K", [0, 8, 56, 64, 72, 128, 136, 1032])
@pytest.mark.parametrize("tile", [0, 3], ids=["256x256", "64x64"])
def test_k_edges(K, tile):
    w = workloads.WORKLOADS["c2"].with_shape(batch=1, M=136, N=72, K=K)
    inp = workloads.generate(w, sensitive=True)
    compare(w, inp, gpu_run(w, inp, tile), f"K={K}")


@pytest.mark.parametrize("K", [8, 64, 72, 200])
@pytest.mark.parametrize("tile", PAIR_TILES, ids=[TILE_NAMES[t] for t in PAIR_TILES])
def test_k_edges_pairwise(K, tile):
    w = workloads.WORKLOADS["c3"].with_shape(batch=1, M=72, N=136, K=K)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp, tile), f"pairwise K={K}")


@pytest.mark.parametrize("shape", [dict(M=0), dict(N=0), dict(batch=0)], ids=["M0", "N0", "batch0"])
def test_empty_problem_zeroes_amax_and_writes_nothing(shape):
    base = dict(batch=1, M=64, N=64, K=64)
    base.update(shape)
    w = workloads.WORKLOADS["c1"].with_shape(**base)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp, y_fill=0x5A)
    assert prob.amax_host() == 0.0
    assert bool((prob.Y.view(torch.uint8) == 0x5A).all())


def test_single_row_and_narrow_columns():
    w = workloads.WORKLOADS["c1"].with_shape(batch=1, M=1, N=8, K=64)
    inp = workloads.generate(w, sensitive=True)
    compare(w, inp, gpu_run(w, inp), "1x8")


def test_outputs_outside_the_problem_are_untouched():
    """Y is written exactly once inside [M, N]; padding columns of a wider ldy keep their bytes."""
    w = workloads.WORKLOADS["c2"].with_shape(batch=2, M=100, N=40, K=64)
    inp = workloads.generate(w)
    dev = "cuda"
    t = {k: runner.to_device_bf16(v, dev) for k, v in inp.items()}
    ldy = 56
    Y = torch.full((2, 100, ldy), 7.0, dtype=torch.bfloat16, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    desc = ge.make_desc(2, 100, 40, 64, ge.make_ops(w.chain), ldy=ldy)
    plan = ge.Plan(desc)
    plan.run(ge.make_args(A=t["A"], B=t["B"], bias=t["bias"], Y=Y, amax=amax, alpha=w.alpha))
    torch.cuda.synchronize()
    ref = oracle.run_workload(w, inp)
    ybits = Y.cpu().view(torch.int16).numpy().view(np.uint16)
    check_bf16(np.ascontiguousarray(ybits[:, :, :40]), ref.y, "ldy=56")
    assert np.all(oracle.decode_bf16(ybits[:, :, 40:]) == 7.0)
    check_amax(float(amax.item()), ref.amax, "ldy=56")


def test_strided_operands_and_broadcast_b():
    """lda > K, ldb > N and a batch stride of 0 on B (one weight shared by every batch)."""
    batch, M, N, K = 3, 96, 48, 80
    lda, ldb = 96, 64
    w = workloads.WORKLOADS["c2"].with_shape(batch=batch, M=M, N=N, K=K)
    inp = workloads.generate(w, sensitive=True)
    A_pad = np.zeros((batch, M, lda), dtype=np.uint16)
    A_pad[:, :, :K] = inp["A"]
    B_pad = np.zeros((1, K, ldb), dtype=np.uint16)
    B_pad[0, :, :N] = inp["B"][0]
    dev = "cuda"
    A = runner.to_device_bf16(A_pad, dev)
    B = runner.to_device_bf16(B_pad, dev)
    bias = runner.to_device_bf16(inp["bias"], dev)
    Y = torch.empty((batch, M, N), dtype=torch.bfloat16, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    desc = ge.make_desc(batch, M, N, K, ge.make_ops(w.chain), lda=lda, ldb=ldb, stride_b=0)
    plan = ge.Plan(desc)
    plan.run(ge.make_args(A=A, B=B, bias=bias, Y=Y, amax=amax, alpha=w.alpha))
    torch.cuda.synchronize()
    B_bcast = np.repeat(inp["B"][:1], batch, axis=0)
    ref = oracle.run_chain(w.chain, inp["A"], B_bcast, bias=inp["bias"], alpha=w.alpha)
    check_bf16(Y.cpu().view(torch.int16).numpy().view(np.uint16), ref.y, "strided")
    check_amax(float(amax.item()), ref.amax, "strided")


def test_external_row_scale_and_signed_amax():
    """ROW_SCALE from a caller vector, no activation, and an output whose largest magnitude is negative."""
    batch, M, N, K = 2, 130, 72, 96
    chain = (("scale",), ("row_scale",), ("bias",), ("residual",), ("amax",))
    w = workloads.Workload(name="rs", config_id=9, batch=batch, M=M, N=N, K=K, chain=chain, alpha=0.75)
    inp = workloads.generate(w)
    rng = np.random.default_rng(5)
    inp["row_scale"] = rng.uniform(0.5, 2.0, size=(batch, M)).astype(np.float32)
    inp["bias"][5] = 0xC2C8      # bf16 -100.0: the largest |y| sits in column 5 and is negative
    prob = gpu_run(w, inp)
    ref = oracle.run_workload(w, inp)
    check_bf16(prob.y_host_bits(), ref.y, "row_scale")
    assert ref.y.min() < -90
    check_amax(prob.amax_host(), ref.amax, "row_scale")


def test_rmsnorm_mlp_chain():
    """ROW_RMS with a pairwise product and no activation (the RMSNorm-MLP graph): s^2 * (X@Wu)(X@Wg)."""
    chain = (("row_rms", 1e-6), ("pairwise", "none"))
    w = workloads.Workload(name="rmsmlp", config_id=10, batch=1, M=272, N=136, K=256, chain=chain,
                           a_var="1", b_var="1/K")
    inp = workloads.generate(w)
    for tile in PAIR_TILES:
        compare(w, inp, gpu_run(w, inp, tile), f"rms-mlp tile {TILE_NAMES[tile]}")


def test_fp8_writer_over_every_bf16_value_in_range():
    """A = 0, so y = bias[n]: the E4M3 writer sees every bf16 value in [-512, 512] once, scale 1 and 1.37."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.decode_bf16(bits)
    sel = bits[np.isfinite(vals) & (np.abs(vals) <= 512)]
    N = ((len(sel) + 7) // 8) * 8
    bias = np.zeros(N, dtype=np.uint16)
    bias[:len(sel)] = sel
    for qs in (1.0, 1.37):
        w = workloads.Workload(name="fp8", config_id=11, batch=1, M=4, N=N, K=8,
                               chain=(("bias",), ("amax",), ("quant_fp8",)), quant_scale=qs, out="fp8_e4m3")
        inp = {"A": np.zeros((1, 4, 8), dtype=np.uint16), "B": np.zeros((1, 8, N), dtype=np.uint16), "bias": bias}
        prob = gpu_run(w, inp)
        ref = oracle.run_workload(w, inp)
        codes = prob.y_host_bits()
        check_fp8(codes, ref.codes, f"fp8 writer qs={qs}")
        if qs == 1.0:
            # y*1 is exact in fp32, so the writer's rounding alone decides the code: it must be RNE exactly
            mism = int((codes != ref.codes).sum())
            assert mism == 0, f"{mism} codes differ from round-to-nearest-even"
        check_amax(prob.amax_host(), ref.amax, "fp8 amax")


# ---------------------------------------------------------------------------------------------
# The five workloads at full size, in the benchmark's launch configuration.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", workloads.CONFIG_ORDER + ["f1", "f2"])
def test_full_workload(name):
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    print(f"\n{name}: {prob.plan.describe()}", flush=True)
    compare(w, inp, prob, f"{name} full")
    assert_counters_zero(w, prob, f"{name} full")


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_full_workload_sensitive(name):
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w, sensitive=True)
    compare(w, inp, gpu_run(w, inp), f"{name} full sensitive")


def test_nan_bias_gives_the_fp8_nan_code_and_a_nan_amax():
    """A NaN in the epilogue's input reaches the output as the OCP e4m3 NaN code 0x7F (the
    oracle's encoder) rather than a saturated +-448, and makes AMAX a NaN."""
    w = workloads.WORKLOADS["c5"].with_shape(M=300, N=264, K=256)
    inp = workloads.generate(w)
    bias = inp["bias"].copy()
    bias[7] = 0x7FC0                        # quiet NaN
    bias[200] = 0xFFC0                      # NaN with the sign bit set
    inp = {**inp, "bias": bias}
    prob = gpu_run(w, inp)
    ref = oracle.run_workload(w, inp)
    codes = prob.y_host_bits()
    nan = np.isnan(ref.y)
    assert nan[..., 7].all() and nan[..., 200].all() and int(nan.sum()) == 2 * w.M
    assert (ref.codes[nan] == 0x7F).all()
    assert (codes[nan] == 0x7F).all(), np.unique(codes[nan])
    check_fp8(codes[~nan], ref.codes[~nan], "finite outputs beside the NaN columns")
    assert np.isnan(ref.amax) and np.isnan(prob.amax_host())


def test_nan_residual_stays_nan_in_bf16():
    """A NaN residual element gives a NaN output element (bf16) and nothing else changes."""
    w = workloads.WORKLOADS["c4"].with_shape(M=300, N=264, K=256)
    inp = workloads.generate(w)
    r = inp["R"].copy()
    r[0, 17, 33] = 0x7FC0
    inp = {**inp, "R": r}
    prob = gpu_run(w, inp)
    ref = oracle.run_workload(w, inp)
    y = prob.y_host_bits()
    nan = np.isnan(ref.y)
    assert int(nan.sum()) == 1 and nan[0, 17, 33]
    assert np.isnan(oracle.decode_bf16(y[nan])).all()
    check_bf16(y[~nan], ref.y[~nan], "finite outputs beside the NaN")


def test_amax_workspace_is_left_zeroed_and_checked():
    w = workloads.WORKLOADS["c2"].with_shape(batch=2, M=512, N=512, K=256)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    assert prob.plan.workspace is not None
    # nine counters (1024 words) plus one slot per workgroup of the tile the plan chose
    assert prob.plan.workspace.numel() == 4 * (1024 + workspace_words(w, prob)["wgs"])
    # the ticket counters (first 4 KiB) are zero again after the run; slots hold partial maxima
    assert int(prob.plan.workspace[:4096].count_nonzero()) == 0
    ref = oracle.run_workload(w, inp)
    check_amax(prob.amax_host(), ref.amax, "first run")
    # a workspace smaller than gemm_epilogue_workspace_size is rejected before any launch
    args = ge.make_args(A=prob.tensors["A"], B=prob.tensors["B"], bias=prob.tensors["bias"], Y=prob.Y,
                        amax=prob.amax, alpha=w.alpha, workspace=prob.plan.workspace[:8])
    st = ge.gemm_epilogue_run(prob.plan.handle, args, torch.cuda.current_stream().cuda_stream)
    assert st == ge.GE_ERR_INVALID_ARG


def test_repeated_runs_are_identical_and_amax_is_overwritten():
    w = workloads.WORKLOADS["c2"]
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    y1, a1 = prob.Y.clone(), prob.amax_host()
    for _ in range(3):
        prob.run()
    torch.cuda.synchronize()
    assert torch.equal(prob.Y, y1)
    assert prob.amax_host() == a1


@pytest.mark.parametrize("name", ["c2", "c4", "c5", "f2"])
def test_graph_replays_match_eager_runs(name):
    """The benchmark replays the launches from a HIP graph: every replay, with eager work and
    synchronisation between replays, gives the eager output, AMAX and column sums, and leaves
    the ticket counters at zero."""
    w = workloads.WORKLOADS[name]
    if name == "c5":
        w = w.with_shape(M=1024, N=2048, K=1024)
    if name == "f2":
        w = w.with_shape(M=1024, N=1376, K=512)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    y_eager, a_eager = prob.Y.clone(), prob.amax_host()
    cs_eager = None if prob.col_sum is None else prob.col_sum.clone()
    compare(w, inp, prob, f"{name} eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            prob.run()
    for rep in range(3):
        prob.Y.zero_()
        if prob.amax is not None:
            prob.amax.fill_(-1.0)
        if prob.col_sum is not None:
            prob.col_sum.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(prob.Y, y_eager), f"replay {rep}"
        assert prob.amax_host() == a_eager, f"replay {rep}"
        if cs_eager is not None:
            assert torch.equal(prob.col_sum, cs_eager), f"replay {rep}"      # bit-identical
        assert_counters_zero(w, prob, f"replay {rep}")
        prob.run()                                  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(prob.Y, y_eager)



# ---------------------------------------------------------------------------------------------
# Backward-pass epilogues: activation gradient with the saved pre-activation, column sums.
# ---------------------------------------------------------------------------------------------

BACKWARD_CHAINS = [
    (("act_grad", "gelu_tanh"), ("col_sum",)),
    (("act_grad", "silu"), ("col_sum",)),
    (("act_grad", "relu"), ("residual",), ("col_sum",), ("amax",)),
    (("scale",), ("bias",), ("act_grad", "gelu_tanh"), ("col_sum",)),
    (("act_grad", "none"),),
    (("act", "relu"), ("col_sum",)),
]


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("tile", SINGLE_TILES, ids=[TILE_NAMES[t] for t in SINGLE_TILES])
@pytest.mark.parametrize("chain", BACKWARD_CHAINS, ids=lambda c: "-".join(op[0] + (op[1] if len(op) > 1 and isinstance(op[1], str) else "") for op in c))
def test_backward_chains_every_tile(chain, tile, layout):
    w = dataclasses.replace(workloads.WORKLOADS["f2"], chain=chain, b_layout=layout, alpha=0.75,
                            bias_var=0.3).with_shape(**RAGGED)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp, tile), f"backward {chain} tile {TILE_NAMES[tile]} {layout}")


@pytest.mark.parametrize("tile", PAIR_TILES, ids=[TILE_NAMES[t] for t in PAIR_TILES])
def test_col_sum_of_the_pairwise_product(tile):
    w = dataclasses.replace(workloads.WORKLOADS["c3"], chain=(("pairwise", "silu"), ("col_sum",))).with_shape(**RAGGED)
    inp = workloads.generate(w)
    compare(w, inp, gpu_run(w, inp, tile), f"pairwise col_sum tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("with_amax", [False, True], ids=["col_sum", "col_sum+amax"])
def test_col_sum_is_deterministic_and_leaves_the_workspace_zeroed(with_amax):
    w = workloads.WORKLOADS["f2"]
    if with_amax:
        w = dataclasses.replace(w, chain=w.chain + (("amax",),))
    w = w.with_shape(batch=2, M=1000, N=1032, K=512)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    first = prob.col_sum.clone()
    amax_first = prob.amax_host()
    compare(w, inp, prob, f"f2 batch 2{' + amax' if with_amax else ''}")
    assert_counters_zero(w, prob, "first run")
    for _ in range(3):
        prob.run()
    torch.cuda.synchronize()
    assert torch.equal(prob.col_sum, first)          # fixed summation order: bit-identical
    assert prob.amax_host() == amax_first
    assert_counters_zero(w, prob, "after repeats")


def test_col_sum_of_an_empty_problem_is_zero():
    w = dataclasses.replace(workloads.WORKLOADS["f2"]).with_shape(batch=1, M=0, N=264, K=64)
    inp = workloads.generate(w)
    prob = gpu_run(w, inp)
    assert float(prob.col_sum.abs().max().item()) == 0.0


def test_act_grad_rejects_fp8_output_and_row_rms():
    base = dict(batch=1, M=64, N=64, K=64)
    bad1 = ge.make_desc(ops=ge.make_ops([("act_grad", "gelu_tanh"), ("quant_fp8",)]), y_type=ge.GE_DT_FP8_E4M3, **base)
    bad2 = ge.make_desc(ops=ge.make_ops([("row_rms", 1e-6), ("act_grad", "gelu_tanh")]), **base)
    assert ge.gemm_epilogue_validate(bad1) == ge.GE_ERR_UNSUPPORTED
    assert ge.gemm_epilogue_validate(bad2) == ge.GE_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------------------------
# Largest supported operand: A's byte extent just under the 2**31 limit of the kernels' 32-bit
# buffer offsets, so the offsets of the last rows come closest to it (and the last row tile is
# ragged).  A is drawn on the GPU by torch's seeded generator (not by the HIP path); the sampled
# rows are copied back and checked against the oracle.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("in_dtype", ["bf16", "fp8_e4m3"])
def test_largest_supported_operand_extent(in_dtype):
    K, N = 4096, 256
    fp8 = in_dtype == "fp8_e4m3"
    # validate() admits (M + 255) * K + K + slot <= 2**31 - 16 elements times the element size
    M = 524024 if fp8 else 261880
    base = workloads.WORKLOADS["f3" if fp8 else "c2"]
    w = dataclasses.replace(base, chain=(("scale",), ("bias",), ("act", "relu")), out="bf16",
                            alpha=base.alpha if fp8 else 1.25).with_shape(batch=1, M=M, N=N, K=K)
    g = torch.Generator(device="cuda")
    g.manual_seed(20261203)
    A = torch.randn((1, M, K), generator=g, device="cuda", dtype=torch.float32)
    if fp8:
        A = (A * w.a_qscale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        A = A.to(torch.bfloat16)
    small = workloads.generate(w.with_shape(M=8))                 # B and bias from the generator
    prob = runner.prepare(w.with_shape(M=8), small)                # uploads B and bias
    desc = ge.make_desc(1, M, N, K, ge.make_ops(w.chain), a_type=ge.GE_DT_FP8_E4M3 if fp8 else ge.GE_DT_BF16,
                        b_type=ge.GE_DT_FP8_E4M3 if fp8 else ge.GE_DT_BF16,
                        b_layout=ge.GE_LAYOUT_NK if fp8 else ge.GE_LAYOUT_KN)
    assert ge.gemm_epilogue_validate(desc) == ge.GE_OK
    desc_big = ge.make_desc(1, M + 8, N, K, ge.make_ops(w.chain),
                            a_type=desc.a_type, b_type=desc.b_type, b_layout=desc.b_layout)
    assert ge.gemm_epilogue_validate(desc_big) == ge.GE_ERR_UNSUPPORTED   # the limit is where it says
    Y = torch.empty((1, M, N), dtype=torch.bfloat16, device="cuda")
    plan = ge.Plan(desc)
    print(f"\nlargest extent {in_dtype}: M={M} K={K}: {plan.describe()}", flush=True)
    plan.run(ge.make_args(A=A, B=prob.tensors["B"], bias=prob.tensors["bias"], Y=Y, alpha=w.alpha))
    torch.cuda.synchronize()
    rows = np.r_[0:64, M // 2:M // 2 + 64, M - 264:M]            # head, middle, ragged tail
    a_rows = A[0, torch.from_numpy(rows).cuda()].cpu()
    a_bits = a_rows.numpy() if fp8 else a_rows.view(torch.int16).numpy().view(np.uint16)
    ref = oracle.run_workload(w.with_shape(M=len(rows)), {**small, "A": a_bits[None]})
    y = Y[0, torch.from_numpy(rows).cuda()].cpu().view(torch.int16).numpy().view(np.uint16)
    # fp8 operands: allow the fp8 instruction's accumulation error (ReLU's slope is 1)
    allow = fp8_acc_bound(a_bits[None], small["B"], w.alpha) if fp8 else None
    check_bf16(y[None], ref.y, f"largest extent {in_dtype}", allow=allow)


def test_run_rejects_bad_arguments_without_launching():
    """run() returns GE_ERR_INVALID_ARG, and enqueues nothing, for a pointer the chain needs
    that is NULL or misaligned, and for a too-small workspace; the output stays untouched."""
    stream = torch.cuda.current_stream().cuda_stream

    def expect_invalid(prob, **changes):
        args = ge.ge_args_t.from_buffer_copy(prob.args)
        if prob.plan.workspace is not None:
            args.workspace, args.workspace_bytes = prob.plan.workspace.data_ptr(), prob.plan.workspace.numel()
        for k, v in changes.items():
            setattr(args, k, v)
        before = prob.Y.clone()
        assert ge.gemm_epilogue_run(prob.plan.handle, args, stream) == ge.GE_ERR_INVALID_ARG, changes
        torch.cuda.synchronize()
        assert torch.equal(prob.Y, before), changes

    fwd = workloads.WORKLOADS["c5"].with_shape(M=128, N=128, K=128)
    p = runner.prepare(fwd, workloads.generate(fwd))
    for ptr in ("A", "B", "Y", "bias", "amax"):
        expect_invalid(p, **{ptr: None})
    expect_invalid(p, Y=p.Y.data_ptr() + 2)                     # 16-byte alignment
    expect_invalid(p, A=p.tensors["A"].data_ptr() + 8)
    expect_invalid(p, bias=p.tensors["bias"].data_ptr() + 4)
    expect_invalid(p, amax=p.amax.data_ptr() + 2)               # 4-byte alignment
    expect_invalid(p, workspace_bytes=p.plan.workspace.numel() - 4)
    expect_invalid(p, workspace=None, workspace_bytes=0)

    pair = workloads.WORKLOADS["c3"].with_shape(M=128, N=128, K=128)
    pp = runner.prepare(pair, workloads.generate(pair))
    expect_invalid(pp, B2=None)

    bwd = workloads.WORKLOADS["f2"].with_shape(M=128, N=128, K=128)
    pb = runner.prepare(bwd, workloads.generate(bwd))
    expect_invalid(pb, aux=None)                                 # the saved pre-activation Z
    expect_invalid(pb, col_sum=None)

    rms = workloads.WORKLOADS["c4"].with_shape(M=128, N=128, K=128)
    pr = runner.prepare(rms, workloads.generate(rms))
    expect_invalid(pr, residual=None)


# ---------------------------------------------------------------------------------------------
# Two-wave instances (two waves per SIMD alternating memory and matrix phases): forward chains
# on bf16 operands with B given [K][N] and K a multiple of 64.  Ragged M and N, K = 192 (the
# loop's leading all-zero steps included), batch 2; every chain of the workloads; full sizes.
# ---------------------------------------------------------------------------------------------

TWO_WAVE = {"single": 5, "pair": 6}
TWO_WAVE_SHAPE = dict(batch=2, M=300, N=264, K=192)


def run_two_wave(w, inp):
    prob = gpu_run(w, inp, TWO_WAVE["pair" if w.pairwise else "single"])
    assert "threads=512" in prob.plan.describe(), prob.plan.describe()
    return prob


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "f1"])
def test_two_wave_ragged(name):
    w = workloads.WORKLOADS[name].with_shape(**TWO_WAVE_SHAPE)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave(w, inp), f"{name} two-wave ragged")


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_two_wave_sensitive(name):
    w = workloads.WORKLOADS[name].with_shape(**TWO_WAVE_SHAPE)
    inp = workloads.generate(w, sensitive=True)
    compare(w, inp, run_two_wave(w, inp), f"{name} two-wave sensitive")


@pytest.mark.parametrize("chain", [(("scale",), ("row_scale",), ("bias",), ("act", "silu"), ("residual",), ("col_sum",),
                                    ("amax",)),
                                   (("row_rms", 1e-6), ("bias",), ("act", "relu"), ("amax",)),
                                   (("scale",), ("pairwise", "gelu_tanh"), ("residual",), ("col_sum",)),
                                   (("row_rms", 1e-6), ("pairwise", "silu"), ("amax",)),
                                   (("scale",), ("row_rms", 0.5), ("residual",), ("col_sum",))],
                         ids=["rowscale-bias-silu-res-colsum-amax", "rms-bias-relu-amax", "pair-gelu-res-colsum",
                              "rms-pair-silu-amax", "scale-rms-eps-res-colsum"])
def test_two_wave_chains(chain):
    base = workloads.WORKLOADS["c3" if any(op[0] == "pairwise" for op in chain) else "c2"]
    w = dataclasses.replace(base, chain=chain).with_shape(**TWO_WAVE_SHAPE)
    inp = workloads.generate(w)
    if w.has("row_scale"):
        inp = {**inp, "row_scale": np.random.default_rng(5).uniform(0.5, 1.5, (w.batch, w.M)).astype(np.float32)}
    prob = run_two_wave(w, inp)
    compare(w, inp, prob, f"two-wave {chain}")
    assert_counters_zero(w, prob, f"two-wave {chain}")


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("K", [0, 64, 128, 256, 320])
def test_two_wave_k_steps(K, layout):
    """K of 0, 1, 2, 4 and 5 steps of 64: whole and partial rings of the four-step loop."""
    w = dataclasses.replace(workloads.WORKLOADS["c2"], b_layout=layout).with_shape(batch=1, M=256, N=512, K=K)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave(w, inp), f"two-wave K={K} {layout}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "f1"])
def test_two_wave_ragged_b_nk(name):
    """B given [N][K]: staged in two-step slots like A on the two-wave instances."""
    w = dataclasses.replace(workloads.WORKLOADS[name], b_layout="nk").with_shape(**TWO_WAVE_SHAPE)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave(w, inp), f"{name} two-wave ragged B [N][K]")


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("chain", BACKWARD_CHAINS, ids=lambda c: "-".join(op[0] + (op[1] if len(op) > 1 and isinstance(op[1], str) else "") for op in c))
def test_two_wave_backward_chains(chain, layout):
    w = dataclasses.replace(workloads.WORKLOADS["f2"], chain=chain, b_layout=layout, alpha=0.75,
                            bias_var=0.3).with_shape(**TWO_WAVE_SHAPE)
    inp = workloads.generate(w)
    compare(w, inp, run_two_wave(w, inp), f"two-wave backward {chain} {layout}")


def test_two_wave_is_refused_where_it_does_not_apply():
    """A requested two-wave instance with K not a multiple of two steps (64 bf16 or 128 fp8
    values) is GE_ERR_UNSUPPORTED at validation."""
    ops = ge.make_ops((("scale",), ("act", "relu")))
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 192, ops, tile=5)) == ge.GE_OK
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 200, ops, tile=5)) == ge.GE_ERR_UNSUPPORTED
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 192, ops, tile=5,
                                                  b_layout=ge.GE_LAYOUT_NK)) == ge.GE_OK
    rms = ge.make_ops((("row_rms", 1e-6), ("act", "relu")))
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 192, rms, tile=5)) == ge.GE_OK
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 200, rms, tile=5)) == ge.GE_ERR_UNSUPPORTED
    grad = ge.make_ops((("act_grad", "gelu_tanh"),))
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 192, grad, tile=5)) == ge.GE_OK
    assert ge.gemm_epilogue_validate(ge.make_desc(1, 256, 256, 200, grad, tile=5)) == ge.GE_ERR_UNSUPPORTED
    f8 = ge.make_desc(1, 256, 256, 192, ops, tile=5, a_type=ge.GE_DT_FP8_E4M3, b_type=ge.GE_DT_FP8_E4M3,
                      b_layout=ge.GE_LAYOUT_NK)
    assert ge.gemm_epilogue_validate(f8) == ge.GE_ERR_UNSUPPORTED          # fp8: K % 128


@pytest.mark.parametrize("name,threads", [("c1", 256), ("c2", 512), ("c3", 512), ("c4", 512), ("c5", 512),
                                          ("f1", 512), ("f2", 512), ("f3", 512)])
def test_default_instance(name, threads):
    """With no tile requested the library takes the two-wave instances wherever they apply at
    >= 256 workgroups (c2 .. c5, f1 .. f3) and the one-wave-per-SIMD instances for small grids
    (c1)."""
    assert not os.environ.get("GE_FORCE_TILE")
    h = ge.gemm_epilogue_create(runner.descriptor(workloads.WORKLOADS[name]))
    try:
        assert f"threads={threads}" in ge.gemm_epilogue_describe(h), ge.gemm_epilogue_describe(h)
    finally:
        ge.gemm_epilogue_destroy(h)


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5", "f1", "f2"])
def test_two_wave_full_workload(name):
    """The workloads at full size on the two-wave instances (sampled rows for the largest)."""
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    prob = run_two_wave(w, inp)
    rows = None if name == "c2" else np.r_[0:40, 1000:1040, w.M - 300:w.M]
    compare(w, inp, prob, f"{name} two-wave full", rows=rows)
    assert_counters_zero(w, prob, f"{name} two-wave full")
    if rows is not None and w.has("amax"):
        check_amax(prob.amax_host(), oracle.run_workload(w, inp).amax, f"{name} two-wave full amax")


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_two_wave_strided_operands_and_broadcast_b(layout):
    """Two-wave instance: lda > K, a padded ldb and a batch stride of 0 on B (one weight shared
    by every batch), ragged M and N, in both B layouts."""
    batch, M, N, K = 3, 300, 264, 192
    nk = layout == "nk"
    lda, ldb = K + 40, (K + 24 if nk else N + 24)
    w = dataclasses.replace(workloads.WORKLOADS["c2"], b_layout=layout).with_shape(batch=batch, M=M, N=N, K=K)
    inp = workloads.generate(w, sensitive=True)
    A_pad = np.zeros((batch, M, lda), dtype=np.uint16)
    A_pad[:, :, :K] = inp["A"]
    rows, cols = (N, K) if nk else (K, N)
    B_pad = np.zeros((1, rows, ldb), dtype=np.uint16)
    B_pad[0, :, :cols] = inp["B"][0]
    dev = "cuda"
    A = runner.to_device_bf16(A_pad, dev)
    B = runner.to_device_bf16(B_pad, dev)
    bias = runner.to_device_bf16(inp["bias"], dev)
    Y = torch.empty((batch, M, N), dtype=torch.bfloat16, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    desc = ge.make_desc(batch, M, N, K, ge.make_ops(w.chain), lda=lda, ldb=ldb, stride_b=0, tile=TWO_WAVE["single"],
                        b_layout=ge.GE_LAYOUT_NK if nk else ge.GE_LAYOUT_KN)
    plan = ge.Plan(desc)
    assert "threads=512" in plan.describe(), plan.describe()
    plan.run(ge.make_args(A=A, B=B, bias=bias, Y=Y, amax=amax, alpha=w.alpha))
    torch.cuda.synchronize()
    B_bcast = np.repeat(inp["B"][:1], batch, axis=0)
    ref = oracle.run_chain(w.chain, inp["A"], B_bcast, bias=inp["bias"], alpha=w.alpha, b_layout=layout)
    check_bf16(Y.cpu().view(torch.int16).numpy().view(np.uint16), ref.y, f"two-wave strided {layout}")
    check_amax(float(amax.item()), ref.amax, f"two-wave strided {layout}")
