"""Race tests: the fused library against its reference build, bit for bit.

The reference build (``libgemm_epilogue_serial.so``: the same kernel sources compiled with
``GE_SERIAL_PIPELINE=1``) loads each two-step operand slot, waits for every load and reads
the slot between two full barriers, so no LDS stage is read before its loads land or refilled
while a wave still reads it.  Every comparison runs the same instance (tile shape, waves,
matrix-core instruction) in both builds: its MFMAs take the same fragments in the same order,
the RMS row statistic and the column sums are summed in the same order, and the epilogue is
the same code, so outputs, AMAX and column sums must agree bit for bit; a difference is a
synchronisation mistake in the pipelined mainloop.

Every comparison also checks both results against the oracle where the problem is small, so
the reference build is itself pinned; at full size the comparison covers every output of the
launch the benchmark times, which the oracle's sampled rows cannot.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import check_amax, check_bf16, check_col_sum, check_fp8

pytestmark = pytest.mark.gpu

ge = pytest.importorskip("gemm_epilogue_transformer_tiled_amd")
from gemm_epilogue_transformer_tiled_amd import runner  # noqa: E402
from tests.test_parity_gpu import TILE_NAMES  # noqa: E402

ONE_WAVE_SINGLE = [ge.GE_TILE_256x256, ge.GE_TILE_128x128, ge.GE_TILE_64x64]
ONE_WAVE_PAIR = [ge.GE_TILE_256x128_PAIR, ge.GE_TILE_128x128_PAIR]
F3 = workloads.WORKLOADS["f3"]
SHAPES = {"ragged": dict(batch=2, M=300, N=264, K=200), "long": dict(batch=1, M=520, N=392, K=1032)}
SHAPES8 = {"ragged": dict(batch=2, M=300, N=264, K=208), "long": dict(batch=1, M=520, N=392, K=1040)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def serial_lib():
    return ge.load_serial_library()


def _outputs(prob):
    out = {"Y": prob.Y.clone()}
    if prob.amax is not None:
        out["amax"] = prob.amax.clone()
    if prob.col_sum is not None:
        out["col_sum"] = prob.col_sum.clone()
    return out


def _clear(prob):
    """Fills the outputs with values no run writes, so an output left unwritten shows."""
    prob.Y.view(torch.uint8).fill_(0x5A)
    if prob.amax is not None:
        prob.amax.fill_(-1.0)
    if prob.col_sum is not None:
        prob.col_sum.fill_(float("nan"))


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _assert_same_bits(a, b, what):
    for key in a:
        x, y = _bits(a[key]), _bits(b[key])
        diff = np.flatnonzero(x != y)
        assert diff.size == 0, (f"{what}: {key} differs from the reference build in {diff.size} of {x.size} "
                                f"bytes, first at byte {diff[:4].tolist()}")


def run_both(w, inp, serial_lib, tile=None, ref_tile=None):
    """Runs `w` on instance `tile` of the fused library (None: create's choice) and on
    `ref_tile` of the reference build (None: the same instance), compares every output bit
    for bit, and returns the fused library's problem (holding its outputs again)."""
    prob = runner.prepare(w, inp, tile=tile)
    _clear(prob)
    prob.run()
    torch.cuda.synchronize()
    fused = _outputs(prob)
    desc = prob.plan.describe()
    assert "pipeline=serial" not in desc
    if ref_tile is None:
        ref_tile = tile
    assert ref_tile is not None
    ser = prob.with_tile(ref_tile, library=serial_lib)
    assert "pipeline=serial" in ser.plan.describe()
    _clear(prob)
    ser.run()
    torch.cuda.synchronize()
    reference = _outputs(prob)
    _assert_same_bits(fused, reference, f"{w.name} fused [{desc}] vs reference tile {TILE_NAMES[ref_tile]}")
    for k, v in fused.items():          # leave the fused library's outputs in place
        getattr(prob, k).copy_(v)
    ser.plan.close()
    return prob


def check_oracle(w, inp, prob, what):
    ref = oracle.run_workload(w, inp)
    y = prob.y_host_bits()
    if w.out == "fp8_e4m3":
        check_fp8(y, ref.codes, what)
    else:
        check_bf16(y, ref.y, what)
    if w.has("amax"):
        check_amax(prob.amax_host(), ref.amax, what)
    if w.has("col_sum"):
        check_col_sum(prob.col_sum_host(), ref.col_sum, what)


# chains for the single-B instances: AMAX + ReLU, RMS + residual, fp8 output, backward
SINGLE_CHAINS = {
    "c2": workloads.WORKLOADS["c2"],
    "c4": workloads.WORKLOADS["c4"],
    "c5": workloads.WORKLOADS["c5"],
    "f2": workloads.WORKLOADS["f2"],
}
PAIR_CHAINS = {"c3": workloads.WORKLOADS["c3"], "f1": workloads.WORKLOADS["f1"]}


@pytest.mark.parametrize("shape", list(SHAPES), ids=list(SHAPES))
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("tile", ONE_WAVE_SINGLE, ids=[TILE_NAMES[t] for t in ONE_WAVE_SINGLE])
@pytest.mark.parametrize("name", list(SINGLE_CHAINS))
def test_one_wave_single_matches_reference(name, tile, layout, shape, serial_lib):
    w = dataclasses.replace(SINGLE_CHAINS[name], b_layout=layout).with_shape(**SHAPES[shape])
    inp = workloads.generate(w)
    prob = run_both(w, inp, serial_lib, tile=tile)
    check_oracle(w, inp, prob, f"{name} {layout} {shape} tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("shape", list(SHAPES), ids=list(SHAPES))
@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("tile", ONE_WAVE_PAIR, ids=[TILE_NAMES[t] for t in ONE_WAVE_PAIR])
@pytest.mark.parametrize("name", list(PAIR_CHAINS))
def test_one_wave_pairwise_matches_reference(name, tile, layout, shape, serial_lib):
    w = dataclasses.replace(PAIR_CHAINS[name], b_layout=layout).with_shape(**SHAPES[shape])
    inp = workloads.generate(w)
    prob = run_both(w, inp, serial_lib, tile=tile)
    check_oracle(w, inp, prob, f"{name} {layout} {shape} tile {TILE_NAMES[tile]}")


@pytest.mark.parametrize("shape", list(SHAPES8), ids=list(SHAPES8))
@pytest.mark.parametrize("tile", ONE_WAVE_SINGLE + ONE_WAVE_PAIR, ids=[TILE_NAMES[t] for t in ONE_WAVE_SINGLE + ONE_WAVE_PAIR])
def test_one_wave_fp8_operands_match_reference(tile, shape, serial_lib):
    pair = tile in ONE_WAVE_PAIR
    w = F3 if not pair else dataclasses.replace(F3, out="bf16", chain=(("scale",), ("pairwise", "silu")))
    w = w.with_shape(**SHAPES8[shape])
    inp = workloads.generate(w)
    run_both(w, inp, serial_lib, tile=tile)


# The two-wave instances against their reference-build twins (same tile, waves and MFMA form);
# K a multiple of 64 (128 for fp8 operands).
TWO_WAVE_CASES = {
    "c2-kn": (workloads.WORKLOADS["c2"], "kn", dict(batch=2, M=600, N=776, K=576)),
    "c4-kn": (workloads.WORKLOADS["c4"], "kn", dict(batch=1, M=520, N=1032, K=640)),
    "c4-nk": (workloads.WORKLOADS["c4"], "nk", dict(batch=2, M=264, N=392, K=1024)),
    # more tiles than the GPU holds at once: later tiles of a tile row read the statistic that
    # earlier ones published instead of recomputing it
    "c4-rounds": (workloads.WORKLOADS["c4"], "kn", dict(batch=1, M=8192, N=8192, K=128)),
    "f1-rounds": (workloads.WORKLOADS["f1"], "nk", dict(batch=2, M=4096, N=11008, K=128)),
    "rms-chain-rounds": (dataclasses.replace(workloads.WORKLOADS["c4"], chain=(
        ("scale",), ("row_rms", 1e-6), ("bias",), ("act", "gelu_tanh"), ("residual",), ("col_sum",), ("amax",))),
        "kn", dict(batch=2, M=4096, N=4104, K=64)),
    "c5-nk": (workloads.WORKLOADS["c5"], "nk", dict(batch=1, M=520, N=1032, K=1088)),
    "f2-nk": (workloads.WORKLOADS["f2"], "nk", dict(batch=1, M=776, N=520, K=640)),
    "f2-kn": (workloads.WORKLOADS["f2"], "kn", dict(batch=2, M=300, N=392, K=512)),
    "relu-res-kn": (dataclasses.replace(workloads.WORKLOADS["c2"], chain=(("scale",), ("act", "relu"), ("residual",))),
                    "kn", dict(batch=1, M=520, N=520, K=1024)),
    "c3-kn": (workloads.WORKLOADS["c3"], "kn", dict(batch=1, M=600, N=520, K=576)),
    "c3-nk": (workloads.WORKLOADS["c3"], "nk", dict(batch=2, M=264, N=392, K=1024)),
    "f1-kn": (workloads.WORKLOADS["f1"], "kn", dict(batch=1, M=600, N=776, K=512)),
    "f1-nk": (workloads.WORKLOADS["f1"], "nk", dict(batch=1, M=264, N=520, K=640)),
    "f3": (F3, "nk", dict(batch=1, M=520, N=776, K=1152)),
    "f3-pair": (dataclasses.replace(F3, out="bf16", chain=(("scale",), ("pairwise", "silu"))), "nk",
                dict(batch=1, M=600, N=392, K=640)),
}


@pytest.mark.parametrize("case", list(TWO_WAVE_CASES))
def test_two_wave_matches_reference(case, serial_lib):
    w0, layout, shape = TWO_WAVE_CASES[case]
    w = dataclasses.replace(w0, b_layout=layout).with_shape(**shape)
    tile = ge.GE_TILE_256x128_PAIR_2W if w.pairwise else ge.GE_TILE_256x256_2W
    inp = workloads.generate(w)
    prob = run_both(w, inp, serial_lib, tile=tile)
    assert "threads=512" in prob.plan.describe()
    if w.in_dtype == "bf16" and w.M * w.N * w.batch <= 2 ** 22:
        check_oracle(w, inp, prob, f"two-wave {case}")


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5", "f1", "f2", "f3"])
def test_full_workload_matches_reference(name, serial_lib):
    """The benchmark's launch (create's choice of instance) on the full workload, every output
    against the reference build's twin of that instance."""
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    prob = runner.prepare(w, inp)
    tile = {"256x256": ge.GE_TILE_256x256_2W, "256x128": ge.GE_TILE_256x128_PAIR_2W}[
        "x".join(prob.plan.describe().split("tile=")[1].split("x")[:2])]
    prob.plan.close()
    prob = run_both(w, inp, serial_lib, tile=tile)
    assert "threads=512" in prob.plan.describe()


@pytest.mark.parametrize("name", ["c4", "f1", "f2"])
def test_full_workload_one_wave_matches_reference(name, serial_lib):
    """The chains with a row statistic or column sums at full size on the one-wave instance of
    the benchmark's tile shape."""
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    tile = ge.GE_TILE_256x128_PAIR if w.pairwise else ge.GE_TILE_256x256
    run_both(w, inp, serial_lib, tile=tile)
