"""gemm_epilogue_run_noalloc (the entry point for callers that cannot allocate) against
gemm_epilogue_run, through the C-ABI on the GPU.

Both entry points run the same plan and the same kernels; only where the AMAX / COL_SUM scratch
lives differs (the library's static device array instead of a caller-given workspace).  The
outputs must therefore be bit-identical, and each is also checked against the oracle.  Two
calls in a row, the second on a smaller problem whose workspace layout differs, show that the
counters the static array keeps between calls are cleared.
"""
from __future__ import annotations

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    yield
    torch.cuda.synchronize()


def _noalloc_args(prob):
    """The problem's argument pack without a workspace."""
    a = ge.ge_args_t.from_buffer_copy(prob.args)
    a.workspace, a.workspace_bytes = None, 0
    return a


def _outputs(prob):
    torch.cuda.synchronize()
    return (prob.Y.clone(), None if prob.amax is None else prob.amax.clone(),
            None if prob.col_sum is None else prob.col_sum.clone())


def _check_oracle(w, inp, prob, what):
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


def _both(w, what):
    """Runs w through gemm_epilogue_run, then (outputs poisoned) gemm_epilogue_run_noalloc;
    returns the two sets of outputs."""
    inp = workloads.generate(w)
    prob = runner.prepare(w, inp)
    prob.run()
    ref = _outputs(prob)
    _check_oracle(w, inp, prob, what + " run")
    prob.Y.view(torch.uint8).fill_(0x5A)
    if prob.amax is not None:
        prob.amax.fill_(-1.0)
    if prob.col_sum is not None:
        prob.col_sum.fill_(float("nan"))
    st = ge.gemm_epilogue_run_noalloc(prob.plan.handle, _noalloc_args(prob), torch.cuda.current_stream().cuda_stream)
    assert st == ge.GE_OK, ge.gemm_epilogue_status_string(st)
    got = _outputs(prob)
    _check_oracle(w, inp, prob, what + " run_noalloc")
    return ref, got


def _same(ref, got, what):
    assert torch.equal(ref[0], got[0]), f"{what}: Y differs"
    for r, g, name in ((ref[1], got[1], "amax"), (ref[2], got[2], "col_sum")):
        if r is not None:
            assert torch.equal(r, g), f"{what}: {name} differs: {r[:4]} vs {g[:4]}"


# A larger problem first, then a smaller one with a different workspace layout: the second
# call finds the first call's partial sums and slots in the static array.
CASES = [
    ("amax", dataclasses.replace(workloads.WORKLOADS["c2"]).with_shape(batch=4, M=512, N=1024, K=256),
     dataclasses.replace(workloads.WORKLOADS["c2"]).with_shape(batch=1, M=200, N=136, K=64)),
    ("col_sum+amax",
     dataclasses.replace(workloads.WORKLOADS["f2"], chain=(("act_grad", "gelu_tanh"), ("col_sum",), ("amax",)))
     .with_shape(batch=2, M=1000, N=1032, K=512),
     dataclasses.replace(workloads.WORKLOADS["f2"], chain=(("act_grad", "gelu_tanh"), ("col_sum",), ("amax",)))
     .with_shape(batch=1, M=64, N=72, K=64)),
    ("fp8 out", workloads.WORKLOADS["c5"].with_shape(M=1024, N=2048, K=512),
     workloads.WORKLOADS["c5"].with_shape(M=300, N=264, K=200)),
    # two-wave RMS plans share the row statistic along a tile row through the scratch array
    ("rms shared", workloads.WORKLOADS["c4"].with_shape(M=8192, N=2048, K=256),
     dataclasses.replace(workloads.WORKLOADS["c4"], chain=(("row_rms", 1e-6), ("residual",), ("amax",)))
     .with_shape(M=4096, N=4096, K=128)),
]


@pytest.mark.parametrize("name,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_run_on_two_calls_in_a_row(name, big, small):
    ref, got = _both(big, f"{name} first call")
    _same(ref, got, f"{name} first call")
    ref, got = _both(small, f"{name} second call (smaller)")
    _same(ref, got, f"{name} second call (smaller)")


def test_noalloc_without_scratch_ops_and_on_empty_problems():
    """Chains without AMAX / COL_SUM use no scratch; an empty problem writes AMAX = 0."""
    w = workloads.WORKLOADS["c4"].with_shape(M=300, N=264, K=256)
    ref, got = _both(w, "c4 chain")
    _same(ref, got, "c4 chain")
    e = workloads.WORKLOADS["c2"].with_shape(batch=1, M=0, N=64, K=64)
    prob = runner.prepare(e, workloads.generate(e))
    st = ge.gemm_epilogue_run_noalloc(prob.plan.handle, _noalloc_args(prob), torch.cuda.current_stream().cuda_stream)
    assert st == ge.GE_OK
    torch.cuda.synchronize()
    assert prob.amax_host() == 0.0


def test_noalloc_rejects_a_plan_beyond_the_scratch_limit():
    """COL_SUM partials of 128 row tiles x 8200 columns (64x64 tile) need just over 4 MiB:
    rejected before anything is enqueued (col_sum keeps its poison).  The tensors have their
    full sizes, so nothing could be read out of bounds even if a launch happened."""
    w = dataclasses.replace(workloads.WORKLOADS["f2"]).with_shape(batch=1, M=8192, N=8200, K=64)
    desc = ge.make_desc(w.batch, w.M, w.N, w.K, ge.make_ops(w.chain), b_layout=ge.GE_LAYOUT_NK,
                        tile=ge.GE_TILE_64x64)
    plan = ge.Plan(desc)
    assert ge.gemm_epilogue_workspace_size(plan.handle) > ge.GE_NOALLOC_SCRATCH_BYTES
    dev = "cuda"
    col = torch.full((w.N,), 7.0, dtype=torch.float32, device=dev)
    args = ge.make_args(A=torch.zeros((w.M, w.K), dtype=torch.bfloat16, device=dev),
                        B=torch.zeros((w.N, w.K), dtype=torch.bfloat16, device=dev),
                        Y=torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev),
                        aux=torch.zeros((w.M, w.N), dtype=torch.bfloat16, device=dev), col_sum=col)
    st = ge.gemm_epilogue_run_noalloc(plan.handle, args, torch.cuda.current_stream().cuda_stream)
    assert st == ge.GE_ERR_SCRATCH
    assert "GE_NOALLOC_SCRATCH_BYTES" in ge.gemm_epilogue_status_string(st)
    torch.cuda.synchronize()
    assert float(col.min().item()) == 7.0 == float(col.max().item())
