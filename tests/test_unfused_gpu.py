"""GPU checks of the unfused comparator sequence and the calibration probes.

The unfused sequence (one kernel per epilogue operation, bf16 between kernels) is what the fused
kernel's bytes saved and speed-up are measured against, so it must compute the same function:
each workload's chain at reduced size against the float64 oracle.  Every intermediate is rounded
to bf16 (2**-9 relative per rounding), and a later addition that cancels (bias, residual) or an
activation's steep tail turns that into a large *relative* error on small outputs -- which is the
accuracy the unfused sequence really has, and part of what fusion buys.  So its outputs are
checked normwise against the oracle: the largest error within 2e-2 of max |y| and the RMS error
within 4e-3 of RMS |y| (a missing or wrong operation errs by tens of percent on both).  fp8
outputs, decoded, against the oracle's own codes decoded: each within one e4m3 spacing at that
value plus 2e-2 of the largest |v| (v = y * scale), the RMS difference within 2e-2 of RMS |v|.
AMAX (over the bf16-rounded output): within 4e-3 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

bl = pytest.importorskip("gemm_epilogue_transformer_tiled_amd.baselines")

SHAPES = {
    "c1": {},
    "c2": dict(batch=3, M=256, N=512, K=320),
    "c3": dict(M=512, N=704, K=512),
    "c4": dict(M=512, N=512, K=1024),
    "c5": dict(M=512, N=1024, K=512),
    "f1": dict(M=512, N=704, K=512),
    "f2": dict(M=512, N=704, K=512),
    "f3": dict(M=512, N=1024, K=512),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", list(SHAPES))
def test_unfused_sequence_matches_oracle(name, monkeypatch):
    w = workloads.WORKLOADS[name].with_shape(**SHAPES[name])
    inp = workloads.generate(w)
    u = bl.Unfused(w, inp)
    u.run()
    torch.cuda.synchronize()
    ref = oracle.run_workload(w, inp)
    y = u.y_host_bits()
    if w.out == "fp8_e4m3":
        v = np.clip(ref.y * w.quant_scale, -448.0, 448.0)
        d = np.abs(oracle.decode_e4m3(y) - oracle.decode_e4m3(ref.codes))
        spacing = np.maximum(2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -9))) - 3))
        top = float(np.abs(v).max())
        bad = d > spacing + 2e-2 * top
        assert not bad.any(), (name, int(bad.sum()), float(d.max()), top)
        assert float(np.sqrt(np.mean(d ** 2))) <= 2e-2 * float(np.sqrt(np.mean(v ** 2)))
    else:
        got = oracle.decode_bf16(y)
        err = np.abs(got - ref.y)
        top = float(np.abs(ref.y).max())
        rms = float(np.sqrt(np.mean(ref.y ** 2)))
        assert float(err.max()) <= 2e-2 * top, (name, float(err.max()), top)
        assert float(np.sqrt(np.mean(err ** 2))) <= 4e-3 * rms, (name, float(np.sqrt(np.mean(err ** 2))), rms)
    if w.has("amax"):
        monkeypatch.setattr(parity, "AMAX_TOL", 4e-3)
        parity.check_amax(u.amax_host(), ref.amax, f"unfused {name}")
    if w.has("col_sum"):
        # sums of bf16-rounded values: normwise against the largest column sum
        got, want = u.col_sum_host(), ref.col_sum
        assert float(np.abs(got - want).max()) <= 2e-2 * float(np.abs(want).max()), name
    # the sequence is the literal one: a GEMM per B operand plus one kernel per other operation
    n_ops = len([op for op in w.chain if op[0] not in ("pairwise",)])
    assert len(u.kernels()) == 1 + (2 if w.pairwise else 0) + n_ops + (1 if w.has("row_rms") else 0)
    assert u.algorithmic_bytes() > w.algorithmic_bytes()


def test_unfused_ops_on_ragged_sizes():
    """Vector bodies and scalar tails of the elementwise kernels (n not a multiple of 8)."""
    n = 8 * 1000 + 5
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda().to(torch.bfloat16)
    r = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda().to(torch.bfloat16)
    y = torch.empty_like(x)
    s = torch.cuda.current_stream().cuda_stream
    xd = x.double().cpu().numpy()
    rd = r.double().cpu().numpy()
    bl.call("ge_unfused_scale", x.data_ptr(), y.data_ptr(), n, 1.5, s)
    np.testing.assert_array_equal(y.float().cpu().numpy(), torch.from_numpy(xd * 1.5).to(torch.bfloat16).float().numpy())
    bl.call("ge_unfused_add", x.data_ptr(), r.data_ptr(), y.data_ptr(), n, s)
    np.testing.assert_array_equal(y.float().cpu().numpy(), torch.from_numpy(xd + rd).to(torch.bfloat16).float().numpy())
    bl.call("ge_unfused_act", x.data_ptr(), y.data_ptr(), n, 1, s)
    np.testing.assert_array_equal(y.float().cpu().numpy(), np.maximum(xd, 0).astype(np.float32))
    amax = torch.zeros(1, device="cuda")
    bl.call("ge_unfused_amax", x.data_ptr(), n, amax.data_ptr(), s)
    assert float(amax.item()) == float(np.abs(xd).max())
    bl.call("ge_unfused_amax", x.data_ptr(), 0, amax.data_ptr(), s)
    assert float(amax.item()) == 0.0
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    bl.call("ge_unfused_quant_fp8", x.data_ptr(), q.data_ptr(), n, 112.0, s)
    ref = oracle.encode_e4m3(np.clip(xd * 112.0, -448, 448))
    np.testing.assert_array_equal(q.cpu().numpy(), ref)
    # invalid arguments are reported, not launched
    assert bl.lib.ge_unfused_act(x.data_ptr(), y.data_ptr(), n, 9, s) == 1
    assert bl.lib.ge_unfused_bias_col(x.data_ptr(), x.data_ptr(), y.data_ptr(), 3, 12, s) == 1


def test_probes_report_plausible_peaks():
    m = bl.probe_mfma(workgroups=256, iters=256)
    assert 100.0 < m["tflops"] < 2600.0, m
    m16 = bl.probe_mfma(workgroups=256, iters=256, form="bf16_16x16x32")
    assert 100.0 < m16["tflops"] < 2600.0, m16
    m8 = bl.probe_mfma(workgroups=256, iters=256, form="fp8_32x32x64")
    assert 200.0 < m8["tflops"] < 5200.0, m8
    ll = bl.probe_lds_load(src_kb=1024, workgroups=256, iters=64)
    assert 500.0 < ll["gbs"] < 200000.0, ll
    lr = bl.probe_lds_read(workgroups=256, iters=1024)
    assert 1000.0 < lr["gbs"] < 1000000.0, lr
    assert 0.5 < lr["implied_clock_ghz"] < 3.5, lr            # s_memtime counts shader clocks
    assert 16.0 < lr["bytes_per_clk_cu"] <= 1024.0, lr
    c = bl.probe_copy(mib=64)
    assert 100.0 < c["gbs"] < 9000.0, c
