"""Golden fixtures: the pages' printed constants, and the oracle's regression digest."""
import json
import math
import os

import workloads
from tests.golden.make_golden import digest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_page_constants_are_what_the_workloads_use():
    c = json.load(open(os.path.join(HERE, "page_constants.json")))
    W = workloads.WORKLOADS
    assert abs(c["log2e"]["value"] - 1 / math.log(2)) < 1e-8
    assert W["c5"].quant_scale == c["fp8_scale"]["value"] == 448.0 / 4.0
    assert W["c4"].op("row_rms")[1] == c["rms_eps"]["value"]
    assert W["c1"].alpha == c["alpha_single"]["value"]
    assert W["c2"].alpha == c["alpha_batched"]["value"]


def _same(got, want):
    """Codes exactly; float64 values to 1e-12 (BLAS summation order may differ between hosts)."""
    assert got["shape"] == want["shape"]
    assert got["codes_sha256"] == want["codes_sha256"]
    if want["amax"] is None:
        assert got["amax"] is None
    else:
        assert math.isclose(got["amax"], want["amax"], rel_tol=1e-12)
    for a, b in zip(got["y_first"], want["y_first"]):
        assert math.isclose(a, b, rel_tol=1e-12, abs_tol=1e-15)


def test_oracle_digest_unchanged():
    stored = json.load(open(os.path.join(HERE, "oracle_digest.json")))
    _same(digest(workloads.WORKLOADS["c1"]), stored["c1_full"])
    for name in workloads.CONFIG_ORDER:
        w = workloads.WORKLOADS[name].with_shape(batch=min(2, workloads.WORKLOADS[name].batch), M=40, N=24, K=48)
        _same(digest(w), stored[name + "_tiny"])
