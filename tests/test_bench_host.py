"""Host logic of bench.py, on the CPU: the one-GPU refusal, the suite runner's per-configuration
status records (a failed configuration is recorded and the suite carries on; one that ends
abnormally stops it), the oracle's CPU baseline on a bounded sample, the roofline bound and
the measured-traffic table.  Child processes are replaced by canned results; nothing here
touches a GPU."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _args(bench, monkeypatch, *argv):
    monkeypatch.setattr(sys, "argv", ["bench.py", *argv])
    return bench.parse()


def _child_line(name, value):
    w = workloads.WORKLOADS[name]
    return json.dumps({
        "metric": "m", "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": 3, "warmup": 1,
        "ms_per_step": w.flops() / (value * 1e12) * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "kernel": "k"},
        "roofline": {"bound": "mfma", "frac": value / 2500.0, "frac_mfma": value / 2500.0, "traffic": 1,
                     "hbm_gbs_at_algorithmic_bytes": 1.0, "hbm_frac": 0.1, "algorithmic_bytes_per_launch": 2},
        "epilogue_overhead_pct": 1.5, "launch": {"mode": "eager"},
    })


class _FakeChildren:
    """Stands in for subprocess.run: per configuration a return code (0: a JSON line on
    stdout), or "timeout"; records the configurations started."""

    def __init__(self, outcomes):
        self.outcomes = outcomes
        self.started = []

    def __call__(self, cmd, capture_output, text, timeout):
        name = cmd[cmd.index("--config") + 1]
        self.started.append(name)
        what = self.outcomes.get(name, 0)
        if what == "timeout":
            raise subprocess.TimeoutExpired(cmd, timeout, output=b"partial", stderr=b"still running")
        out = _child_line(name, 1000.0 + len(self.started)) + "\n" if what == 0 else "progress\n"
        return subprocess.CompletedProcess(cmd, what, stdout=out, stderr=f"{name} stderr line\n")


def _run_suite(bench, monkeypatch, capsys, outcomes, *argv):
    fake = _FakeChildren(outcomes)
    monkeypatch.setattr(bench.subprocess, "run", fake)
    args = _args(bench, monkeypatch, "--steps", "3", "--warmup", "1", *argv)
    code = 0
    try:
        bench.run_suite(args)
    except SystemExit as e:
        code = e.code
    out = capsys.readouterr().out.strip().splitlines()
    assert len(out) == 1, out                      # one JSON line
    return json.loads(out[0]), fake, code


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_suite_is_headline_first_and_every_config_reports(bench, monkeypatch, capsys):
    d, fake, code = _run_suite(bench, monkeypatch, capsys, {})
    assert code == 0
    assert fake.started == bench.SUITE and bench.SUITE[0] == "c3"
    assert d["config"]["workload"] == "c3" and d["value"] == 1001.0
    assert set(d["per_config"]) == set(bench.SUITE)
    for name, rec in d["per_config"].items():
        assert rec["status"] == "ok" and rec["workload"] == name
        assert rec["frac"] == pytest.approx(rec["value"] / 2500.0)


def test_a_failed_config_is_recorded_and_the_suite_carries_on(bench, monkeypatch, capsys):
    d, fake, code = _run_suite(bench, monkeypatch, capsys, {"c1": 1, "c4": 2})
    assert code == 0 and fake.started == bench.SUITE
    assert d["per_config"]["c1"]["status"] == "failed" and d["per_config"]["c1"]["rc"] == 1
    assert "c1 stderr line" in d["per_config"]["c1"]["stderr_tail"]
    assert d["per_config"]["c4"]["status"] == "failed"
    assert all(d["per_config"][n]["status"] == "ok" for n in bench.SUITE if n not in ("c1", "c4"))


@pytest.mark.parametrize("abnormal", [134, -11, 139, "timeout"])
def test_an_abnormal_end_stops_the_suite(bench, monkeypatch, capsys, abnormal):
    d, fake, code = _run_suite(bench, monkeypatch, capsys, {"c2": abnormal})
    assert code == 0
    assert fake.started == ["c3", "c1", "c2"]          # nothing more started after c2
    rc = d["per_config"]["c2"]["rc"]
    assert rc == (124 if abnormal == "timeout" else abnormal) and rc in bench.ABNORMAL_RC
    for n in bench.SUITE[3:]:
        assert d["per_config"][n]["status"] == "skipped" and "c2" in d["per_config"][n]["reason"]


def test_a_failed_headline_gives_a_null_value_and_a_nonzero_exit(bench, monkeypatch, capsys):
    d, fake, code = _run_suite(bench, monkeypatch, capsys, {"c3": 1})
    assert code == 1
    assert d["value"] is None and d["config"]["workload"] == "c3"
    assert d["status"]["status"] == "failed"
    assert d["per_config"]["c1"]["status"] == "ok"       # the others still ran


def test_child_command_passes_the_budget_flags(bench, monkeypatch, capsys):
    seen = []

    def fake(cmd, capture_output, text, timeout):
        seen.append(cmd)
        name = cmd[cmd.index("--config") + 1]
        return subprocess.CompletedProcess(cmd, 0, stdout=_child_line(name, 900.0) + "\n", stderr="")

    monkeypatch.setattr(bench.subprocess, "run", fake)
    args = _args(bench, monkeypatch, "--suite", "c3,c2", "--no-probes", "--cpu-seconds", "7",
                 "--suite-cpu-seconds", "1.5")
    bench.run_suite(args)
    capsys.readouterr()
    assert [c[c.index("--config") + 1] for c in seen] == ["c3", "c2"]
    assert all("--no-probes" in c for c in seen)
    assert seen[0][seen[0].index("--cpu-seconds") + 1] == "7.0"      # the headline's budget
    assert seen[1][seen[1].index("--cpu-seconds") + 1] == "1.5"      # the rest: the short one


def test_unknown_suite_entry_is_refused(bench, monkeypatch, capsys):
    args = _args(bench, monkeypatch, "--suite", "c3,zz")
    with pytest.raises(SystemExit) as e:
        bench.run_suite(args)
    assert e.value.code == 2


def test_roofline_bound_of_the_workloads(bench):
    bound = {n: bench.roofline_bound(w, bench.PEAK_FP8_TFLOPS if w.in_dtype == "fp8_e4m3" else bench.PEAK_BF16_TFLOPS)
             for n, w in workloads.WORKLOADS.items()}
    assert bound["c1"][0] == "hbm"                      # 256^3: bytes outweigh flops
    for n in ("c2", "c3", "c4", "c5", "f1", "f2", "f3"):
        assert bound[n][0] == "mfma", (n, bound[n])
    b, t_mfma, t_hbm = bound["c3"]
    assert t_mfma == pytest.approx(workloads.WORKLOADS["c3"].flops() / 2.5e15 * 1e6)
    assert t_hbm == pytest.approx(workloads.WORKLOADS["c3"].algorithmic_bytes() / 8e12 * 1e6)


def test_measured_traffic_covers_the_suite_and_is_at_least_the_algorithmic_bytes(bench):
    assert set(bench.MEASURED_TRAFFIC) == set(bench.SUITE)
    for n, t in bench.MEASURED_TRAFFIC.items():
        # counters see every byte the kernel moves: at least what the method must move
        # (within the counters' rounding), and not absurdly more
        alg = workloads.WORKLOADS[n].algorithmic_bytes()
        assert 0.98 * alg <= t <= 10 * alg, (n, t, alg)


def test_cpu_baseline_is_the_oracle_on_a_bounded_sample(bench):
    w = workloads.WORKLOADS["c1"]
    inputs = workloads.generate(w)
    r = bench.cpu_baseline(w, inputs, 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "rows 0..255 of 256" in r["sample"]
    assert r["gemm_s_per_sample"] >= 0
