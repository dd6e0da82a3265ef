"""Writes tests/golden/oracle_digest.json from the oracle alone.

A regression fixture: it records what the pinned oracle computes for the
small single-GEMM workload (M=N=K=256) and for tiny shapes of every workload,
so an accidental change to the oracle's arithmetic shows up as a diff.  It
calls only ``oracle`` and the seeded input generator.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def digest(w):
    res = oracle.run_workload(w, workloads.generate(w))
    return {
        "shape": [w.batch, w.M, w.N, w.K],
        "codes_sha256": hashlib.sha256(res.codes.tobytes()).hexdigest(),
        "amax": res.amax,
        "y_first": [float(v) for v in res.y.ravel()[:4]],
    }


def main():
    out = {"c1_full": digest(workloads.WORKLOADS["c1"])}
    for name in workloads.CONFIG_ORDER:
        w = workloads.WORKLOADS[name].with_shape(batch=min(2, workloads.WORKLOADS[name].batch), M=40, N=24, K=48)
        out[name + "_tiny"] = digest(w)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digest.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
