"""Builds libgemm_epilogue.so (the fused path) and libge_baselines.so (unfused comparators and
calibration probes) in-tree with hipcc for gfx950.

Usage: python gemm_epilogue_transformer_tiled_amd/build.py  (runs by path: importing the
package itself needs the library this script builds)
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
# library -> its sources
TARGETS = {
    os.path.join(HERE, "libgemm_epilogue.so"): [
        f"ge_tile_{t}_{lay}.hip" for t in ("256x256", "256x128_pair", "128x128", "64x64", "128x128_pair")
        for lay in ("kn", "nk", "f8")] + [f"ge_tile_{t}_{lay}.hip" for t in ("256x256w8", "256x128w8_pair")
                                          for lay in ("kn", "nk", "f8")] + [
        "ge_kernels.hip", "noalloc.hip", "tiles.cpp", "api.cpp"],
    os.path.join(HERE, "libge_baselines.so"): ["baselines.hip"],
}
LIB = os.path.join(HERE, "libgemm_epilogue.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = [src for srcs in TARGETS.values() for src in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(sources), os.cpu_count() or 4)) as ex:
        objs = dict(zip(sources, ex.map(_compile, sources)))
    for lib, srcs in TARGETS.items():
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[objs[s] for s in srcs]]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed for {lib}:\n{r.stderr[-6000:]}")
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
