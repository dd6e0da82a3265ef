"""Builds libgemm_epilogue.so (the fused path), libgemm_epilogue_serial.so (its reference build:
every instance with a mainloop that overlaps nothing, for bit-for-bit race tests) and
libge_baselines.so (unfused comparators and calibration probes) in-tree with hipcc for gfx950.

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
ONE_WAVE = [f"ge_tile_{t}_{lay}.hip" for t in ("256x256", "256x128_pair", "128x128", "64x64", "128x128_pair")
            for lay in ("kn", "nk", "f8")]
TWO_WAVE = [f"ge_tile_{t}_{lay}.hip" for t in ("256x256w8", "256x128w8_pair") for lay in ("kn", "nk", "f8")]
COMMON = ["ge_kernels.hip", "noalloc.hip", "tiles.cpp", "api.cpp"]
# library -> (its sources, extra compiler flags)
TARGETS = {
    os.path.join(HERE, "libgemm_epilogue.so"): (ONE_WAVE + TWO_WAVE + COMMON, ()),
    os.path.join(HERE, "libgemm_epilogue_serial.so"): (ONE_WAVE + TWO_WAVE + COMMON, ("-DGE_SERIAL_PIPELINE=1",)),
    os.path.join(HERE, "libge_baselines.so"): (["baselines.hip", "probe_mfma16.hip"], ()),
}
# per-source compiler flags (the 16x16x32 probe keeps its accumulators in VGPRs: see its header)
SOURCE_FLAGS = {"probe_mfma16.hip": ("-mllvm", "-amdgpu-mfma-vgpr-form")}
LIB = os.path.join(HERE, "libgemm_epilogue.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(job) -> str:
    src, extra = job
    out_dir = os.path.join(BUILD_DIR, "serial") if extra else BUILD_DIR
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, ()), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} {' '.join(extra)}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(BUILD_DIR, "serial"), exist_ok=True)
    jobs = sorted({(src, extra) for srcs, extra in TARGETS.values() for src in srcs})
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(jobs, ex.map(_compile, jobs)))
    for lib, (srcs, extra) in TARGETS.items():
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[objs[(s, extra)] for s in srcs]]
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
