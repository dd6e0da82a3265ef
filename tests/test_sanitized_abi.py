"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

``api.cpp`` (validation, plan creation, argument checks) and ``tiles.cpp`` are compiled for
the host with g++ and ``-fsanitize=address,undefined``, linked with stand-ins for the device
entry points (``tests/asan/device_stubs.cpp``) and driven by ``tests/asan/fuzz_abi.cpp``: random
and mutated descriptors through ``gemm_epilogue_validate`` (only documented status codes, the
same code twice), ``gemm_epilogue_create`` (``GE_ERR_DEVICE`` without a gfx950 GPU) and NULL or
out-of-range arguments to every entry point.  Any sanitizer report aborts the run.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_epilogue_transformer_tiled_amd", "csrc")
ASAN = os.path.join(ROOT, "tests", "asan")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path_factory.mktemp("asan") / "fuzz_abi")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "tiles.cpp"), os.path.join(ASAN, "device_stubs.cpp"),
           os.path.join(ASAN, "fuzz_abi.cpp"), f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_fuzz_abi_under_asan_and_ubsan(fuzzer, seed):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "abort_on_error=1:detect_leaks=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["LSAN_OPTIONS"] = f"suppressions={os.path.join(ASAN, 'lsan.supp')}"
    env["HIP_VISIBLE_DEVICES"] = ""          # no device: create() must report GE_ERR_DEVICE
    r = subprocess.run([fuzzer, str(seed), "100000"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "fuzz ok" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
