"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and its HIP-free descriptor validation returns the documented codes.
No compute is launched here."""
import ctypes
import glob
import os
import re

import pytest

import gemm_epilogue_transformer_tiled_amd as ge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols(pattern=r"gemm_epilogue_\w+"):
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(" + pattern + r")\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert len(names) >= 7
    lib = ctypes.CDLL(ge.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ge.EXPORTED)


def test_reference_build_exports_the_same_symbols_and_validates_alike():
    """The reference build (serial mainloop) loads beside the fused library, exports the same
    entry points and accepts and refuses the same descriptors, two-wave instances included."""
    names = _declared_symbols()
    ser = ge.load_serial_library()
    assert ser is not ge.lib
    for n in names:
        assert hasattr(ser, n), n
    for tile in (ge.GE_TILE_256x256_2W, ge.GE_TILE_256x128_PAIR_2W):
        pair = tile == ge.GE_TILE_256x128_PAIR_2W
        ops = ge.make_ops([("pairwise", "silu")] if pair else [("scale",), ("amax",)])
        for K, want in ((256, ge.GE_OK), (200, ge.GE_ERR_UNSUPPORTED)):
            d = ge.make_desc(1, 512, 512, K, ops, tile=tile)
            assert ge.lib.gemm_epilogue_validate(ctypes.byref(d)) == want
            assert ser.gemm_epilogue_validate(ctypes.byref(d)) == want


def test_device_code_hash_reads_the_fatbin_section():
    """bench.py keys its measured-traffic table on the device code: the hash covers the
    library's .hip_fatbin section, which the reference build (other kernels) does not share."""
    import hashlib
    import importlib.util
    import shutil
    import subprocess
    spec = importlib.util.spec_from_file_location("bench_for_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    h = bench.kernel_code_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert bench.kernel_code_hash(ge.SERIAL_LIB_PATH) != h
    if shutil.which("objcopy"):
        import tempfile
        with tempfile.TemporaryDirectory() as tmp:
            out = os.path.join(tmp, "fatbin.bin")
            subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", ge.LIB_PATH, out], check=True)
            assert hashlib.sha256(open(out, "rb").read()).hexdigest()[:16] == h


def test_baselines_library_exports_every_declared_symbol():
    from gemm_epilogue_transformer_tiled_amd import baselines
    names = _declared_symbols(r"ge_(?:unfused|probe)_\w+")
    assert len(names) == 17
    lib = ctypes.CDLL(baselines.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(baselines.EXPORTED)


def test_baselines_reject_invalid_arguments_without_launching():
    from gemm_epilogue_transformer_tiled_amd import baselines
    lib = baselines.lib
    assert lib.ge_unfused_scale(None, None, -1, 1.0, None) == 1
    assert lib.ge_unfused_act(None, None, 8, 1, None) == 1          # null pointers with n > 0
    assert lib.ge_unfused_act(None, None, 0, 7, None) == 1          # unknown activation
    assert lib.ge_unfused_bias_col(None, None, None, 0, 12, None) == 1
    assert lib.ge_unfused_amax(None, 0, None, None) == 1
    assert lib.ge_probe_copy(None, None, 24, None) == 1             # not a multiple of 16
    assert lib.ge_probe_mfma(None, 1, 1, None) == 1
    assert lib.ge_probe_mfma_variant(None, 1, 1, 0, None) == 1
    sink = ctypes.c_float()
    assert lib.ge_probe_mfma_variant(ctypes.byref(sink), 1, 1, 3, None) == 1   # unknown form
    assert lib.ge_probe_lds_read(None, None, 1, 1, None) == 1
    assert lib.ge_probe_lds_read(ctypes.byref(sink), ctypes.byref(sink), 0, 1, None) == 1   # no workgroups
    assert lib.ge_unfused_scale(None, None, 0, 1.0, None) == 0      # empty: nothing to do


def _desc(**kw):
    base = dict(batch=1, M=64, N=64, K=64, ops=ge.make_ops([("scale",), ("bias",), ("act", "gelu_tanh"), ("amax",)]))
    base.update(kw)
    return ge.make_desc(**base)


def test_validate_accepts_every_workload_chain():
    import workloads
    for w in workloads.WORKLOADS.values():
        in_t = ge.GE_DT_FP8_E4M3 if w.in_dtype == "fp8_e4m3" else ge.GE_DT_BF16
        d = ge.make_desc(w.batch, w.M, w.N, w.K, ge.make_ops(w.chain),
                         y_type=ge.GE_DT_FP8_E4M3 if w.out == "fp8_e4m3" else ge.GE_DT_BF16,
                         a_type=in_t, b_type=in_t,
                         b_layout=ge.GE_LAYOUT_NK if w.b_layout == "nk" else ge.GE_LAYOUT_KN)
        assert ge.gemm_epilogue_validate(d) == ge.GE_OK, w.name


@pytest.mark.parametrize("kw,want", [
    (dict(M=-1), ge.GE_ERR_INVALID_ARG),
    (dict(K=-8), ge.GE_ERR_INVALID_ARG),
    (dict(N=12), ge.GE_ERR_UNSUPPORTED),                  # N not a multiple of 8
    (dict(K=20), ge.GE_ERR_UNSUPPORTED),
    (dict(lda=32), ge.GE_ERR_INVALID_ARG),                # lda < K
    (dict(ldb=72, ldy=72), ge.GE_OK),
    (dict(ldb=68), ge.GE_ERR_UNSUPPORTED),                # ld not a multiple of 8
    (dict(a_type=ge.GE_DT_FP8_E4M3), ge.GE_ERR_UNSUPPORTED),
    (dict(y_type=ge.GE_DT_FP32), ge.GE_ERR_UNSUPPORTED),
    (dict(y_type=ge.GE_DT_FP8_E4M3), ge.GE_ERR_INVALID_ARG),  # fp8 output without QUANT_FP8
    (dict(batch=2, stride_y=0), ge.GE_ERR_INVALID_ARG),   # batches would overwrite each other
    (dict(batch=2, stride_b=0), ge.GE_OK),                # broadcast B
    (dict(M=0), ge.GE_OK),
    (dict(batch=0), ge.GE_OK),
    (dict(K=0), ge.GE_OK),
    (dict(M=1 << 20, K=1 << 12), ge.GE_ERR_UNSUPPORTED),  # A extent beyond 2 GiB
])
def test_validate_status_codes(kw, want):
    assert ge.gemm_epilogue_validate(_desc(**kw)) == want


@pytest.mark.parametrize("chain,want", [
    ([("bias",), ("scale",)], ge.GE_ERR_INVALID_ARG),                 # out of canonical order
    ([("scale",), ("scale",)], ge.GE_ERR_INVALID_ARG),                # duplicate
    ([("act", "relu"), ("pairwise", "silu")], ge.GE_ERR_INVALID_ARG),  # exclusive
    ([("row_rms", 1e-6), ("row_scale",)], ge.GE_ERR_INVALID_ARG),      # exclusive
    ([("bias",), ("pairwise", "silu")], ge.GE_ERR_UNSUPPORTED),       # bias with pairwise
    ([("row_rms", -1.0)], ge.GE_ERR_INVALID_ARG),
    ([("row_rms", 1e-6), ("pairwise", "none")], ge.GE_OK),            # RMSNorm-MLP shape of chain
    ([("scale",), ("row_scale",), ("bias",), ("act", "silu"), ("residual",), ("amax",)], ge.GE_OK),
])
def test_validate_chain_rules(chain, want):
    assert ge.gemm_epilogue_validate(_desc(ops=ge.make_ops(chain))) == want


def test_bad_op_kind_and_act():
    d = _desc()
    d.ops[0].kind = 42
    assert ge.gemm_epilogue_validate(d) == ge.GE_ERR_INVALID_ARG
    d = _desc()
    d.ops[2].act = 9
    assert ge.gemm_epilogue_validate(d) == ge.GE_ERR_INVALID_ARG
    d = _desc()
    d.n_ops = 9
    assert ge.gemm_epilogue_validate(d) == ge.GE_ERR_INVALID_ARG


def test_rms_needs_k():
    d = _desc(K=0, ops=ge.make_ops([("row_rms", 1e-6)]))
    assert ge.gemm_epilogue_validate(d) == ge.GE_ERR_INVALID_ARG


def test_quant_requires_fp8_output_and_is_last():
    ok = _desc(ops=ge.make_ops([("bias",), ("act", "gelu_tanh"), ("amax",), ("quant_fp8",)]),
               y_type=ge.GE_DT_FP8_E4M3)
    assert ge.gemm_epilogue_validate(ok) == ge.GE_OK
    bf16_out = _desc(ops=ge.make_ops([("bias",), ("quant_fp8",)]))
    assert ge.gemm_epilogue_validate(bf16_out) == ge.GE_ERR_INVALID_ARG


def test_null_arguments_and_status_strings():
    assert ge.lib.gemm_epilogue_validate(None) == ge.GE_ERR_INVALID_ARG
    assert ge.lib.gemm_epilogue_create(None, None) == ge.GE_ERR_INVALID_ARG
    assert ge.lib.gemm_epilogue_run(None, None, None) == ge.GE_ERR_INVALID_ARG
    assert ge.lib.gemm_epilogue_run_noalloc(None, None, None) == ge.GE_ERR_INVALID_ARG
    ge.gemm_epilogue_destroy(None)
    for s in range(6):
        assert ge.gemm_epilogue_status_string(s).startswith("GE_")
    assert "unknown" in ge.gemm_epilogue_status_string(77)


def test_create_without_a_gfx950_device_reports_device_error():
    """On a host with no GPU, create() must fail cleanly with GE_ERR_DEVICE (and set no handle)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ge.ge_handle_t(1234)
    st = ge.lib.gemm_epilogue_create(ctypes.byref(_desc()), ctypes.byref(h))
    assert st == ge.GE_ERR_DEVICE
    assert not h.value


FP8_OPS = dict(a_type=ge.GE_DT_FP8_E4M3, b_type=ge.GE_DT_FP8_E4M3, b_layout=ge.GE_LAYOUT_NK)


@pytest.mark.parametrize("kw,chain,want", [
    (dict(), [("scale",), ("bias",), ("act", "relu"), ("amax",)], ge.GE_OK),
    (dict(), [("scale",), ("pairwise", "silu")], ge.GE_OK),
    (dict(b_layout=ge.GE_LAYOUT_KN), [("scale",)], ge.GE_ERR_UNSUPPORTED),     # fp8 B must be [N][K]
    (dict(b_type=ge.GE_DT_BF16), [("scale",)], ge.GE_ERR_UNSUPPORTED),         # mixed operand types
    (dict(K=24, lda=32, ldb=32), [("scale",)], ge.GE_ERR_UNSUPPORTED),         # K not a multiple of 16
    (dict(K=48, lda=56, ldb=48), [("scale",)], ge.GE_ERR_UNSUPPORTED),         # lda not a multiple of 16
    (dict(K=48), [("scale",)], ge.GE_OK),
    (dict(), [("row_rms", 1e-6)], ge.GE_ERR_UNSUPPORTED),                      # no in-kernel row statistic
    (dict(), [("act_grad", "gelu_tanh")], ge.GE_ERR_UNSUPPORTED),
    (dict(a_type=7, b_type=7), [("scale",)], ge.GE_ERR_INVALID_ARG),           # unknown dtype
    # extents count bytes: an A of just under 2 GiB fits as fp8 and not as bf16
    (dict(M=(1 << 19) - 4096, K=4096), [("scale",)], ge.GE_OK),
    (dict(M=(1 << 19) - 4096, K=4096, a_type=ge.GE_DT_BF16, b_type=ge.GE_DT_BF16), [("scale",)],
     ge.GE_ERR_UNSUPPORTED),
    (dict(M=1 << 19, K=4096), [("scale",)], ge.GE_ERR_UNSUPPORTED),
])
def test_validate_fp8_operands(kw, chain, want):
    args = dict(batch=1, M=64, N=64, K=64, ops=ge.make_ops(chain), **FP8_OPS)
    args.update(kw)
    assert ge.gemm_epilogue_validate(ge.make_desc(**args)) == want
