"""Python binding of libgemm_epilogue.so (fused GEMM + epilogue on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI declared in ``include/gemm_epilogue.h``.  The
functions below carry the C names.  PyTorch supplies device memory and the
stream; nothing here computes on the host, and there is no fallback: if the
shared library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_epilogue.so")
# The reference build of the same sources: the one-wave instances with a mainloop that
# overlaps nothing, bit-identical to this library by construction (race tests only).
SERIAL_LIB_PATH = os.path.join(_HERE, "libgemm_epilogue_serial.so")

# ---- enums (mirror include/gemm_epilogue.h) ----
GE_OK, GE_ERR_INVALID_ARG, GE_ERR_UNSUPPORTED, GE_ERR_DEVICE, GE_ERR_HIP, GE_ERR_SCRATCH = range(6)
GE_NOALLOC_SCRATCH_BYTES = 4 << 20
GE_DT_BF16, GE_DT_FP8_E4M3, GE_DT_FP32 = range(3)
GE_ACT_NONE, GE_ACT_RELU, GE_ACT_GELU_TANH, GE_ACT_SILU = range(4)
GE_LAYOUT_KN, GE_LAYOUT_NK = range(2)
(GE_TILE_256x256, GE_TILE_256x128_PAIR, GE_TILE_128x128, GE_TILE_64x64, GE_TILE_128x128_PAIR,
 GE_TILE_256x256_2W, GE_TILE_256x128_PAIR_2W, GE_TILE_COUNT) = range(8)
(GE_OP_SCALE, GE_OP_ROW_RMS, GE_OP_ROW_SCALE, GE_OP_BIAS_COL, GE_OP_ACT, GE_OP_PAIRWISE_ACT_MUL,
 GE_OP_RESIDUAL, GE_OP_AMAX, GE_OP_QUANT_FP8, GE_OP_ACT_GRAD, GE_OP_COL_SUM) = range(11)
GE_MAX_OPS = 8

ACT_NAMES = {"none": GE_ACT_NONE, "relu": GE_ACT_RELU, "gelu_tanh": GE_ACT_GELU_TANH, "silu": GE_ACT_SILU}
OP_NAMES = {"scale": GE_OP_SCALE, "row_rms": GE_OP_ROW_RMS, "row_scale": GE_OP_ROW_SCALE,
            "bias": GE_OP_BIAS_COL, "act": GE_OP_ACT, "pairwise": GE_OP_PAIRWISE_ACT_MUL,
            "residual": GE_OP_RESIDUAL, "amax": GE_OP_AMAX, "quant_fp8": GE_OP_QUANT_FP8,
            "act_grad": GE_OP_ACT_GRAD, "col_sum": GE_OP_COL_SUM}


class ge_op_t(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("act", ctypes.c_int32), ("eps", ctypes.c_float)]


class ge_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldy", ctypes.c_int64), ("ldr", ctypes.c_int64),
        ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64), ("stride_y", ctypes.c_int64),
        ("stride_r", ctypes.c_int64),
        ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32), ("y_type", ctypes.c_int32),
        ("n_ops", ctypes.c_int32),
        ("ops", ge_op_t * GE_MAX_OPS),
        ("b_layout", ctypes.c_int32), ("tile", ctypes.c_int32),
        ("ldz", ctypes.c_int64), ("stride_z", ctypes.c_int64),
    ]


class ge_tile_info_t(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("pairwise", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32)]


class ge_args_t(ctypes.Structure):
    _fields_ = [
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("B2", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("row_scale", ctypes.c_void_p), ("residual", ctypes.c_void_p), ("Y", ctypes.c_void_p),
        ("amax", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("alpha", ctypes.c_float), ("quant_scale", ctypes.c_float),
        ("aux", ctypes.c_void_p), ("col_sum", ctypes.c_void_p),
    ]


ge_handle_t = ctypes.c_void_p

EXPORTED = ("gemm_epilogue_validate", "gemm_epilogue_create", "gemm_epilogue_workspace_size",
            "gemm_epilogue_run", "gemm_epilogue_run_noalloc", "gemm_epilogue_destroy",
            "gemm_epilogue_status_string", "gemm_epilogue_describe", "gemm_epilogue_tile_info")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python gemm_epilogue_transformer_tiled_amd/build.py` "
            "(there is no host fallback for this library)")
    # One HIP runtime per process: torch ships its own libamdhip64 (DT_NEEDED
    # "libamdhip64.so", soname "libamdhip64.so.7").  Loading torch first makes this
    # library's "libamdhip64.so.7" dependency resolve to that same loaded runtime;
    # loading this library first would make torch pull in a second runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    lib.gemm_epilogue_validate.argtypes = [ctypes.POINTER(ge_desc_t)]
    lib.gemm_epilogue_validate.restype = ctypes.c_int
    lib.gemm_epilogue_create.argtypes = [ctypes.POINTER(ge_desc_t), ctypes.POINTER(ge_handle_t)]
    lib.gemm_epilogue_create.restype = ctypes.c_int
    lib.gemm_epilogue_workspace_size.argtypes = [ge_handle_t, ctypes.POINTER(ctypes.c_size_t)]
    lib.gemm_epilogue_workspace_size.restype = ctypes.c_int
    lib.gemm_epilogue_run.argtypes = [ge_handle_t, ctypes.POINTER(ge_args_t), ctypes.c_void_p]
    lib.gemm_epilogue_run.restype = ctypes.c_int
    lib.gemm_epilogue_run_noalloc.argtypes = [ge_handle_t, ctypes.POINTER(ge_args_t), ctypes.c_void_p]
    lib.gemm_epilogue_run_noalloc.restype = ctypes.c_int
    lib.gemm_epilogue_destroy.argtypes = [ge_handle_t]
    lib.gemm_epilogue_destroy.restype = None
    lib.gemm_epilogue_status_string.argtypes = [ctypes.c_int]
    lib.gemm_epilogue_status_string.restype = ctypes.c_char_p
    lib.gemm_epilogue_describe.argtypes = [ge_handle_t, ctypes.c_char_p, ctypes.c_size_t]
    lib.gemm_epilogue_describe.restype = ctypes.c_int
    lib.gemm_epilogue_tile_info.argtypes = [ctypes.c_int32, ctypes.POINTER(ge_tile_info_t)]
    lib.gemm_epilogue_tile_info.restype = ctypes.c_int
    return lib


lib = _load()
_serial_lib: Optional[ctypes.CDLL] = None


def load_serial_library() -> ctypes.CDLL:
    """The reference build (``SERIAL_LIB_PATH``), loaded once; pass it to ``Plan(library=...)``."""
    global _serial_lib
    if _serial_lib is None:
        _serial_lib = _load(SERIAL_LIB_PATH)
    return _serial_lib


class GemmEpilogueError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gemm_epilogue_status_string(status)}")


# ---- the C functions, same names ----

def gemm_epilogue_validate(desc: ge_desc_t) -> int:
    return lib.gemm_epilogue_validate(ctypes.byref(desc))


def gemm_epilogue_create(desc: ge_desc_t) -> int:
    """Returns the handle (an int); raises GemmEpilogueError on a non-OK status."""
    h = ge_handle_t()
    st = lib.gemm_epilogue_create(ctypes.byref(desc), ctypes.byref(h))
    if st != GE_OK:
        raise GemmEpilogueError(st, "gemm_epilogue_create")
    return h.value


def gemm_epilogue_workspace_size(handle: int) -> int:
    n = ctypes.c_size_t()
    st = lib.gemm_epilogue_workspace_size(handle, ctypes.byref(n))
    if st != GE_OK:
        raise GemmEpilogueError(st, "gemm_epilogue_workspace_size")
    return n.value


def gemm_epilogue_run(handle: int, args: ge_args_t, stream: int = 0) -> int:
    return lib.gemm_epilogue_run(handle, ctypes.byref(args), stream)


def gemm_epilogue_run_noalloc(handle: int, args: ge_args_t, stream: int = 0) -> int:
    """gemm_epilogue_run with the library's static device scratch instead of args.workspace."""
    return lib.gemm_epilogue_run_noalloc(handle, ctypes.byref(args), stream)


def gemm_epilogue_destroy(handle: Optional[int]) -> None:
    lib.gemm_epilogue_destroy(handle)


def gemm_epilogue_status_string(status: int) -> str:
    return lib.gemm_epilogue_status_string(status).decode()


def gemm_epilogue_describe(handle: int) -> str:
    buf = ctypes.create_string_buffer(256)
    st = lib.gemm_epilogue_describe(handle, buf, len(buf))
    if st != GE_OK:
        raise GemmEpilogueError(st, "gemm_epilogue_describe")
    return buf.value.decode()


def gemm_epilogue_tile_info(tile: int) -> ge_tile_info_t:
    info = ge_tile_info_t()
    st = lib.gemm_epilogue_tile_info(tile, ctypes.byref(info))
    if st != GE_OK:
        raise GemmEpilogueError(st, "gemm_epilogue_tile_info")
    return info


# ---- marshalling helpers ----

def make_ops(chain: Iterable[tuple]) -> Sequence[Tuple[int, int, float]]:
    """Plain chain tuples (("scale",), ("act", "relu"), ("row_rms", 1e-6), ...) -> (kind, act, eps)."""
    out = []
    for op in chain:
        kind = OP_NAMES[op[0]]
        act, eps = 0, 0.0
        if op[0] in ("act", "pairwise", "act_grad"):
            act = ACT_NAMES[op[1]]
        elif op[0] == "row_rms":
            eps = float(op[1])
        out.append((kind, act, eps))
    return out


def make_desc(batch: int, M: int, N: int, K: int, ops: Sequence[Tuple[int, int, float]],
              y_type: int = GE_DT_BF16, lda: Optional[int] = None, ldb: Optional[int] = None,
              ldy: Optional[int] = None, ldr: Optional[int] = None, stride_a: Optional[int] = None,
              stride_b: Optional[int] = None, stride_y: Optional[int] = None,
              stride_r: Optional[int] = None, a_type: int = GE_DT_BF16, b_type: int = GE_DT_BF16,
              b_layout: int = GE_LAYOUT_KN, ldz: Optional[int] = None,
              stride_z: Optional[int] = None, tile: Optional[int] = None) -> ge_desc_t:
    """Descriptor for packed row-major operands unless leading dims / strides are given.
    b_layout GE_LAYOUT_NK: B (and B2) are [batch][N][K].  tile: a ge_tile_t to request that
    kernel instance (None: create chooses)."""
    d = ge_desc_t()
    d.tile = 0 if tile is None else tile + 1
    d.batch, d.M, d.N, d.K = batch, M, N, K
    d.b_layout = b_layout
    d.lda = K if lda is None else lda
    d.ldb = (K if b_layout == GE_LAYOUT_NK else N) if ldb is None else ldb
    d.ldy = N if ldy is None else ldy
    d.ldr = N if ldr is None else ldr
    d.stride_a = M * d.lda if stride_a is None else stride_a
    d.stride_b = (N if b_layout == GE_LAYOUT_NK else K) * d.ldb if stride_b is None else stride_b
    d.stride_y = M * d.ldy if stride_y is None else stride_y
    d.stride_r = M * d.ldr if stride_r is None else stride_r
    d.ldz = N if ldz is None else ldz
    d.stride_z = M * d.ldz if stride_z is None else stride_z
    d.a_type, d.b_type, d.y_type = a_type, b_type, y_type
    if len(ops) > GE_MAX_OPS:
        raise ValueError("too many epilogue ops")
    d.n_ops = len(ops)
    for i, (kind, act, eps) in enumerate(ops):
        d.ops[i].kind, d.ops[i].act, d.ops[i].eps = kind, act, eps
    return d


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_args(A=None, B=None, B2=None, bias=None, row_scale=None, residual=None, Y=None, amax=None,
              alpha: float = 1.0, quant_scale: float = 1.0, workspace=None, aux=None, col_sum=None) -> ge_args_t:
    """Variant pack from torch device tensors (or None)."""
    a = ge_args_t()
    a.aux, a.col_sum = _ptr(aux), _ptr(col_sum)
    a.A, a.B, a.B2, a.bias = _ptr(A), _ptr(B), _ptr(B2), _ptr(bias)
    a.row_scale, a.residual, a.Y, a.amax = _ptr(row_scale), _ptr(residual), _ptr(Y), _ptr(amax)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.alpha, a.quant_scale = alpha, quant_scale
    return a


class Plan:
    """Owns one handle (and its zero-filled device workspace, allocated by torch):
    create once, run many times on torch tensors and the current stream.  `library`: a
    library loaded by this module (default: ``lib``; the reference build for race tests)."""

    def __init__(self, desc: ge_desc_t, device="cuda", library: Optional[ctypes.CDLL] = None):
        self.desc = desc
        self.lib = lib if library is None else library
        h = ge_handle_t()
        st = self.lib.gemm_epilogue_create(ctypes.byref(desc), ctypes.byref(h))
        if st != GE_OK:
            raise GemmEpilogueError(st, "gemm_epilogue_create")
        self.handle = h.value
        self.workspace = None
        n = ctypes.c_size_t()
        st = self.lib.gemm_epilogue_workspace_size(self.handle, ctypes.byref(n))
        if st != GE_OK:
            raise GemmEpilogueError(st, "gemm_epilogue_workspace_size")
        nbytes = n.value
        if nbytes:
            import torch
            self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(256)
        st = self.lib.gemm_epilogue_describe(self.handle, buf, len(buf))
        if st != GE_OK:
            raise GemmEpilogueError(st, "gemm_epilogue_describe")
        return buf.value.decode()

    def run(self, args: ge_args_t, stream: Optional[int] = None) -> None:
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        if self.workspace is not None and not args.workspace:
            args.workspace = self.workspace.data_ptr()
            args.workspace_bytes = self.workspace.numel()
        st = self.lib.gemm_epilogue_run(self.handle, ctypes.byref(args), stream)
        if st != GE_OK:
            raise GemmEpilogueError(st, "gemm_epilogue_run")

    def close(self) -> None:
        if self.handle:
            self.lib.gemm_epilogue_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
