"""ctypes binding of libfusedproj (include/fusedproj.h).

Argument marshalling only: every function here forwards to the C entry point
of the same name.  Device pointers are plain Python ints.  Importing this
module raises if the library has not been built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfusedproj.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fusedproj.h")

FP_BF16, FP_F32, FP_MXFP8, FP_MXFP4, FP_NVFP4 = 0, 1, 2, 3, 4
FP_OK, FP_ERR_INVALID_ARG, FP_ERR_UNSUPPORTED, FP_ERR_HIP, FP_ERR_WORKSPACE = range(5)
FP_PATH_NONE, FP_PATH_SKINNY, FP_PATH_SKINNY_SPLITK, FP_PATH_MFMA, FP_PATH_MFMA_SMALL = range(5)
FP_MAX_PROJ = 16
FP_MAX_M = 256

STATUS_NAMES = {
    FP_OK: "FP_OK", FP_ERR_INVALID_ARG: "FP_ERR_INVALID_ARG",
    FP_ERR_UNSUPPORTED: "FP_ERR_UNSUPPORTED", FP_ERR_HIP: "FP_ERR_HIP",
    FP_ERR_WORKSPACE: "FP_ERR_WORKSPACE",
}
PATH_NAMES = {FP_PATH_NONE: "none", FP_PATH_SKINNY: "skinny",
              FP_PATH_SKINNY_SPLITK: "skinny_splitk", FP_PATH_MFMA: "mfma",
              FP_PATH_MFMA_SMALL: "mfma_small"}


class FpTiling(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("kparts", ctypes.c_int32),
                ("chunks", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("groups", ctypes.c_int32)]

    def as_tuple(self):
        return (self.path, self.kparts, self.chunks, self.splits, self.rows, self.groups)


class FusedProjError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        extra = ""
        if status == FP_ERR_HIP:
            extra = ", hipError_t %d" % fp_last_hip_error()
        super().__init__("%s: %s (%s%s)" % (what, STATUS_NAMES.get(status, status),
                                            fp_status_str(status), extra))


if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libfusedproj.so is not built (expected at %s); build it with "
        "`python -m projection_gemm_sparse_amd.build` or __graft_entry__.build()"
        % LIB_PATH)

# torch ships its own libamdhip64.so.7.  Loading torch first makes the
# library's libamdhip64.so.7 dependency resolve (by soname) to that same
# runtime; loading the library first would bring in a second HIP runtime,
# and whichever initialises second sees no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_P_i64 = ctypes.POINTER(ctypes.c_int64)
_P_p = ctypes.POINTER(ctypes.c_void_p)
_P_i32 = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "fp_workspace_bytes": (ctypes.c_size_t, [_i32, _i64, _i32, _P_i64, _i64]),
    "fp_plan_create": (_i32, [_i32, _i64, _i32, _P_i64, _P_p, _p, _p, ctypes.c_size_t,
                              _i64, _p, ctypes.POINTER(_p)]),
    "fp_plan_view": (_i32, [_p, _i32, ctypes.POINTER(_p), _P_i64, _P_i64]),
    "fp_plan_destroy": (_i32, [_p]),
    "fp_supported": (_i32, [_p, _i64, _p, _i64]),
    "fp_forward": (_i32, [_p, _i64, _i64, _p, _p, _P_p]),
    "fp_forward_separate": (_i32, [_p, _i64, _i64, _p, _p, _P_p, _P_p]),
    "fp_forward_noalloc": (_i32, [_p, _i64, _i64, _p, _p, _P_p]),
    "fp_mxfp8_to_bf16": (_i32, [_p, _i64, _i64, _p, _p]),
    "fp_mxfp4_to_bf16": (_i32, [_p, _i64, _i64, _p, _p]),
    "fp_nvfp4_to_bf16": (_i32, [_p, _i64, _i64, ctypes.c_float, _p, _p]),
    "fp_plan_set_tensor_scales": (_i32, [_p, ctypes.POINTER(ctypes.c_float)]),
    "fp_stream_read": (_i32, [_p, _i64, _p, _p]),
    "fp_stream_read_shaped": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _p]),
    "fp_forward_rmsnorm": (_i32, [_p, _i64, _i64, _p, _p, _P_p, ctypes.c_float, _P_p]),
    "fp_forward_swiglu": (_i32, [_p, _i64, _i64, _p, _p, _p]),
    "fp_rmsnorm": (_i32, [_p, _i64, _i64, _p, ctypes.c_float, _p, _p]),
    "fp_swiglu": (_i32, [_p, _p, _i64, _i64, _p, _p]),
    "fp_plan_query": (_i32, [_p, _i64, _P_i32, _P_i32, _P_i32]),
    "fp_plan_set_out_dtype": (_i32, [_p, _i32]),
    "fp_plan_set_mfma_min_m": (_i32, [_p, _i64]),
    "fp_plan_set_tiling": (_i32, [_p, _i64, ctypes.POINTER(FpTiling)]),
    "fp_plan_get_tiling": (_i32, [_p, _i64, _i64, ctypes.POINTER(FpTiling)]),
    "fp_default_tiling": (_i32, [_i32, _i64, _i64, _i64, _i64, ctypes.POINTER(FpTiling)]),
    "fp_status_str": (ctypes.c_char_p, [_i32]),
    "fp_last_hip_error": (_i32, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def header_functions(path: str = HEADER) -> list:
    """Names of the functions include/fusedproj.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z_0-9]+)\s*\(", text)))


def _i64_array(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _ptr_array(vals):
    return (ctypes.c_void_p * len(vals))(*[None if v is None else int(v) for v in vals])


# ----------------------------------------------------- entry points (same names)
def fp_workspace_bytes(dtype: int, K: int, N, max_M: int) -> int:
    return int(_lib.fp_workspace_bytes(dtype, K, len(N), _i64_array(N), max_M))


def fp_plan_create(dtype: int, K: int, N, w_src, w_cat: int, workspace: int,
                   ws_bytes: int, max_M: int, stream: int):
    """Returns (status, plan handle or None).  ``w_src`` is None or a list of
    device pointers (None entries allowed)."""
    out = _p()
    src = None if w_src is None else _ptr_array(w_src)
    st = _lib.fp_plan_create(dtype, K, len(N), _i64_array(N), src, w_cat, workspace,
                             ws_bytes, max_M, stream, ctypes.byref(out))
    return st, (out.value if st == FP_OK else None)


def fp_plan_view(plan: int, i: int):
    w, off, rows = _p(), ctypes.c_int64(), ctypes.c_int64()
    st = _lib.fp_plan_view(plan, i, ctypes.byref(w), ctypes.byref(off), ctypes.byref(rows))
    return st, w.value, off.value, rows.value


def fp_plan_destroy(plan: int) -> int:
    return _lib.fp_plan_destroy(plan)


def fp_supported(plan: int, M: int, x: int, ldx: int) -> int:
    return _lib.fp_supported(plan, M, x, ldx)


def fp_forward(x: int, M: int, ldx: int, plan: int, stream: int, y) -> int:
    return _lib.fp_forward(x, M, ldx, plan, stream, _ptr_array(y))


def fp_forward_separate(x: int, M: int, ldx: int, plan: int, stream: int, y,
                        w_override=None) -> int:
    ov = None if w_override is None else _ptr_array(w_override)
    return _lib.fp_forward_separate(x, M, ldx, plan, stream, _ptr_array(y), ov)


def fp_forward_noalloc(x: int, M: int, ldx: int, plan: int, stream: int, y) -> int:
    return _lib.fp_forward_noalloc(x, M, ldx, plan, stream, _ptr_array(y))


def fp_mxfp8_to_bf16(w: int, rows: int, K: int, out: int, stream: int) -> int:
    return _lib.fp_mxfp8_to_bf16(w, rows, K, out, stream)


def fp_mxfp4_to_bf16(w: int, rows: int, K: int, out: int, stream: int) -> int:
    return _lib.fp_mxfp4_to_bf16(w, rows, K, out, stream)


def fp_nvfp4_to_bf16(w: int, rows: int, K: int, g: float, out: int, stream: int) -> int:
    return _lib.fp_nvfp4_to_bf16(w, rows, K, float(g), out, stream)


def fp_plan_set_tensor_scales(plan: int, scales) -> int:
    """``scales``: one fp32 tensor scale per projection (host values), or
    None (passed as a null pointer)."""
    if scales is None:
        return _lib.fp_plan_set_tensor_scales(plan, None)
    arr = (ctypes.c_float * len(scales))(*[float(v) for v in scales])
    return _lib.fp_plan_set_tensor_scales(plan, arr)


def fp_stream_read(buf: int, nbytes: int, sink: int, stream: int) -> int:
    return _lib.fp_stream_read(buf, nbytes, sink, stream)


def fp_stream_read_shaped(buf: int, nbytes: int, groups: int, threads: int, batch: int,
                          sink: int, stream: int) -> int:
    return _lib.fp_stream_read_shaped(buf, nbytes, groups, threads, batch, sink, stream)


def fp_forward_rmsnorm(x: int, M: int, ldx: int, plan: int, stream: int, gamma, eps: float,
                       out) -> int:
    """``gamma``: per projection a device pointer or None (not normalised)."""
    return _lib.fp_forward_rmsnorm(x, M, ldx, plan, stream, _ptr_array(gamma), float(eps),
                                   _ptr_array(out))


def fp_forward_swiglu(x: int, M: int, ldx: int, plan: int, stream: int, h: int) -> int:
    return _lib.fp_forward_swiglu(x, M, ldx, plan, stream, h)


def fp_rmsnorm(y: int, M: int, N: int, gamma: int, eps: float, out: int, stream: int) -> int:
    return _lib.fp_rmsnorm(y, M, N, gamma, float(eps), out, stream)


def fp_swiglu(g: int, u: int, M: int, N: int, h: int, stream: int) -> int:
    return _lib.fp_swiglu(g, u, M, N, h, stream)


def fp_plan_query(plan: int, M: int):
    path, lf, ls = _i32(), _i32(), _i32()
    st = _lib.fp_plan_query(plan, M, ctypes.byref(path), ctypes.byref(lf), ctypes.byref(ls))
    return st, path.value, lf.value, ls.value


def fp_plan_set_out_dtype(plan: int, out_dtype: int) -> int:
    return _lib.fp_plan_set_out_dtype(plan, out_dtype)


def fp_plan_set_mfma_min_m(plan: int, min_m: int) -> int:
    return _lib.fp_plan_set_mfma_min_m(plan, min_m)


def fp_plan_set_tiling(plan: int, M: int, tiling) -> int:
    """``tiling``: None (restore default) or a 6-tuple
    (path, kparts, chunks, splits, rows, groups)."""
    if tiling is None:
        return _lib.fp_plan_set_tiling(plan, M, None)
    t = FpTiling(*[int(v) for v in tiling])
    return _lib.fp_plan_set_tiling(plan, M, ctypes.byref(t))


def fp_plan_get_tiling(plan: int, M: int, n_rows: int):
    t = FpTiling()
    st = _lib.fp_plan_get_tiling(plan, M, n_rows, ctypes.byref(t))
    return st, t.as_tuple()


def fp_default_tiling(dtype: int, K: int, n_total: int, M: int, n_rows: int):
    t = FpTiling()
    st = _lib.fp_default_tiling(dtype, K, n_total, M, n_rows, ctypes.byref(t))
    return st, t.as_tuple()


def fp_status_str(status: int) -> str:
    return _lib.fp_status_str(status).decode()


def fp_last_hip_error() -> int:
    return _lib.fp_last_hip_error()


def check(status: int, what: str) -> None:
    if status != FP_OK:
        raise FusedProjError(status, what)
