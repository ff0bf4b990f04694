"""ctypes declarations of the C ABI in include/xtvxy.h (argument marshalling only).

Every function here has the name and the argument list of its C counterpart;
pointers are passed as Python ints (device addresses) and a nonzero status
raises XtvxyError. The library must have been built (``build.py``); there is no
fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

XTVXY_SUCCESS = 0
XTVXY_ERROR_INVALID_VALUE = 1
XTVXY_ERROR_NULL_POINTER = 2
XTVXY_ERROR_ALIASING = 3
XTVXY_ERROR_WORKSPACE = 4
XTVXY_ERROR_UNSUPPORTED = 5
XTVXY_ERROR_LAUNCH = 6
XTVXY_ERROR_LIBRARY = 7

XTVXY_DENSE_WAVE_ROWS = 1
XTVXY_DENSE_BLOCK_ROWS = 2
XTVXY_DENSE_GROUP_ROWS = 3
XTVXY_CSR_TILES = 11
XTVXY_CSR_WAVES = 12
XTVXY_CSR_ROWS = 13

XTVXY_PROBE_ATOMIC_PER_XCD = 0
XTVXY_PROBE_ATOMIC_DEVICE = 1
XTVXY_PROBE_ITEM_STORES = 2
XTVXY_PROBE_GATHERS = 3


class xtvxy_device_info(ctypes.Structure):
    _fields_ = [("compute_units", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("l2_bytes", ctypes.c_int32), ("xcds", ctypes.c_int32),
                ("hbm_bytes_per_s", ctypes.c_double)]


class xtvxy_launch_params(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("vec", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("lanes_per_row", ctypes.c_int32), ("chunks", ctypes.c_int32), ("group", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("rows_per_unit", ctypes.c_int64),
                ("entries_per_thread", ctypes.c_int32), ("lds_window", ctypes.c_int32),
                ("y_window", ctypes.c_int32), ("bin_columns", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("predicted_seconds", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


XTVXY_UNFUSED_TRANSPOSE_OP = 0
XTVXY_UNFUSED_EXPLICIT_TRANSPOSE = 1

XTVXY_LOGREG_FUSED = 0
XTVXY_LOGREG_UNFUSED = 1
XTVXY_LOGREG_CONVERGED = 0
XTVXY_LOGREG_ITERATION_LIMIT = 1
XTVXY_LOGREG_LINE_SEARCH_FAILED = 2


class xtvxy_logreg_options(ctypes.Structure):
    _fields_ = [("lambda_", ctypes.c_float), ("max_newton", ctypes.c_int32), ("max_cg", ctypes.c_int32),
                ("max_backtracks", ctypes.c_int32), ("grad_tol", ctypes.c_double), ("cg_forcing", ctypes.c_double),
                ("fixed_cg", ctypes.c_int32), ("engine", ctypes.c_int32)]


class xtvxy_logreg_report(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("newton_iterations", ctypes.c_int32),
                ("cg_iterations", ctypes.c_int32), ("line_search_trials", ctypes.c_int32),
                ("loss0", ctypes.c_double), ("loss", ctypes.c_double), ("grad_norm0", ctypes.c_double),
                ("grad_norm", ctypes.c_double), ("seconds", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class xtvxy_tune_report(ctypes.Structure):
    _fields_ = [("model", xtvxy_launch_params), ("best", xtvxy_launch_params), ("model_seconds", ctypes.c_double),
                ("best_seconds", ctypes.c_double), ("candidates", ctypes.c_int32), ("from_cache", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {"model": self.model.as_dict(), "best": self.best.as_dict(), "model_seconds": self.model_seconds,
                "best_seconds": self.best_seconds, "candidates": self.candidates, "from_cache": self.from_cache}


class XtvxyError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = int(status)
        name = _lib.xtvxy_status_string(self.status).decode() if _lib is not None else str(status)
        super().__init__("%s returned %s" % (where or "xtvxy", name))


_i64, _f32, _vp, _sz, _i32 = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_P = ctypes.POINTER

# name -> argument types (all return xtvxy_status, an int)
SIGNATURES = {
    "xtvxy_get_device_info": [_i32, _P(xtvxy_device_info)],
    "xtvxy_dense_f32_plan": [_i64, _i64, _i64, _i32, _P(xtvxy_device_info), _P(xtvxy_launch_params)],
    "xtvxy_dense_f32_plan_complete": [_i64, _i64, _i64, _P(xtvxy_device_info), _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_plan": [_i64, _i64, _i64, _P(xtvxy_device_info), _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_plan_rows": [_i64, _i64, _i64, _i64, _P(xtvxy_device_info), _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_plan_complete": [_i64, _i64, _i64, _P(xtvxy_device_info), _P(xtvxy_launch_params)],
    "xtvxy_dense_f32_workspace_size": [_i64, _i64, _i64, _P(_sz)],
    "xtvxy_dense_f32": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_dense_f32_ex": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp,
                           _P(xtvxy_launch_params)],
    "xtvxy_dense_bf16_workspace_size": [_i64, _i64, _i64, _P(_sz)],
    "xtvxy_dense_bf16_plan": [_i64, _i64, _i64, _i32, _P(xtvxy_device_info), _P(xtvxy_launch_params)],
    "xtvxy_dense_bf16_plan_complete": [_i64, _i64, _i64, _P(xtvxy_device_info), _P(xtvxy_launch_params)],
    "xtvxy_dense_bf16": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_dense_bf16_ex": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp,
                            _P(xtvxy_launch_params)],
    "xtvxy_dense_f16": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_dense_f16_ex": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp,
                            _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_workspace_size": [_i64, _i64, _i64, _P(_sz)],
    "xtvxy_csr_f32": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_csr_bf16": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_csr_f32_ex": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp,
                         _P(xtvxy_launch_params)],
    "xtvxy_csr_bf16_ex": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp,
                         _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_rowdot": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp],
    "xtvxy_csr_f32_rowdot_ex": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp,
                                _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_tmv": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_csr_f32_tmv_ex": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp,
                             _P(xtvxy_launch_params)],
    "xtvxy_csr_bf16_rowdot": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp],
    "xtvxy_csr_bf16_rowdot_ex": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp,
                                 _P(xtvxy_launch_params)],
    "xtvxy_csr_bf16_tmv": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_csr_bf16_tmv_ex": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp,
                              _P(xtvxy_launch_params)],
    "xtvxy_csr_check": [_i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "xtvxy_dense_f32_unfused_reference_workspace_size": [_i64, _i64, _P(_sz)],
    "xtvxy_dense_f32_unfused_reference": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_dense_f32_transpose": [_i64, _i64, _vp, _i64, _vp, _i64, _vp],
    "xtvxy_dense_f32_unfused_reference_explicit": [_i64, _i64, _f32, _vp, _i64, _vp, _i64, _vp, _vp, _f32, _vp, _vp,
                                                   _vp, _sz, _vp],
    "xtvxy_csr_f32_unfused_plan_create": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _P(_vp)],
    "xtvxy_csr_f32_unfused_plan_destroy": [_vp],
    "xtvxy_csr_f32_unfused_plan_create_ex": [_i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _P(_vp)],
    "xtvxy_csr_f32_unfused_reference": [_vp, _f32, _vp, _vp, _f32, _vp, _vp, _vp],
    "xtvxy_set_kernel_timing_events": [_vp, _vp],
    "xtvxy_test_group_wait": [_i32, _i32],
    "xtvxy_csr_f32_analyse": [_i64, _i64, _i64, _vp, _vp, _vp, _P(_vp)],
    "xtvxy_csr_f32_analysis_destroy": [_vp],
    "xtvxy_csr_f32_analysed_plan": [_vp, _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_analysed_plan_complete": [_vp, _P(xtvxy_launch_params)],
    "xtvxy_csr_f32_analysed_workspace_size": [_vp, _P(_sz)],
    "xtvxy_csr_f32_analysed": [_vp, _f32, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_csr_f32_analysed_ex": [_vp, _f32, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp, _P(xtvxy_launch_params)],
    "xtvxy_csr_bf16_analysed": [_vp, _f32, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp],
    "xtvxy_csr_bf16_analysed_ex": [_vp, _f32, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp, _P(xtvxy_launch_params)],
    "xtvxy_read_probe": [_vp, _sz, _i64, _vp, _vp],
    "xtvxy_tile_stream_probe": [_vp, _vp, _i64, _i64, _i32, _vp, _vp],
    "xtvxy_scatter_probe": [_i32, _vp, _sz, ctypes.c_uint32, ctypes.c_uint32, _i32, _i64, _vp, _vp],
    "xtvxy_dense_f32_noalloc_max_workspace": [_P(_sz)],
    "xtvxy_dense_f32_noalloc": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _vp],
    "xtvxy_dense_f32_tune": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _i32, _vp,
                             _P(xtvxy_tune_report)],
    "xtvxy_dense_bf16_tune": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _i32, _vp,
                              _P(xtvxy_tune_report)],
    "xtvxy_csr_f32_tune": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _i32, _vp,
                           _P(xtvxy_tune_report)],
    "xtvxy_dense_f16_tune": [_i64, _i64, _f32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _i32, _vp,
                             _P(xtvxy_tune_report)],
    "xtvxy_csr_bf16_tune": [_i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _i32, _vp,
                            _P(xtvxy_tune_report)],
    "xtvxy_tune_cache_lookup": [_i32, _i64, _i64, _i64, _i32, _P(xtvxy_tune_report), _P(ctypes.c_int32)],
    "xtvxy_tune_cache_clear": [],
    "xtvxy_tune_cache_save": [ctypes.c_char_p],
    "xtvxy_tune_cache_load": [ctypes.c_char_p],
    "xtvxy_logreg_newton_cg_f32_workspace_size": [_i64, _i64, _i64, _P(_sz)],
    "xtvxy_logreg_newton_cg_f32": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _P(xtvxy_logreg_options), _vp, _vp,
                                   _sz, _vp, _P(xtvxy_logreg_report), _P(ctypes.c_double), _i64],
    "xtvxy_logreg_newton_cg_bf16": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _P(xtvxy_logreg_options), _vp, _sz,
                                    _vp, _P(xtvxy_logreg_report), _P(ctypes.c_double), _i64],
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libxtvxy.so and declare every exported entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libxtvxy.so is not built (%s); run `python -m dense_linear_algebra_alpha_amd.build`"
                           % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.xtvxy_status_string.argtypes = [_i32]
    lib.xtvxy_status_string.restype = ctypes.c_char_p
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def call(name: str, *args) -> int:
    """Call entry point `name`; raise XtvxyError on a nonzero status."""
    st = getattr(load(), name)(*args)
    if st != XTVXY_SUCCESS:
        raise XtvxyError(st, name)
    return st


def status_string(status: int) -> str:
    return load().xtvxy_status_string(int(status)).decode()
