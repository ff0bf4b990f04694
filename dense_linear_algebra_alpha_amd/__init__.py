"""Python binding of the xtvxy C ABI (include/xtvxy.h).

Evaluates out = alpha * X^T (v .* (X y)) + beta * z — the generic pattern of
"On optimizing machine learning workloads via kernel fusion" (abstract) — for
dense row-major or CSR fp32 X on an AMD gfx950 GPU, in one fused pass of
hand-written HIP kernels (libxtvxy.so), or through the operator-level library
comparator.

Two layers, both argument marshalling only:
  * ``xtvxy_*`` functions with the C names and argument lists (device pointers
    as ints, the stream as an int handle);
  * tensor helpers (``dense``, ``csr``, ``dense_unfused``, ``CsrUnfusedPlan``)
    that take torch CUDA tensors, allocate the workspace with torch, and call
    the C entry points on the current torch stream.
Every computation happens in the library's kernels; a missing library raises.
"""
from __future__ import annotations

import ctypes

from . import _abi
from ._abi import (XTVXY_CSR_ROWS, XTVXY_CSR_TILES, XTVXY_CSR_WAVES, XTVXY_DENSE_BLOCK_ROWS, XTVXY_DENSE_GROUP_ROWS,  # noqa: F401
                   XTVXY_DENSE_WAVE_ROWS, XTVXY_LOGREG_CONVERGED, XTVXY_LOGREG_FUSED, XTVXY_PROBE_ATOMIC_DEVICE,
                   XTVXY_PROBE_ATOMIC_PER_XCD, XTVXY_PROBE_GATHERS, XTVXY_PROBE_ITEM_STORES,
                   XTVXY_UNFUSED_EXPLICIT_TRANSPOSE, XTVXY_UNFUSED_TRANSPOSE_OP,
                   XTVXY_LOGREG_ITERATION_LIMIT, XTVXY_LOGREG_LINE_SEARCH_FAILED, XTVXY_LOGREG_UNFUSED, XtvxyError,
                   xtvxy_device_info, xtvxy_launch_params, xtvxy_logreg_options, xtvxy_logreg_report,
                   xtvxy_tune_report)

__all__ = [
    "xtvxy_get_device_info", "xtvxy_dense_f32_plan", "xtvxy_dense_f32_plan_complete", "xtvxy_csr_f32_plan",
    "xtvxy_csr_f32_plan_complete", "xtvxy_csr_f32_plan_rows", "xtvxy_dense_f32_workspace_size", "xtvxy_dense_f32", "xtvxy_dense_f32_ex",
    "xtvxy_csr_f32_workspace_size", "xtvxy_csr_f32", "xtvxy_csr_f32_ex", "xtvxy_csr_check",
    "xtvxy_dense_f32_unfused_reference_workspace_size", "xtvxy_dense_f32_unfused_reference",
    "xtvxy_dense_f32_transpose", "xtvxy_dense_f32_unfused_reference_explicit",
    "xtvxy_csr_f32_unfused_plan_create", "xtvxy_csr_f32_unfused_plan_destroy", "xtvxy_csr_f32_unfused_reference",
    "xtvxy_status_string", "xtvxy_set_kernel_timing_events", "xtvxy_test_group_wait", "xtvxy_read_probe", "xtvxy_scatter_probe",
    "xtvxy_dense_f32_noalloc", "xtvxy_dense_f32_noalloc_max_workspace", "XtvxyError", "xtvxy_device_info", "xtvxy_launch_params",
    "dense", "csr", "csr_tensor", "dense_unfused", "dense_transpose", "CsrUnfusedPlan", "csr_check", "dense_plan", "csr_plan", "load",
    "xtvxy_csr_f32_rowdot", "xtvxy_csr_f32_rowdot_ex", "xtvxy_csr_f32_tmv", "xtvxy_csr_f32_tmv_ex", "csr_rowdot",
    "csr_tmv", "xtvxy_logreg_newton_cg_f32_workspace_size", "xtvxy_logreg_newton_cg_f32", "logreg_newton_cg",
    "xtvxy_logreg_options", "xtvxy_logreg_report", "xtvxy_csr_f32_unfused_plan_create_ex",
    "xtvxy_dense_f32_tune", "xtvxy_csr_f32_tune", "xtvxy_tune_cache_lookup", "xtvxy_tune_cache_clear",
    "xtvxy_tune_cache_save", "xtvxy_tune_cache_load", "xtvxy_tune_report", "dense_tune", "csr_tune",
    "xtvxy_dense_bf16_workspace_size", "xtvxy_dense_bf16_plan", "xtvxy_dense_bf16_plan_complete",
    "xtvxy_dense_bf16", "xtvxy_dense_bf16_ex", "xtvxy_dense_bf16_tune",
    "xtvxy_csr_f32_analyse", "xtvxy_csr_f32_analysis_destroy", "xtvxy_csr_f32_analysed_plan",
    "xtvxy_csr_f32_analysed_plan_complete", "xtvxy_csr_f32_analysed_workspace_size", "xtvxy_csr_f32_analysed",
    "xtvxy_csr_f32_analysed_ex", "CsrAnalysis", "xtvxy_csr_bf16", "xtvxy_csr_bf16_ex", "xtvxy_csr_bf16_analysed",
    "xtvxy_csr_bf16_analysed_ex", "xtvxy_dense_f16", "xtvxy_dense_f16_ex", "xtvxy_csr_bf16_rowdot",
    "xtvxy_csr_bf16_rowdot_ex", "xtvxy_csr_bf16_tmv", "xtvxy_csr_bf16_tmv_ex", "xtvxy_logreg_newton_cg_bf16",
    "xtvxy_tile_stream_probe", "xtvxy_dense_f16_tune", "xtvxy_csr_bf16_tune",
]

load = _abi.load


# ---------------------------------------------------------------------------
# C names
# ---------------------------------------------------------------------------

def xtvxy_status_string(status: int) -> str:
    return _abi.status_string(status)


def xtvxy_set_kernel_timing_events(before_main, after_main):
    return _abi.call("xtvxy_set_kernel_timing_events", before_main, after_main)


def xtvxy_test_group_wait(polls: int, unanswered: int):
    return _abi.call("xtvxy_test_group_wait", int(polls), int(unanswered))


def xtvxy_dense_f32_noalloc_max_workspace() -> int:
    b = ctypes.c_size_t()
    _abi.call("xtvxy_dense_f32_noalloc_max_workspace", ctypes.byref(b))
    return b.value


def xtvxy_dense_f32_noalloc(m, n, alpha, X, ldx, v, y, beta, z, out, stream):
    return _abi.call("xtvxy_dense_f32_noalloc", m, n, alpha, X, ldx, v, y, beta, z, out, stream)


def xtvxy_read_probe(buffer, nbytes, grid, sink, stream):
    return _abi.call("xtvxy_read_probe", buffer, nbytes, grid, sink, stream)


def xtvxy_scatter_probe(kind, buffer, nbytes, n, items, skew, grid, sink, stream):
    return _abi.call("xtvxy_scatter_probe", kind, buffer, nbytes, n, items, skew, grid, sink, stream)


def xtvxy_get_device_info(device: int = -1) -> xtvxy_device_info:
    info = xtvxy_device_info()
    _abi.call("xtvxy_get_device_info", device, ctypes.byref(info))
    return info


def xtvxy_dense_f32_plan(m, n, ldx, X_aligned16=1, dev=None) -> xtvxy_launch_params:
    p = xtvxy_launch_params()
    _abi.call("xtvxy_dense_f32_plan", m, n, ldx, int(X_aligned16), ctypes.byref(dev) if dev else None,
              ctypes.byref(p))
    return p


def xtvxy_dense_f32_plan_complete(m, n, ldx, plan: xtvxy_launch_params, dev=None) -> xtvxy_launch_params:
    _abi.call("xtvxy_dense_f32_plan_complete", m, n, ldx, ctypes.byref(dev) if dev else None, ctypes.byref(plan))
    return plan


def xtvxy_dense_bf16_plan(m, n, ldx, X_aligned16=1, dev=None) -> xtvxy_launch_params:
    p = xtvxy_launch_params()
    _abi.call("xtvxy_dense_bf16_plan", m, n, ldx, int(X_aligned16), ctypes.byref(dev) if dev else None,
              ctypes.byref(p))
    return p


def xtvxy_dense_bf16_plan_complete(m, n, ldx, plan: xtvxy_launch_params, dev=None) -> xtvxy_launch_params:
    _abi.call("xtvxy_dense_bf16_plan_complete", m, n, ldx, ctypes.byref(dev) if dev else None, ctypes.byref(plan))
    return plan


def xtvxy_dense_bf16_workspace_size(m, n, ldx) -> int:
    b = ctypes.c_size_t()
    _abi.call("xtvxy_dense_bf16_workspace_size", m, n, ldx, ctypes.byref(b))
    return b.value


def xtvxy_dense_bf16(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream):
    return _abi.call("xtvxy_dense_bf16", m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes,
                     stream)


def xtvxy_dense_bf16_ex(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, force):
    return _abi.call("xtvxy_dense_bf16_ex", m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes,
                     stream, ctypes.byref(force) if force is not None else None)


def xtvxy_dense_f16(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream):
    return _abi.call("xtvxy_dense_f16", m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes,
                     stream)


def xtvxy_dense_f16_ex(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, force):
    return _abi.call("xtvxy_dense_f16_ex", m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes,
                     stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_f32_plan(m, n, nnz, dev=None) -> xtvxy_launch_params:
    p = xtvxy_launch_params()
    _abi.call("xtvxy_csr_f32_plan", m, n, nnz, ctypes.byref(dev) if dev else None, ctypes.byref(p))
    return p


def xtvxy_csr_f32_plan_rows(m, n, nnz, longest_row, dev=None) -> xtvxy_launch_params:
    p = xtvxy_launch_params()
    _abi.call("xtvxy_csr_f32_plan_rows", m, n, nnz, longest_row, ctypes.byref(dev) if dev else None, ctypes.byref(p))
    return p


def xtvxy_csr_f32_plan_complete(m, n, nnz, plan: xtvxy_launch_params, dev=None) -> xtvxy_launch_params:
    _abi.call("xtvxy_csr_f32_plan_complete", m, n, nnz, ctypes.byref(dev) if dev else None, ctypes.byref(plan))
    return plan


def xtvxy_dense_f32_workspace_size(m, n, ldx) -> int:
    b = ctypes.c_size_t()
    _abi.call("xtvxy_dense_f32_workspace_size", m, n, ldx, ctypes.byref(b))
    return b.value


def xtvxy_csr_f32_workspace_size(m, n, nnz) -> int:
    b = ctypes.c_size_t()
    _abi.call("xtvxy_csr_f32_workspace_size", m, n, nnz, ctypes.byref(b))
    return b.value


def xtvxy_dense_f32_unfused_reference_workspace_size(m, n) -> int:
    b = ctypes.c_size_t()
    _abi.call("xtvxy_dense_f32_unfused_reference_workspace_size", m, n, ctypes.byref(b))
    return b.value


def xtvxy_dense_f32(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream):
    return _abi.call("xtvxy_dense_f32", m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes,
                     stream)


def xtvxy_dense_f32_ex(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, force):
    return _abi.call("xtvxy_dense_f32_ex", m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes,
                     stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_f32(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                  stream):
    return _abi.call("xtvxy_csr_f32", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace,
                     workspace_bytes, stream)


def xtvxy_csr_f32_ex(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                     stream, force):
    return _abi.call("xtvxy_csr_f32_ex", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out,
                     workspace, workspace_bytes, stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_bf16(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                   stream):
    return _abi.call("xtvxy_csr_bf16", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace,
                     workspace_bytes, stream)


def xtvxy_csr_bf16_ex(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                      stream, force):
    return _abi.call("xtvxy_csr_bf16_ex", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out,
                     workspace, workspace_bytes, stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_f32_rowdot(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream):
    return _abi.call("xtvxy_csr_f32_rowdot", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream)


def xtvxy_csr_f32_rowdot_ex(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream, force):
    return _abi.call("xtvxy_csr_f32_rowdot_ex", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t,
                     stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_f32_tmv(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes,
                      stream):
    return _abi.call("xtvxy_csr_f32_tmv", m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace,
                     workspace_bytes, stream)


def xtvxy_csr_f32_tmv_ex(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes,
                         stream, force):
    return _abi.call("xtvxy_csr_f32_tmv_ex", m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out,
                     workspace, workspace_bytes, stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_bf16_rowdot(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream):
    return _abi.call("xtvxy_csr_bf16_rowdot", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream)


def xtvxy_csr_bf16_rowdot_ex(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream, force):
    return _abi.call("xtvxy_csr_bf16_rowdot_ex", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t,
                     stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_bf16_tmv(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes,
                       stream):
    return _abi.call("xtvxy_csr_bf16_tmv", m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace,
                     workspace_bytes, stream)


def xtvxy_csr_bf16_tmv_ex(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes,
                          stream, force):
    return _abi.call("xtvxy_csr_bf16_tmv_ex", m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out,
                     workspace, workspace_bytes, stream, ctypes.byref(force) if force is not None else None)


def xtvxy_tile_stream_probe(indices, values, entries, grid, interleave, sink, stream):
    return _abi.call("xtvxy_tile_stream_probe", indices, values, entries, grid, interleave, sink, stream)


def xtvxy_csr_f32_analyse(m, n, nnz, row_ptr, col_idx, stream) -> int:
    h = ctypes.c_void_p()
    _abi.call("xtvxy_csr_f32_analyse", m, n, nnz, row_ptr, col_idx, stream, ctypes.byref(h))
    return h.value or 0


def xtvxy_csr_f32_analysis_destroy(analysis):
    return _abi.call("xtvxy_csr_f32_analysis_destroy", analysis)


def xtvxy_csr_f32_analysed_plan(analysis) -> xtvxy_launch_params:
    p = xtvxy_launch_params()
    _abi.call("xtvxy_csr_f32_analysed_plan", analysis, ctypes.byref(p))
    return p


def xtvxy_csr_f32_analysed_plan_complete(analysis, plan: xtvxy_launch_params) -> xtvxy_launch_params:
    _abi.call("xtvxy_csr_f32_analysed_plan_complete", analysis, ctypes.byref(plan))
    return plan


def xtvxy_csr_f32_analysed_workspace_size(analysis) -> int:
    b = ctypes.c_size_t()
    _abi.call("xtvxy_csr_f32_analysed_workspace_size", analysis, ctypes.byref(b))
    return b.value


def xtvxy_csr_f32_analysed(analysis, alpha, values, v, y, beta, z, out, workspace, workspace_bytes, stream):
    return _abi.call("xtvxy_csr_f32_analysed", analysis, alpha, values, v, y, beta, z, out, workspace,
                     workspace_bytes, stream)


def xtvxy_csr_f32_analysed_ex(analysis, alpha, values, v, y, beta, z, out, workspace, workspace_bytes, stream,
                              force):
    return _abi.call("xtvxy_csr_f32_analysed_ex", analysis, alpha, values, v, y, beta, z, out, workspace,
                     workspace_bytes, stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_bf16_analysed(analysis, alpha, values, v, y, beta, z, out, workspace, workspace_bytes, stream):
    return _abi.call("xtvxy_csr_bf16_analysed", analysis, alpha, values, v, y, beta, z, out, workspace,
                     workspace_bytes, stream)


def xtvxy_csr_bf16_analysed_ex(analysis, alpha, values, v, y, beta, z, out, workspace, workspace_bytes, stream,
                               force):
    return _abi.call("xtvxy_csr_bf16_analysed_ex", analysis, alpha, values, v, y, beta, z, out, workspace,
                     workspace_bytes, stream, ctypes.byref(force) if force is not None else None)


def xtvxy_csr_check(m, n, nnz, row_ptr, col_idx, d_flag, stream):
    return _abi.call("xtvxy_csr_check", m, n, nnz, row_ptr, col_idx, d_flag, stream)


def xtvxy_dense_f32_unfused_reference(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes,
                                      stream):
    return _abi.call("xtvxy_dense_f32_unfused_reference", m, n, alpha, X, ldx, v, y, beta, z, out, workspace,
                     workspace_bytes, stream)


def xtvxy_dense_f32_transpose(m, n, X, ldx, Xt, ldxt, stream):
    return _abi.call("xtvxy_dense_f32_transpose", m, n, X, ldx, Xt, ldxt, stream)


def xtvxy_dense_f32_unfused_reference_explicit(m, n, alpha, X, ldx, Xt, ldxt, v, y, beta, z, out, workspace,
                                               workspace_bytes, stream):
    return _abi.call("xtvxy_dense_f32_unfused_reference_explicit", m, n, alpha, X, ldx, Xt, ldxt, v, y, beta, z, out,
                     workspace, workspace_bytes, stream)


def xtvxy_csr_f32_unfused_plan_create(m, n, nnz, row_ptr, col_idx, values, stream) -> int:
    h = ctypes.c_void_p()
    _abi.call("xtvxy_csr_f32_unfused_plan_create", m, n, nnz, row_ptr, col_idx, values, stream, ctypes.byref(h))
    return h.value or 0


def xtvxy_csr_f32_unfused_plan_create_ex(m, n, nnz, row_ptr, col_idx, values, options, stream) -> int:
    h = ctypes.c_void_p()
    _abi.call("xtvxy_csr_f32_unfused_plan_create_ex", m, n, nnz, row_ptr, col_idx, values, int(options), stream,
              ctypes.byref(h))
    return h.value or 0


def xtvxy_csr_f32_unfused_plan_destroy(plan: int):
    return _abi.call("xtvxy_csr_f32_unfused_plan_destroy", plan)


def xtvxy_csr_f32_unfused_reference(plan, alpha, v, y, beta, z, out, stream):
    return _abi.call("xtvxy_csr_f32_unfused_reference", plan, alpha, v, y, beta, z, out, stream)


def xtvxy_dense_f32_tune(m, n, alpha, X, ldx, v, y, beta, z, out, repeats, stream) -> xtvxy_tune_report:
    rep = xtvxy_tune_report()
    _abi.call("xtvxy_dense_f32_tune", m, n, alpha, X, ldx, v, y, beta, z, out, int(repeats), stream,
              ctypes.byref(rep))
    return rep


def xtvxy_dense_bf16_tune(m, n, alpha, X, ldx, v, y, beta, z, out, repeats, stream) -> xtvxy_tune_report:
    rep = xtvxy_tune_report()
    _abi.call("xtvxy_dense_bf16_tune", m, n, alpha, X, ldx, v, y, beta, z, out, int(repeats), stream,
              ctypes.byref(rep))
    return rep


def xtvxy_csr_f32_tune(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, repeats,
                       stream) -> xtvxy_tune_report:
    rep = xtvxy_tune_report()
    _abi.call("xtvxy_csr_f32_tune", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, int(repeats),
              stream, ctypes.byref(rep))
    return rep


def xtvxy_csr_bf16_tune(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, repeats,
                        stream) -> xtvxy_tune_report:
    rep = xtvxy_tune_report()
    _abi.call("xtvxy_csr_bf16_tune", m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, int(repeats),
              stream, ctypes.byref(rep))
    return rep


def xtvxy_dense_f16_tune(m, n, alpha, X, ldx, v, y, beta, z, out, repeats, stream) -> xtvxy_tune_report:
    rep = xtvxy_tune_report()
    _abi.call("xtvxy_dense_f16_tune", m, n, alpha, X, ldx, v, y, beta, z, out, int(repeats), stream,
              ctypes.byref(rep))
    return rep


def xtvxy_tune_cache_lookup(kind, m, n, k, aligned):
    """(report, found) for a shape on the current device."""
    rep = xtvxy_tune_report()
    found = ctypes.c_int32()
    _abi.call("xtvxy_tune_cache_lookup", int(kind), m, n, k, int(aligned), ctypes.byref(rep), ctypes.byref(found))
    return rep, bool(found.value)


def xtvxy_tune_cache_clear():
    return _abi.call("xtvxy_tune_cache_clear")


def xtvxy_tune_cache_save(path: str):
    return _abi.call("xtvxy_tune_cache_save", path.encode())


def xtvxy_tune_cache_load(path: str):
    return _abi.call("xtvxy_tune_cache_load", path.encode())


def xtvxy_logreg_newton_cg_f32_workspace_size(m, n, nnz) -> int:
    b = ctypes.c_size_t()
    _abi.call("xtvxy_logreg_newton_cg_f32_workspace_size", m, n, nnz, ctypes.byref(b))
    return b.value


def xtvxy_logreg_newton_cg_f32(m, n, nnz, row_ptr, col_idx, values, labels, w, opt, unfused, workspace,
                               workspace_bytes, stream, report, history, history_rows):
    return _abi.call("xtvxy_logreg_newton_cg_f32", m, n, nnz, row_ptr, col_idx, values, labels, w,
                     ctypes.byref(opt), unfused, workspace, workspace_bytes, stream,
                     ctypes.byref(report) if report is not None else None, history, history_rows)


def xtvxy_logreg_newton_cg_bf16(m, n, nnz, row_ptr, col_idx, values, labels, w, opt, workspace, workspace_bytes,
                                stream, report, history, history_rows):
    return _abi.call("xtvxy_logreg_newton_cg_bf16", m, n, nnz, row_ptr, col_idx, values, labels, w,
                     ctypes.byref(opt), workspace, workspace_bytes, stream,
                     ctypes.byref(report) if report is not None else None, history, history_rows)


# ---------------------------------------------------------------------------
# torch tensor helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> int | None:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _check_vec(name, t, length, device, required=True):
    torch = _torch()
    if t is None:
        if required:
            raise ValueError("%s is required" % name)
        return
    if t.dtype != torch.float32 or t.device != device or t.numel() != length or not t.is_contiguous():
        raise ValueError("%s must be a contiguous float32 tensor of %d elements on %s" % (name, length, device))


def _workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def _keep_for_stream(stream, *tensors):
    """Tensors allocated here on the current stream but used by kernels launched on `stream`: tell
    the caching allocator, so that their memory is not handed out again before that stream has
    passed the call (it would otherwise be reusable as soon as the helper returns)."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def dense_plan(m, n, ldx=None, aligned=True, dev=None, bf16=False) -> xtvxy_launch_params:
    fn = xtvxy_dense_bf16_plan if bf16 else xtvxy_dense_f32_plan
    return fn(m, n, n if ldx is None else ldx, 1 if aligned else 0, dev)


def csr_plan(m, n, nnz, dev=None) -> xtvxy_launch_params:
    return xtvxy_csr_f32_plan(m, n, nnz, dev)


def dense(X, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, *, m=None, n=None, ldx=None, plan=None,
          workspace=None, stream=None):
    """out = alpha X^T (v .* (X y)) + beta z for dense row-major X on the GPU.

    X is a 2-D CUDA tensor with unit column stride (row stride = ldx), or a flat buffer with m,
    n and ldx given; float32, bf16 storage (torch.bfloat16, or uint16 bit patterns), which takes
    the xtvxy_dense_bf16 entry points, or fp16 storage (torch.float16: xtvxy_dense_f16).
    ``plan`` forces launch parameters."""
    torch = _torch()
    if X.dim() == 2 and m is None:
        m, n = X.shape
        if X.stride(1) != 1 and n > 1:
            raise ValueError("X needs unit column stride")
        ldx = X.stride(0) if m > 1 else max(n, 1)
        ldx = max(ldx, n, 1)
    if m is None or n is None or ldx is None:
        raise ValueError("flat X needs m, n and ldx")
    bf16 = X.dtype in (torch.bfloat16, torch.uint16)
    f16 = X.dtype == torch.float16
    if X.dtype != torch.float32 and not bf16 and not f16:
        raise ValueError("X must be float32, bfloat16, uint16 (bf16 bits) or float16")
    device = X.device
    _check_vec("y", y, n, device)
    _check_vec("v", v, m, device, required=False)
    _check_vec("z", z, n, device, required=beta != 0)
    made_out = out is None
    if made_out:
        out = torch.empty(n, dtype=torch.float32, device=device)
    _check_vec("out", out, n, device)
    if plan is None:
        need = (xtvxy_dense_bf16_workspace_size if bf16 or f16 else xtvxy_dense_f32_workspace_size)(m, n, ldx)
    else:
        need = int(plan.workspace_bytes)
    made_ws = workspace is None
    if made_ws:
        workspace = _workspace(need, device)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    args = (m, n, float(alpha), X.data_ptr(), ldx, _ptr(v), y.data_ptr(), float(beta), _ptr(z), out.data_ptr(),
            ws_ptr, ws_bytes, _stream_handle(stream))
    if plan is None:
        (xtvxy_dense_f16 if f16 else xtvxy_dense_bf16 if bf16 else xtvxy_dense_f32)(*args)
    else:
        (xtvxy_dense_f16_ex if f16 else xtvxy_dense_bf16_ex if bf16 else xtvxy_dense_f32_ex)(*args, plan)
    _keep_for_stream(stream, out if made_out else None, workspace if made_ws else None)
    return out


def csr(row_ptr, col_idx, values, n, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, *, plan=None,
        workspace=None, stream=None):
    """The same pattern for CSR X given as int32 row_ptr / col_idx and float32 values tensors; bf16
    values (torch.bfloat16, or uint16 bit patterns) take the xtvxy_csr_bf16 entry points."""
    torch = _torch()
    m = row_ptr.numel() - 1
    nnz = col_idx.numel()
    device = row_ptr.device
    bf16 = values.dtype in (torch.bfloat16, torch.uint16)
    for name, t, dt in (("row_ptr", row_ptr, torch.int32), ("col_idx", col_idx, torch.int32),
                        ("values", values, values.dtype if bf16 else torch.float32)):
        if t.dtype != dt or t.device != device or not t.is_contiguous():
            raise ValueError("%s must be a contiguous %s tensor on %s" % (name, dt, device))
    if values.numel() != nnz:
        raise ValueError("values and col_idx differ in length")
    _check_vec("y", y, n, device)
    _check_vec("v", v, m, device, required=False)
    _check_vec("z", z, n, device, required=beta != 0)
    made_out = out is None
    if made_out:
        out = torch.empty(n, dtype=torch.float32, device=device)
    _check_vec("out", out, n, device)
    need = xtvxy_csr_f32_workspace_size(m, n, nnz) if plan is None else int(plan.workspace_bytes)
    made_ws = workspace is None
    if made_ws:
        workspace = _workspace(need, device)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    args = (m, n, nnz, float(alpha), row_ptr.data_ptr(), _ptr(col_idx) if nnz else None,
            _ptr(values) if nnz else None, _ptr(v), y.data_ptr(), float(beta), _ptr(z), out.data_ptr(), ws_ptr,
            ws_bytes, _stream_handle(stream))
    if plan is None:
        (xtvxy_csr_bf16 if bf16 else xtvxy_csr_f32)(*args)
    else:
        (xtvxy_csr_bf16_ex if bf16 else xtvxy_csr_f32_ex)(*args, plan)
    _keep_for_stream(stream, out if made_out else None, workspace if made_ws else None)
    return out


def csr_tensor(X, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, *, plan=None, workspace=None, stream=None):
    """csr() for X given as a torch sparse CSR tensor (torch.sparse_csr_tensor) with int32 indices
    and float32 (or bfloat16) values on the GPU; its crow_indices, col_indices and values are passed
    as they are."""
    torch = _torch()
    if X.layout != torch.sparse_csr or X.dim() != 2:
        raise ValueError("X must be a 2-D torch.sparse_csr tensor")
    rp, ci, vals = X.crow_indices(), X.col_indices(), X.values()
    if rp.dtype != torch.int32 or ci.dtype != torch.int32:
        raise ValueError("X's indices must be int32 (torch.sparse_csr_tensor(..., dtype=torch.float32) with int32 "
                         "crow_indices and col_indices)")
    return csr(rp, ci, vals, X.shape[1], y, v, z, alpha, beta, out, plan=plan, workspace=workspace, stream=stream)


def _is_bf16(values) -> bool:
    torch = _torch()
    return values.dtype in (torch.bfloat16, torch.uint16)


def _check_csr_arrays(row_ptr, col_idx, values, bf16_ok=False):
    torch = _torch()
    device = row_ptr.device
    vdt = values.dtype if bf16_ok and _is_bf16(values) else torch.float32
    for name, t, dt in (("row_ptr", row_ptr, torch.int32), ("col_idx", col_idx, torch.int32),
                        ("values", values, vdt)):
        if t.dtype != dt or t.device != device or not t.is_contiguous():
            raise ValueError("%s must be a contiguous %s tensor on %s" % (name, dt, device))
    if values.numel() != col_idx.numel():
        raise ValueError("values and col_idx differ in length")
    return row_ptr.numel() - 1, col_idx.numel(), device


def csr_rowdot(row_ptr, col_idx, values, n, y, v=None, t0=None, alpha=1.0, beta=0.0, out=None, *, plan=None,
               stream=None):
    """t = alpha v .* (X y) + beta t0 (the first half of the pattern) for CSR X; returns t. bf16
    values (torch.bfloat16, or uint16 bit patterns) take xtvxy_csr_bf16_rowdot."""
    torch = _torch()
    m, nnz, device = _check_csr_arrays(row_ptr, col_idx, values, bf16_ok=True)
    bf16 = _is_bf16(values)
    _check_vec("y", y, n, device)
    _check_vec("v", v, m, device, required=False)
    _check_vec("t0", t0, m, device, required=beta != 0)
    made_out = out is None
    if made_out:
        out = torch.empty(m, dtype=torch.float32, device=device)
    _check_vec("out", out, m, device)
    args = (m, n, nnz, float(alpha), row_ptr.data_ptr(), _ptr(col_idx) if nnz else None,
            _ptr(values) if nnz else None, _ptr(v), y.data_ptr(), float(beta), _ptr(t0), out.data_ptr(),
            _stream_handle(stream))
    if plan is None:
        (xtvxy_csr_bf16_rowdot if bf16 else xtvxy_csr_f32_rowdot)(*args)
    else:
        (xtvxy_csr_bf16_rowdot_ex if bf16 else xtvxy_csr_f32_rowdot_ex)(*args, plan)
    _keep_for_stream(stream, out if made_out else None)
    return out


def csr_tmv(row_ptr, col_idx, values, n, u, z=None, alpha=1.0, beta=0.0, out=None, *, plan=None, workspace=None,
            stream=None):
    """out = alpha X^T u + beta z (the second half of the pattern) for CSR X; returns out. bf16
    values (torch.bfloat16, or uint16 bit patterns) take xtvxy_csr_bf16_tmv."""
    torch = _torch()
    m, nnz, device = _check_csr_arrays(row_ptr, col_idx, values, bf16_ok=True)
    bf16 = _is_bf16(values)
    _check_vec("u", u, m, device)
    _check_vec("z", z, n, device, required=beta != 0)
    made_out = out is None
    if made_out:
        out = torch.empty(n, dtype=torch.float32, device=device)
    _check_vec("out", out, n, device)
    need = xtvxy_csr_f32_workspace_size(m, n, nnz) if plan is None else int(plan.workspace_bytes)
    made_ws = workspace is None
    if made_ws:
        workspace = _workspace(need, device)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    args = (m, n, nnz, float(alpha), row_ptr.data_ptr(), _ptr(col_idx) if nnz else None,
            _ptr(values) if nnz else None, u.data_ptr(), float(beta), _ptr(z), out.data_ptr(), ws_ptr, ws_bytes,
            _stream_handle(stream))
    if plan is None:
        (xtvxy_csr_bf16_tmv if bf16 else xtvxy_csr_f32_tmv)(*args)
    else:
        (xtvxy_csr_bf16_tmv_ex if bf16 else xtvxy_csr_f32_tmv_ex)(*args, plan)
    _keep_for_stream(stream, out if made_out else None, workspace if made_ws else None)
    return out


def csr_check(row_ptr, col_idx, n, stream=None) -> int:
    """Device-side structure check; returns 0 for a well-formed matrix (synchronizes)."""
    torch = _torch()
    flag = torch.zeros(1, dtype=torch.int32, device=row_ptr.device)
    xtvxy_csr_check(row_ptr.numel() - 1, n, col_idx.numel(), row_ptr.data_ptr(),
                    col_idx.data_ptr() if col_idx.numel() else None, flag.data_ptr(), _stream_handle(stream))
    if stream is not None:  # the check ran on `stream`; .item() below waits for the current stream only
        stream.synchronize()
    return int(flag.item())


def dense_transpose(X, stream=None):
    """X^T as a new row-major n x m fp32 tensor (rocBLAS sgeam): the comparator's copy of X^T."""
    torch = _torch()
    m, n = X.shape
    ldx = max(X.stride(0) if m > 1 else n, n, 1)
    Xt = torch.empty((n, m), dtype=torch.float32, device=X.device)
    xtvxy_dense_f32_transpose(m, n, X.data_ptr(), ldx, Xt.data_ptr(), max(m, 1), _stream_handle(stream))
    _keep_for_stream(stream, Xt)
    return Xt


def dense_unfused(X, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, *, Xt=None, workspace=None, stream=None):
    """The comparator: rocBLAS sgemv, elementwise scale, rocBLAS sgemv; with Xt (X^T, n x m, from
    dense_transpose) the last step is a transposed sgemv on it."""
    torch = _torch()
    m, n = X.shape
    ldx = max(X.stride(0) if m > 1 else n, n, 1)
    device = X.device
    _check_vec("y", y, n, device)
    _check_vec("v", v, m, device, required=False)
    _check_vec("z", z, n, device, required=beta != 0)
    made_out = out is None
    if made_out:
        out = torch.empty(n, dtype=torch.float32, device=device)
    made_ws = workspace is None
    if made_ws:
        workspace = _workspace(xtvxy_dense_f32_unfused_reference_workspace_size(m, n), device)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    if Xt is None:
        xtvxy_dense_f32_unfused_reference(m, n, float(alpha), X.data_ptr(), ldx, _ptr(v), y.data_ptr(), float(beta),
                                          _ptr(z), out.data_ptr(), ws_ptr, ws_bytes, _stream_handle(stream))
    else:
        if tuple(Xt.shape) != (n, m) or Xt.dtype != torch.float32 or Xt.device != device:
            raise ValueError("Xt must be an n x m fp32 tensor on %s" % device)
        ldxt = max(Xt.stride(0) if n > 1 else m, m, 1)
        xtvxy_dense_f32_unfused_reference_explicit(m, n, float(alpha), X.data_ptr(), ldx, Xt.data_ptr(), ldxt, _ptr(v),
                                                   y.data_ptr(), float(beta), _ptr(z), out.data_ptr(), ws_ptr,
                                                   ws_bytes, _stream_handle(stream))
    _keep_for_stream(stream, out if made_out else None, workspace if made_ws else None)
    return out


class CsrAnalysis:
    """A structure analysis of one CSR matrix (xtvxy_csr_f32_analyse) and calls that use it: the
    columns relabelled by frequency, the rows grouped by length class and the model's plan. It keeps
    references to row_ptr (read by every call) and col_idx; values change per call."""

    def __init__(self, row_ptr, col_idx, n, stream=None):
        torch = _torch()
        device = row_ptr.device
        for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
            if t.dtype != torch.int32 or t.device != device or not t.is_contiguous():
                raise ValueError("%s must be a contiguous int32 tensor on %s" % (name, device))
        m, nnz = row_ptr.numel() - 1, col_idx.numel()
        self.m, self.n, self.nnz, self.device = m, int(n), nnz, device
        self._keep = (row_ptr, col_idx)
        self.handle = xtvxy_csr_f32_analyse(m, int(n), nnz, row_ptr.data_ptr(),
                                            col_idx.data_ptr() if nnz else None, _stream_handle(stream))

    def plan(self) -> xtvxy_launch_params:
        return xtvxy_csr_f32_analysed_plan(self.handle)

    def complete(self, plan: xtvxy_launch_params) -> xtvxy_launch_params:
        return xtvxy_csr_f32_analysed_plan_complete(self.handle, plan)

    def __call__(self, values, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, *, plan=None, workspace=None,
                 stream=None):
        torch = _torch()
        bf16 = values.dtype in (torch.bfloat16, torch.uint16)
        if (values.dtype != torch.float32 and not bf16) or values.numel() != self.nnz or not values.is_contiguous():
            raise ValueError("values must be a contiguous float32 (or bf16) tensor of nnz elements")
        _check_vec("y", y, self.n, self.device)
        _check_vec("v", v, self.m, self.device, required=False)
        _check_vec("z", z, self.n, self.device, required=beta != 0)
        made_out = out is None
        if made_out:
            out = torch.empty(self.n, dtype=torch.float32, device=self.device)
        _check_vec("out", out, self.n, self.device)
        need = xtvxy_csr_f32_analysed_workspace_size(self.handle) if plan is None else int(plan.workspace_bytes)
        made_ws = workspace is None
        if made_ws:
            workspace = _workspace(need, self.device)
        ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
        args = (self.handle, float(alpha), _ptr(values) if self.nnz else None, _ptr(v), y.data_ptr(), float(beta),
                _ptr(z), out.data_ptr(), ws_ptr, ws_bytes, _stream_handle(stream))
        if plan is None:
            (xtvxy_csr_bf16_analysed if bf16 else xtvxy_csr_f32_analysed)(*args)
        else:
            (xtvxy_csr_bf16_analysed_ex if bf16 else xtvxy_csr_f32_analysed_ex)(*args, plan)
        _keep_for_stream(stream, out if made_out else None, workspace if made_ws else None)
        return out

    def close(self):
        if getattr(self, "handle", 0):
            xtvxy_csr_f32_analysis_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CsrUnfusedPlan:
    """rocSPARSE descriptors and analysis for one CSR matrix (the comparator's setup). With
    ``explicit_transpose`` the plan also keeps a CSR copy of X^T, so that X^T t is a forward SpMV."""

    def __init__(self, row_ptr, col_idx, values, n, stream=None, explicit_transpose=False):
        self.m = row_ptr.numel() - 1
        self.n = n
        self.nnz = col_idx.numel()
        self._keep = (row_ptr, col_idx, values)
        self.handle = xtvxy_csr_f32_unfused_plan_create_ex(
            self.m, n, self.nnz, row_ptr.data_ptr(), col_idx.data_ptr() if self.nnz else None,
            values.data_ptr() if self.nnz else None,
            XTVXY_UNFUSED_EXPLICIT_TRANSPOSE if explicit_transpose else XTVXY_UNFUSED_TRANSPOSE_OP,
            _stream_handle(stream))

    def __call__(self, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, stream=None):
        torch = _torch()
        made_out = out is None
        if made_out:
            out = torch.empty(self.n, dtype=torch.float32, device=y.device)
        xtvxy_csr_f32_unfused_reference(self.handle, float(alpha), _ptr(v), y.data_ptr(), float(beta), _ptr(z),
                                        out.data_ptr(), _stream_handle(stream))
        _keep_for_stream(stream, out if made_out else None)
        return out

    def close(self):
        if self.handle:
            xtvxy_csr_f32_unfused_plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_HISTORY_KEYS = ("loss", "grad_norm", "cg", "gs", "step", "trials")


def logreg_newton_cg(row_ptr, col_idx, values, n, labels, lam, w=None, *, max_newton=20, max_cg=50,
                     max_backtracks=30, grad_tol=1e-6, cg_forcing=0.5, fixed_cg=False, engine="fused",
                     unfused_plan=None, workspace=None, stream=None):
    """Newton-CG for L2-regularised logistic regression on CSR X (xtvxy_logreg_newton_cg_f32).

    ``w`` (float32 CUDA tensor of n elements) is the start point and is overwritten with the
    result; None starts from zeros. ``engine`` is "fused" (this library's products) or "unfused"
    (rocSPARSE through ``unfused_plan``, a CsrUnfusedPlan of the same tensors; made here when
    None). bf16 values (torch.bfloat16, or uint16 bit patterns) take xtvxy_logreg_newton_cg_bf16,
    which runs the fused engine only. Returns (w, report dict, history list of per-iterate dicts)."""
    torch = _torch()
    m, nnz, device = _check_csr_arrays(row_ptr, col_idx, values, bf16_ok=True)
    bf16 = _is_bf16(values)
    _check_vec("labels", labels, m, device)
    if w is None:
        w = torch.zeros(n, dtype=torch.float32, device=device)
    _check_vec("w", w, n, device)
    if engine not in ("fused", "unfused"):
        raise ValueError("engine must be 'fused' or 'unfused'")
    if bf16 and engine != "fused":
        raise ValueError("bf16 values run the fused engine only")
    plan_handle = None
    if engine == "unfused":
        if unfused_plan is None:
            unfused_plan = CsrUnfusedPlan(row_ptr, col_idx, values, n, stream)
        plan_handle = unfused_plan.handle
    opt = xtvxy_logreg_options(float(lam), int(max_newton), int(max_cg), int(max_backtracks), float(grad_tol),
                               float(cg_forcing), 1 if fixed_cg else 0,
                               XTVXY_LOGREG_FUSED if engine == "fused" else XTVXY_LOGREG_UNFUSED)
    need = xtvxy_logreg_newton_cg_f32_workspace_size(m, n, nnz)
    if workspace is None:
        workspace = _workspace(need, device)
    rows = int(max_newton) + 1
    hist = (ctypes.c_double * (rows * len(_HISTORY_KEYS)))()
    rep = xtvxy_logreg_report()
    mats = (m, n, nnz, row_ptr.data_ptr(), _ptr(col_idx) if nnz else None, _ptr(values) if nnz else None,
            _ptr(labels) if m else None, _ptr(w) if n else None, opt)
    tail = (workspace.data_ptr(), workspace.numel(), _stream_handle(stream), rep, hist, rows)
    if bf16:
        xtvxy_logreg_newton_cg_bf16(*mats, *tail)
    else:
        xtvxy_logreg_newton_cg_f32(*mats, plan_handle, *tail)
    history = []
    for k in range(min(rows, rep.newton_iterations + 1)):
        row = {key: hist[k * len(_HISTORY_KEYS) + i] for i, key in enumerate(_HISTORY_KEYS)}
        history.append(row)
    return w, rep.as_dict(), history


def dense_tune(X, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, *, repeats=10, stream=None) -> dict:
    """Tune the dense fused call on these tensors (2-D X with unit column stride); returns the report."""
    torch = _torch()
    m, n = X.shape
    ldx = max(X.stride(0) if m > 1 else n, n, 1)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=X.device)
    fn = (xtvxy_dense_f16_tune if X.dtype == torch.float16 else
          xtvxy_dense_bf16_tune if X.dtype in (torch.bfloat16, torch.uint16) else xtvxy_dense_f32_tune)
    return fn(m, n, float(alpha), X.data_ptr(), ldx, _ptr(v), y.data_ptr(), float(beta), _ptr(z),
                                out.data_ptr(), repeats, _stream_handle(stream)).as_dict()


def csr_tune(row_ptr, col_idx, values, n, y, v=None, z=None, alpha=1.0, beta=0.0, out=None, *, repeats=10,
             stream=None) -> dict:
    """Tune the CSR fused call on these tensors (bf16 values take xtvxy_csr_bf16_tune); returns the
    report."""
    torch = _torch()
    m, nnz, device = _check_csr_arrays(row_ptr, col_idx, values, bf16_ok=True)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    return (xtvxy_csr_bf16_tune if _is_bf16(values) else xtvxy_csr_f32_tune)(m, n, nnz, float(alpha), row_ptr.data_ptr(), _ptr(col_idx), _ptr(values), _ptr(v),
                              y.data_ptr(), float(beta), _ptr(z), out.data_ptr(), repeats,
                              _stream_handle(stream)).as_dict()
