"""CPU oracle for out = alpha * X^T (v .* (X y)) + beta * z (fp64 accumulation).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline may import this package; the GPU library never does, and this package
imports nothing from the library. The arithmetic lives in ``oracle.cpp``
(plain two-pass evaluation of the generic pattern from "On optimizing machine
learning workloads via kernel fusion", abstract); this module only builds it
with g++ and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def compile_source(src: str, out_path: str) -> str:
    """Compile an oracle source file into a shared library with g++ (OpenMP, no fast-math)."""
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so next to it."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


def _bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64, f32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = ctypes.c_int
    dense_args = [i64, i64, f32, vp, i64, vp, vp, f32, vp, vp]
    csr_args = [i64, i64, i64, f32, vp, vp, vp, vp, vp, f32, vp, vp]
    for name, args in (("oracle_dense", dense_args), ("oracle_dense_bound", dense_args),
                       ("oracle_dense_bf16", dense_args), ("oracle_dense_bf16_bound", dense_args),
                       ("oracle_csr", csr_args), ("oracle_csr_bound", csr_args),
                       ("oracle_csr_rowdot", csr_args), ("oracle_csr_rowdot_bound", csr_args),
                       ("oracle_csr_tmv", csr_args[:8] + [f32, vp, vp]),
                       ("oracle_csr_tmv_bound", csr_args[:8] + [f32, vp, vp])):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(_LIB_PATH)
    return _lib


class OracleError(RuntimeError):
    pass


def set_threads(nthreads: int = 0) -> int:
    """Set the OpenMP thread count (<= 0 keeps it); return the count in use."""
    return int(_load().oracle_set_threads(int(nthreads)))


def _ptr(a, dtype):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a)
    if arr.dtype != dtype:
        raise TypeError("expected %s array, got %s" % (np.dtype(dtype), arr.dtype))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, name: str):
    if rc != 0:
        raise OracleError("%s failed with code %d" % (name, rc))


def dense(X, y, v=None, z=None, alpha=1.0, beta=0.0, *, ldx=None, m=None, n=None, bound=False,
          lib=None):
    """Oracle value (or the error normaliser when ``bound``) for dense row-major X, fp32 or
    bf16 (a uint16 array of bf16 bit patterns).

    ``X`` is a 2-D array (m x n) or, with ``ldx``/``m``/``n`` given, a flat
    buffer whose row i starts at element i*ldx.
    """
    X = np.asarray(X)
    if X.ndim == 2 and ldx is None:
        m, n = X.shape
        ldx = n
    if m is None or n is None or ldx is None:
        raise ValueError("flat X needs m, n and ldx")
    bf16 = np.asarray(X).dtype == np.uint16
    Xa, Xp = _ptr(X, np.uint16 if bf16 else np.float32)
    ya, yp = _ptr(y, np.float32)
    va, vp_ = _ptr(v, np.float32)
    za, zp = _ptr(z, np.float32)
    out = np.empty(int(n), dtype=np.float64)
    lib = lib or _load()
    if bf16:
        fn = lib.oracle_dense_bf16_bound if bound else lib.oracle_dense_bf16
    else:
        fn = lib.oracle_dense_bound if bound else lib.oracle_dense
    rc = fn(int(m), int(n), float(alpha), Xp, int(ldx), vp_, yp, float(beta), zp,
            out.ctypes.data_as(ctypes.c_void_p))
    _check(rc, fn.__name__)
    return out


def csr(row_ptr, col_idx, values, n, y, v=None, z=None, alpha=1.0, beta=0.0, *, bound=False,
        lib=None):
    """Oracle value (or normaliser) for CSR X with int32 indices and fp32 values."""
    rpa, rpp = _ptr(row_ptr, np.int32)
    cia, cip = _ptr(col_idx, np.int32)
    vaa, vap = _ptr(values, np.float32)
    ya, yp = _ptr(y, np.float32)
    va, vp_ = _ptr(v, np.float32)
    za, zp = _ptr(z, np.float32)
    m = rpa.shape[0] - 1
    nnz = cia.shape[0]
    out = np.empty(int(n), dtype=np.float64)
    lib = lib or _load()
    fn = lib.oracle_csr_bound if bound else lib.oracle_csr
    rc = fn(int(m), int(n), int(nnz), float(alpha), rpp, cip, vap, vp_, yp, float(beta), zp,
            out.ctypes.data_as(ctypes.c_void_p))
    _check(rc, fn.__name__)
    return out


def csr_rowdot(row_ptr, col_idx, values, n, y, v=None, t0=None, alpha=1.0, beta=0.0, *, bound=False, lib=None):
    """t_i = alpha v_i (X y)_i + beta t0_i (the first half of the pattern), or its normaliser."""
    rpa, rpp = _ptr(row_ptr, np.int32)
    cia, cip = _ptr(col_idx, np.int32)
    vaa, vap = _ptr(values, np.float32)
    ya, yp = _ptr(y, np.float32)
    va, vp_ = _ptr(v, np.float32)
    ta, tp = _ptr(t0, np.float32)
    m = rpa.shape[0] - 1
    out = np.empty(int(m), dtype=np.float64)
    lib = lib or _load()
    fn = lib.oracle_csr_rowdot_bound if bound else lib.oracle_csr_rowdot
    rc = fn(int(m), int(n), int(cia.shape[0]), float(alpha), rpp, cip, vap, vp_, yp, float(beta), tp,
            out.ctypes.data_as(ctypes.c_void_p))
    _check(rc, fn.__name__)
    return out


def csr_tmv(row_ptr, col_idx, values, n, u, z=None, alpha=1.0, beta=0.0, *, bound=False, lib=None):
    """out_j = alpha (X^T u)_j + beta z_j (the second half of the pattern), or its normaliser."""
    rpa, rpp = _ptr(row_ptr, np.int32)
    cia, cip = _ptr(col_idx, np.int32)
    vaa, vap = _ptr(values, np.float32)
    ua, up = _ptr(u, np.float32)
    za, zp = _ptr(z, np.float32)
    m = rpa.shape[0] - 1
    out = np.empty(int(n), dtype=np.float64)
    lib = lib or _load()
    fn = lib.oracle_csr_tmv_bound if bound else lib.oracle_csr_tmv
    rc = fn(int(m), int(n), int(cia.shape[0]), float(alpha), rpp, cip, vap, up, float(beta), zp,
            out.ctypes.data_as(ctypes.c_void_p))
    _check(rc, fn.__name__)
    return out

