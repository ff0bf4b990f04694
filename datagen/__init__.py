"""Seeded synthetic inputs for out = alpha * X^T (v .* (X y)) + beta * z.

Input generation only: nothing here evaluates the pattern. The tests, the
smoke check and the benchmark draw their inputs from this module and hand the
same fp32/int32 arrays to both the CPU oracle and the GPU library.

The random streams come from ``gen.c`` (counter-based SplitMix64, OpenMP),
so every array is a pure function of (seed, array name) and does not depend on
the thread count. Distribution recipes (the pages give the pattern but no
workload; the shapes below are the measured configurations):

``dense_problem``  X, y, v, z each U(-1, 1), N(0, 1), U(0, 1) or absent.
``csr_bernoulli``  every entry of an m x n grid independently nonzero with
                   probability p (sorted, distinct columns; empty rows occur).
``csr_zipf``       row lengths ~ Zipf(s_row) truncated to 1..K; the columns of
                   a row are the first L distinct values of an i.i.d. stream of
                   ranks ~ Zipf(s_col) truncated to 1..n (column = rank - 1, or
                   a seeded permutation of it), sorted ascending.
``csr_random``     small irregular matrices for edge cases: chosen empty rows,
                   unsorted columns and repeated (duplicate) columns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import zlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libdatagen.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gen.c into libdatagen.so with gcc (OpenMP)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, u64, f32, f64, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
    lib.dg_substream.argtypes = [u64, u64]
    lib.dg_substream.restype = u64
    lib.dg_uniform.argtypes = [vp, i64, u64, f32, f32]
    lib.dg_uniform.restype = None
    lib.dg_normal.argtypes = [vp, i64, u64, f64, f64]
    lib.dg_normal.restype = None
    lib.dg_bernoulli_count.argtypes = [i64, i64, f64, u64, vp]
    lib.dg_bernoulli_fill.argtypes = [i64, i64, f64, u64, vp, vp]
    lib.dg_zipf_lengths.argtypes = [i64, f64, i64, u64, vp]
    lib.dg_zipf_columns.argtypes = [i64, i64, f64, u64, vp, vp, vp]
    lib.dg_logistic_weights.argtypes = [i64, vp, vp, vp, vp, vp]
    lib.dg_logistic_labels.argtypes = [i64, vp, vp, vp, vp, u64, vp]
    for name in ("dg_bernoulli_count", "dg_bernoulli_fill", "dg_zipf_lengths", "dg_zipf_columns",
                 "dg_logistic_weights", "dg_logistic_labels"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def stream_key(seed: int, name: str) -> int:
    """Key of the random stream that fills array ``name`` for a given seed."""
    lib = _load()
    return int(lib.dg_substream(lib.dg_substream(0x5EED, seed & 0xFFFFFFFFFFFFFFFF), zlib.crc32(name.encode())))


def uniform(count: int, seed: int, name: str, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    out = np.empty(int(count), dtype=np.float32)
    _load().dg_uniform(_p(out), int(count), stream_key(seed, name), lo, hi)
    return out


def normal(count: int, seed: int, name: str, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(int(count), dtype=np.float32)
    _load().dg_normal(_p(out), int(count), stream_key(seed, name), mean, std)
    return out


def to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), rounding to nearest with ties to even; NaN stays a
    quiet NaN of the same sign. Storage rounding of an input, done once here."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        rounded[nan] = ((bits[nan] >> 16).astype(np.uint16) & 0x8000) | 0x7FC0
    return rounded


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they denote (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _vector(kind: Optional[str], count: int, seed: int, name: str) -> Optional[np.ndarray]:
    if kind is None:
        return None
    if kind == "uniform":        # U(-1, 1)
        return uniform(count, seed, name)
    if kind == "uniform01":      # U(0, 1)
        return uniform(count, seed, name, 0.0, 1.0)
    if kind == "normal":         # N(0, 1)
        return normal(count, seed, name)
    if kind == "ones":
        return np.ones(int(count), dtype=np.float32)
    raise ValueError("unknown distribution %r" % kind)


@dataclass
class DenseProblem:
    """Dense row-major X (row i starts at X[i*ldx]) and the pattern's vectors and scalars."""
    m: int
    n: int
    ldx: int
    X: np.ndarray                 # flat, length m*ldx (padding columns hold NaN): fp32, uint16 bf16 bits or fp16
    y: np.ndarray
    v: Optional[np.ndarray]
    z: Optional[np.ndarray]
    alpha: float
    beta: float
    name: str = ""
    x_dtype: str = "f32"          # "f32", "bf16" or "f16"

    def X2d(self) -> np.ndarray:
        return self.X.reshape(self.m, self.ldx)[:, : self.n]

    def X_f32(self) -> np.ndarray:
        """X as the fp32 numbers it denotes: bf16 and fp16 widened exactly (fp16 by numpy)."""
        if self.x_dtype == "bf16":
            return bf16_to_f32(self.X)
        if self.x_dtype == "f16":
            return self.X.astype(np.float32)
        return self.X


@dataclass
class CsrProblem:
    """CSR X (zero-based int32 row_ptr[m+1], col_idx[nnz], values[nnz]) and vectors. values are
    fp32, or with values_dtype "bf16" uint16 bf16 bit patterns."""
    m: int
    n: int
    row_ptr: np.ndarray
    col_idx: np.ndarray
    values: np.ndarray
    y: np.ndarray
    v: Optional[np.ndarray]
    z: Optional[np.ndarray]
    alpha: float
    beta: float
    name: str = ""
    info: dict = field(default_factory=dict)
    values_dtype: str = "f32"     # "f32" or "bf16"

    @property
    def nnz(self) -> int:
        return int(self.col_idx.shape[0])

    def values_f32(self) -> np.ndarray:
        """The values as the fp32 numbers they denote (bf16 widened exactly)."""
        return bf16_to_f32(self.values) if self.values_dtype == "bf16" else self.values


def csr_values_bf16(p: CsrProblem, name: str = "") -> CsrProblem:
    """The same problem with its values rounded to bf16 (to_bf16) and stored as uint16 bit patterns."""
    return CsrProblem(p.m, p.n, p.row_ptr, p.col_idx, to_bf16(p.values), p.y, p.v, p.z, p.alpha, p.beta,
                      name or p.name + "_bf16", dict(p.info), "bf16")


def dense_problem(m, n, seed=0, *, x="uniform", y="uniform", v="uniform", z="uniform", alpha=1.5,
                  beta=0.5, ldx=None, name="", x_dtype="f32") -> DenseProblem:
    """Dense problem whose entries follow the named distributions (None = argument absent). With
    x_dtype "bf16" the same X is rounded to bf16 (to_bf16) and stored as uint16 bit patterns; with
    "f16" it is rounded to IEEE fp16 (to nearest, ties to even; numpy) and stored as float16."""
    ldx = n if ldx is None else int(ldx)
    if ldx < n:
        raise ValueError("ldx < n")
    if x_dtype not in ("f32", "bf16", "f16"):
        raise ValueError("x_dtype must be f32, bf16 or f16")
    body = _vector(x, m * n, seed, "X")
    if ldx == n:
        X = body if body is not None else np.zeros(m * n, np.float32)
    else:
        X = np.full(m * ldx, np.nan, dtype=np.float32)
        X.reshape(m, ldx)[:, :n] = body.reshape(m, n)
    if x_dtype == "bf16":
        X = to_bf16(X)
    elif x_dtype == "f16":
        X = X.astype(np.float16)
    return DenseProblem(m, n, ldx, X, _vector(y, n, seed, "y"), _vector(v, m, seed, "v"),
                        _vector(z, n, seed, "z"), float(alpha), float(beta), name, x_dtype)


def _row_ptr(row_len: np.ndarray) -> np.ndarray:
    rp = np.zeros(row_len.shape[0] + 1, dtype=np.int64)
    np.cumsum(row_len, out=rp[1:])
    if rp[-1] > np.iinfo(np.int32).max:
        raise ValueError("nnz exceeds int32 indexing")
    return rp


def csr_bernoulli(m, n, p, seed=0, *, values="normal", y="normal", v="logistic", z=None, alpha=1.0,
                  beta=0.0, w_std=0.1, name="") -> CsrProblem:
    """Bernoulli(p) sparsity; v = "logistic" gives v_i = p_i(1 - p_i), p = sigmoid(X w),
    w ~ N(0, w_std^2), the curvature weights of a logistic-regression Hessian."""
    lib = _load()
    rl = np.empty(m, dtype=np.int32)
    if lib.dg_bernoulli_count(m, n, p, stream_key(seed, "structure"), _p(rl)) != 0:
        raise ValueError("bad Bernoulli parameters")
    rp64 = _row_ptr(rl)
    cols = np.empty(int(rp64[-1]), dtype=np.int32)
    lib.dg_bernoulli_fill(m, n, p, stream_key(seed, "structure"), _p(rp64), _p(cols))
    vals = _vector(values, cols.shape[0], seed, "values")
    if v == "logistic":
        w = normal(n, seed, "w", 0.0, w_std)
        vv = np.empty(m, dtype=np.float32)
        lib.dg_logistic_weights(m, _p(rp64), _p(cols), _p(vals), _p(w), _p(vv))
    else:
        vv = _vector(v, m, seed, "v")
    return CsrProblem(m, n, rp64.astype(np.int32), cols, vals, _vector(y, n, seed, "y"), vv,
                      _vector(z, n, seed, "z"), float(alpha), float(beta), name,
                      {"density": p})


@dataclass
class LogisticProblem:
    """L2-regularised logistic regression data: CSR X (in ``X``, whose y, v, z are unused),
    labels c_i in {0, 1} and the regularisation weight lambda."""
    X: CsrProblem
    labels: np.ndarray
    lam: float
    name: str = ""


def logistic_labels(X: CsrProblem, seed=0, w_std=0.1) -> np.ndarray:
    """Labels c_i ~ Bernoulli(sigmoid(x_i . w)) of the planted model w ~ N(0, w_std^2) that
    ``csr_bernoulli(..., v="logistic")`` draws for the same seed."""
    lib = _load()
    w = normal(X.n, seed, "w", 0.0, w_std)
    out = np.empty(X.m, dtype=np.float32)
    lib.dg_logistic_labels(X.m, _p(np.ascontiguousarray(X.row_ptr, np.int64)), _p(X.col_idx), _p(X.values),
                           _p(w), stream_key(seed, "labels"), _p(out))
    return out


def logistic_problem(m, n, density, seed=0, *, lam=1.0, w_std=0.1, name="") -> LogisticProblem:
    """Bernoulli(density) CSR X with N(0, 1) values and labels of a planted model."""
    X = csr_bernoulli(m, n, density, seed, values="normal", y="normal", v="logistic", z=None, alpha=1.0,
                      beta=0.0, w_std=w_std, name=name)
    return LogisticProblem(X, logistic_labels(X, seed, w_std), float(lam), name)


def csr_zipf(m, n, seed=0, *, s_row=1.5, max_row=2726, s_col=1.2, permute_columns=False,
             values="uniform", y="uniform", v="uniform", z="uniform", alpha=0.7, beta=0.3,
             name="") -> CsrProblem:
    """Zipf row lengths and Zipf-skewed, per-row-distinct column indices."""
    lib = _load()
    rl = np.empty(m, dtype=np.int32)
    if lib.dg_zipf_lengths(m, s_row, max_row, stream_key(seed, "row_lengths"), _p(rl)) != 0:
        raise ValueError("bad Zipf row parameters")
    if rl.max(initial=0) > n:
        raise ValueError("row longer than n")
    rp64 = _row_ptr(rl)
    cols = np.empty(int(rp64[-1]), dtype=np.int32)
    perm = None
    if permute_columns:
        perm = np.random.Generator(np.random.PCG64(stream_key(seed, "permutation"))).permutation(n).astype(np.int32)
    rc = lib.dg_zipf_columns(m, n, s_col, stream_key(seed, "columns"), _p(rp64),
                             _p(perm) if perm is not None else None, _p(cols))
    if rc != 0:
        raise ValueError("Zipf column sampling failed (code %d)" % rc)
    return CsrProblem(m, n, rp64.astype(np.int32), cols, _vector(values, cols.shape[0], seed, "values"),
                      _vector(y, n, seed, "y"), _vector(v, m, seed, "v"), _vector(z, n, seed, "z"),
                      float(alpha), float(beta), name,
                      {"s_row": s_row, "max_row": max_row, "s_col": s_col, "permuted": permute_columns})


def csr_random(m, n, seed=0, *, mean_len=4.0, empty_frac=0.2, dup_frac=0.1, shuffle=True,
               values="uniform", y="uniform", v="uniform", z="uniform", alpha=1.5, beta=0.5,
               name="") -> CsrProblem:
    """Small irregular CSR: a fraction of rows empty, columns unsorted and some repeated."""
    g = np.random.Generator(np.random.PCG64(stream_key(seed, "csr_random")))
    lens = g.poisson(mean_len, size=m).astype(np.int64)
    lens[g.random(m) < empty_frac] = 0
    rp = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(lens, out=rp[1:])
    nnz = int(rp[-1])
    cols = g.integers(0, max(n, 1), size=nnz).astype(np.int32) if n > 0 else np.zeros(0, np.int32)
    if nnz and dup_frac > 0:
        # repeat the previous column of the same row for a fraction of entries
        rows = np.repeat(np.arange(m), lens)
        pick = np.nonzero((g.random(nnz) < dup_frac) & (np.arange(nnz) > rp[rows]))[0]
        cols[pick] = cols[pick - 1]
    if not shuffle:
        for i in range(m):
            cols[rp[i]:rp[i + 1]].sort()
    return CsrProblem(m, n, rp.astype(np.int32), cols, _vector(values, nnz, seed, "values"),
                      _vector(y, n, seed, "y"), _vector(v, m, seed, "v"), _vector(z, n, seed, "z"),
                      float(alpha), float(beta), name)


def csr_from_dense(X2d: np.ndarray):
    """CSR arrays (row_ptr, col_idx, values) holding the nonzeros of a dense matrix."""
    rows, cols = np.nonzero(X2d)
    rp = np.zeros(X2d.shape[0] + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=X2d.shape[0]), out=rp[1:])
    return rp.astype(np.int32), cols.astype(np.int32), X2d[rows, cols].astype(np.float32)


# Newton-CG for L2-regularised logistic regression on the 10,000,000 x 1000 Hessian-vector workload's
# generator: 1% Bernoulli sparsity, N(0, 1) values, labels of the planted w ~ N(0, 0.1^2), lambda 1.
def logistic_values_bf16(P: LogisticProblem, name: str = "") -> LogisticProblem:
    """The same problem (same labels) with X's values rounded to bf16 (csr_values_bf16)."""
    name = name or P.name + "_bf16"
    return LogisticProblem(csr_values_bf16(P.X, name), P.labels, P.lam, name)


LOGISTIC_WORKLOADS = {
    "logreg_csr_10000000x1000": lambda seed=0, m=10_000_000, n=1000, lam=1.0: logistic_problem(
        m, n, 0.01, seed, lam=lam, w_std=0.1, name="logreg_csr_10000000x1000"),
    # the same problem, its values stored as bf16 (the labels are those of the fp32 values)
    "logreg_csr_10000000x1000_bf16": lambda seed=0, m=10_000_000, n=1000, lam=1.0: logistic_values_bf16(
        logistic_problem(m, n, 0.01, seed, lam=lam, w_std=0.1, name="logreg_csr_10000000x1000"),
        "logreg_csr_10000000x1000_bf16"),
}

# The measured workloads, named by what they are. Each entry builds the full-size
# problem; ``scaled`` variants with the same recipe and smaller sizes serve parity tests.
WORKLOADS = {
    # dense 2048 x 128, X, y, v, z ~ U(-1, 1), alpha 1.5, beta 0.5
    "dense_2048x128": lambda seed=0, m=2048, n=128: dense_problem(
        m, n, seed, x="uniform", y="uniform", v="uniform", z="uniform", alpha=1.5, beta=0.5,
        name="dense_2048x128"),
    # normal equations X^T X y: X, y ~ N(0, 1), v absent (= 1), beta 0
    "dense_1000000x256_normal_equations": lambda seed=0, m=1_000_000, n=256: dense_problem(
        m, n, seed, x="normal", y="normal", v=None, z=None, alpha=1.0, beta=0.0,
        name="dense_1000000x256_normal_equations"),
    # X, y, z ~ U(-1, 1), v ~ U(0, 1), alpha = beta = 1
    "dense_65536x8192": lambda seed=0, m=65536, n=8192: dense_problem(
        m, n, seed, x="uniform", y="uniform", v="uniform01", z="uniform", alpha=1.0, beta=1.0,
        name="dense_65536x8192"),
    # the same recipe with the shape transposed: the output (256 KiB) exceeds the LDS
    "dense_8192x65536": lambda seed=0, m=8192, n=65536: dense_problem(
        m, n, seed, x="uniform", y="uniform", v="uniform01", z="uniform", alpha=1.0, beta=1.0,
        name="dense_8192x65536"),
    # the same three dense workloads with X stored as bf16 (rounded to nearest even from the fp32 draw)
    "dense_1000000x256_normal_equations_bf16": lambda seed=0, m=1_000_000, n=256: dense_problem(
        m, n, seed, x="normal", y="normal", v=None, z=None, alpha=1.0, beta=0.0,
        name="dense_1000000x256_normal_equations_bf16", x_dtype="bf16"),
    "dense_65536x8192_bf16": lambda seed=0, m=65536, n=8192: dense_problem(
        m, n, seed, x="uniform", y="uniform", v="uniform01", z="uniform", alpha=1.0, beta=1.0,
        name="dense_65536x8192_bf16", x_dtype="bf16"),
    "dense_8192x65536_bf16": lambda seed=0, m=8192, n=65536: dense_problem(
        m, n, seed, x="uniform", y="uniform", v="uniform01", z="uniform", alpha=1.0, beta=1.0,
        name="dense_8192x65536_bf16", x_dtype="bf16"),
    # and with X stored as IEEE fp16 (rounded to nearest even from the fp32 draw)
    "dense_1000000x256_normal_equations_f16": lambda seed=0, m=1_000_000, n=256: dense_problem(
        m, n, seed, x="normal", y="normal", v=None, z=None, alpha=1.0, beta=0.0,
        name="dense_1000000x256_normal_equations_f16", x_dtype="f16"),
    "dense_65536x8192_f16": lambda seed=0, m=65536, n=8192: dense_problem(
        m, n, seed, x="uniform", y="uniform", v="uniform01", z="uniform", alpha=1.0, beta=1.0,
        name="dense_65536x8192_f16", x_dtype="f16"),
    "dense_8192x65536_f16": lambda seed=0, m=8192, n=65536: dense_problem(
        m, n, seed, x="uniform", y="uniform", v="uniform01", z="uniform", alpha=1.0, beta=1.0,
        name="dense_8192x65536_f16", x_dtype="f16"),
    # logistic-regression Hessian-vector product: 1% Bernoulli sparsity, values and y ~ N(0, 1),
    # v = p(1 - p) with p = sigmoid(X w), w ~ N(0, 0.1^2), beta 0
    "csr_10000000x1000_logistic_hvp": lambda seed=0, m=10_000_000, n=1000: csr_bernoulli(
        m, n, 0.01, seed, values="normal", y="normal", v="logistic", z=None, alpha=1.0, beta=0.0,
        name="csr_10000000x1000_logistic_hvp"),
    # Zipf(1.5) row lengths (truncated at 2726: mean 40), Zipf(1.2) columns, U(-1, 1) values
    # and vectors, alpha 0.7, beta 0.3
    "csr_5000000x1000000_zipf": lambda seed=0, m=5_000_000, n=1_000_000, permute_columns=False: csr_zipf(
        m, n, seed, s_row=1.5, max_row=2726, s_col=1.2, permute_columns=permute_columns,
        values="uniform", y="uniform", v="uniform", z="uniform", alpha=0.7, beta=0.3,
        name="csr_5000000x1000000_zipf"),
    # the same matrix with a seeded random permutation of the columns: the hot columns are spread
    # over the whole index range instead of sitting at the lowest indices
    "csr_5000000x1000000_zipf_permuted": lambda seed=0, m=5_000_000, n=1_000_000: csr_zipf(
        m, n, seed, s_row=1.5, max_row=2726, s_col=1.2, permute_columns=True,
        values="uniform", y="uniform", v="uniform", z="uniform", alpha=0.7, beta=0.3,
        name="csr_5000000x1000000_zipf_permuted"),
    # the two CSR workloads with their values stored as bf16 (rounded to nearest even from the fp32
    # draw); the structure stays int32
    "csr_10000000x1000_logistic_hvp_bf16": lambda seed=0, m=10_000_000, n=1000: csr_values_bf16(csr_bernoulli(
        m, n, 0.01, seed, values="normal", y="normal", v="logistic", z=None, alpha=1.0, beta=0.0,
        name="csr_10000000x1000_logistic_hvp"), "csr_10000000x1000_logistic_hvp_bf16"),
    "csr_5000000x1000000_zipf_bf16": lambda seed=0, m=5_000_000, n=1_000_000: csr_values_bf16(csr_zipf(
        m, n, seed, s_row=1.5, max_row=2726, s_col=1.2, permute_columns=False,
        values="uniform", y="uniform", v="uniform", z="uniform", alpha=0.7, beta=0.3,
        name="csr_5000000x1000000_zipf"), "csr_5000000x1000000_zipf_bf16"),
}
