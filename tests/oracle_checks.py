"""Checks that pin the CPU oracle to something other than itself.

Each ``check_*`` takes a loaded oracle library handle and raises AssertionError
on a mismatch. They cover the hand-derived golden fixtures, brute force with
the explicit n x n matrix X^T diag(v) X, exact integer arithmetic, closed forms,
invariants of the pattern, a scipy.sparse cross-check and the oracle's own
conventions (quick returns, NaN propagation, error codes). The same list is run
against deliberately broken copies of the oracle in test_oracle_mutations.py.
"""
from __future__ import annotations

import numpy as np
import scipy.sparse as sp

import datagen
import oracle
from parity import golden_names, read_golden


def _dense(lib, X, y, v=None, z=None, alpha=1.0, beta=0.0, bound=False, **kw):
    return oracle.dense(X, y, v, z, alpha, beta, bound=bound, lib=lib, **kw)


def _csr(lib, rp, ci, vals, n, y, v=None, z=None, alpha=1.0, beta=0.0, bound=False):
    return oracle.csr(rp, ci, vals, n, y, v, z, alpha, beta, bound=bound, lib=lib)


def _brute(X, y, v, z, alpha, beta):
    """alpha * (X^T diag(v) X) y + beta * z with the n x n matrix formed explicitly (fp64)."""
    X64 = np.asarray(X, np.float64)
    vv = np.ones(X64.shape[0]) if v is None else np.asarray(v, np.float64)
    M = X64.T @ np.diag(vv) @ X64
    out = float(alpha) * (M @ np.asarray(y, np.float64))
    if beta != 0:
        out = out + float(beta) * np.asarray(z, np.float64)
    return out


def _close(a, b, scale, tol):
    a, b, scale = (np.asarray(t, np.float64) for t in (a, b, scale))
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b) <= tol * np.maximum(scale, 1e-300)
    assert np.all(err), "max abs diff %g" % np.max(np.abs(a - b))


def _dense_to_csr(X2d):
    return datagen.csr_from_dense(X2d)


def _csr_to_dense(rp, ci, vals, m, n):
    X = np.zeros((m, n), np.float64)
    rows = np.repeat(np.arange(m), np.diff(rp))
    np.add.at(X, (rows, ci), vals.astype(np.float64))
    return X


def check_golden(lib):
    for name in golden_names():
        g = read_golden(name)
        if g["kind"] == "dense":
            out = _dense(lib, g["X"], g["y"], g.get("v"), g.get("z"), g["alpha"], g["beta"],
                         m=g["m"], n=g["n"], ldx=g["ldx"])
        else:
            out = _csr(lib, g["row_ptr"], g["col_idx"], g["values"], g["n"], g["y"], g.get("v"),
                       g.get("z"), g["alpha"], g["beta"])
        assert np.array_equal(out, g["expected"]), (name, out, g["expected"])


def check_brute_force_dense(lib):
    for k, (m, n) in enumerate([(1, 1), (2, 3), (3, 2), (7, 5), (13, 64), (64, 64), (64, 7)]):
        for v_kind, z_kind, alpha, beta in (("uniform", "uniform", 1.5, 0.5), (None, None, -0.75, 0.0)):
            p = datagen.dense_problem(m, n, seed=100 + k, v=v_kind, z=z_kind, alpha=alpha, beta=beta)
            out = _dense(lib, p.X2d(), p.y, p.v, p.z, p.alpha, p.beta)
            bnd = _dense(lib, p.X2d(), p.y, p.v, p.z, p.alpha, p.beta, bound=True)
            _close(out, _brute(p.X2d(), p.y, p.v, p.z, p.alpha, p.beta), bnd, 1e-12)
    # padded leading dimension: the padding holds NaN and must not be read
    for k, (m, n, ldx) in enumerate([(5, 3, 4), (31, 17, 24), (8, 64, 129)]):
        p = datagen.dense_problem(m, n, seed=150 + k, ldx=ldx)
        out = _dense(lib, p.X, p.y, p.v, p.z, p.alpha, p.beta, m=m, n=n, ldx=ldx)
        bnd = _dense(lib, p.X, p.y, p.v, p.z, p.alpha, p.beta, m=m, n=n, ldx=ldx, bound=True)
        _close(out, _brute(p.X2d(), p.y, p.v, p.z, p.alpha, p.beta), bnd, 1e-12)


def check_brute_force_csr(lib):
    for k, (m, n) in enumerate([(1, 1), (5, 3), (17, 9), (64, 40), (200, 64)]):
        p = datagen.csr_random(m, n, seed=200 + k, mean_len=3.0, empty_frac=0.25, dup_frac=0.2)
        out = _csr(lib, p.row_ptr, p.col_idx, p.values, n, p.y, p.v, p.z, p.alpha, p.beta)
        bnd = _csr(lib, p.row_ptr, p.col_idx, p.values, n, p.y, p.v, p.z, p.alpha, p.beta, bound=True)
        Xd = _csr_to_dense(p.row_ptr, p.col_idx, p.values, m, n)
        _close(out, _brute(Xd, p.y, p.v, p.z, p.alpha, p.beta), bnd, 1e-12)


def check_exact_integers(lib):
    g = np.random.default_rng(7)
    for (m, n, lim) in ((37, 23, 1), (64, 48, 3), (200, 129, 1)):
        Xi = g.integers(-lim, lim + 1, size=(m, n))
        yi, vi, zi = (g.integers(-lim, lim + 1, size=s) for s in (n, m, n))
        S = Xi.T @ (vi * (Xi @ yi))                       # exact int64
        expected = 1.5 * S.astype(np.float64) + 0.5 * zi  # short dyadics, exact in fp64
        X, y, v, z = (a.astype(np.float32) for a in (Xi, yi, vi, zi))
        out = _dense(lib, X, y, v, z, 1.5, 0.5)
        assert np.array_equal(out, expected)
        rp, ci, vals = _dense_to_csr(X)
        out = _csr(lib, rp, ci, vals, n, y, v, z, 1.5, 0.5)
        assert np.array_equal(out, expected)


def check_closed_forms(lib):
    # X = I: alpha * v .* y + beta * z
    n = 17
    p = datagen.dense_problem(n, n, seed=3)
    eye = np.eye(n, dtype=np.float32)
    out = _dense(lib, eye, p.y, p.v, p.z, 1.25, -0.5)
    exp = 1.25 * (p.v.astype(np.float64) * p.y) - 0.5 * p.z.astype(np.float64)
    _close(out, exp, np.abs(exp) + 1e-30, 1e-15)
    # rank one X = a b^T with power-of-two entries (exact in fp32)
    g = np.random.default_rng(11)
    m, n = 33, 21
    a = (2.0 ** g.integers(-3, 4, size=m) * g.choice([-1, 1], size=m)).astype(np.float32)
    b = (2.0 ** g.integers(-3, 4, size=n) * g.choice([-1, 1], size=n)).astype(np.float32)
    X = np.outer(a, b).astype(np.float32)
    y = datagen.uniform(n, 5, "y")
    v = datagen.uniform(m, 5, "v")
    z = datagen.uniform(n, 5, "z")
    out = _dense(lib, X, y, v, z, 0.75, 2.0)
    exp = 0.75 * float(np.sum(v.astype(np.float64) * a.astype(np.float64) ** 2)) * \
        float(np.dot(b.astype(np.float64), y)) * b.astype(np.float64) + 2.0 * z
    bnd = _dense(lib, X, y, v, z, 0.75, 2.0, bound=True)
    _close(out, exp, bnd, 1e-13)
    # all ones: alpha * m * n + beta * z_j
    m, n = 12, 7
    ones = np.ones((m, n), np.float32)
    z = datagen.uniform(n, 6, "z")
    out = _dense(lib, ones, np.ones(n, np.float32), np.ones(m, np.float32), z, 2.0, 3.0)
    assert np.array_equal(out, 2.0 * m * n + 3.0 * z.astype(np.float64))


def check_special_cases(lib):
    p = datagen.dense_problem(9, 6, seed=4)
    Xnan = p.X2d().copy()
    Xnan[3, 2] = np.nan
    ynan = p.y.copy()
    ynan[1] = np.nan
    # alpha == 0: out = beta z exactly, X, y, v not read
    out = _dense(lib, Xnan, ynan, p.v, p.z, 0.0, 0.5)
    assert np.array_equal(out, 0.5 * p.z.astype(np.float64))
    out = _dense(lib, Xnan, ynan, p.v, p.z, 0.0, 0.0)
    assert np.array_equal(out, np.zeros(6))
    # beta == 0: z not read
    znan = np.full(6, np.nan, np.float32)
    ref = _dense(lib, p.X2d(), p.y, p.v, None, 1.5, 0.0)
    out = _dense(lib, p.X2d(), p.y, p.v, znan, 1.5, 0.0)
    assert np.array_equal(out, ref) and np.all(np.isfinite(out))
    # m == 0: out = beta z
    out = _dense(lib, np.zeros((0, 6), np.float32), p.y, np.zeros(0, np.float32), p.z, 1.0, -2.0)
    assert np.array_equal(out, -2.0 * p.z.astype(np.float64))
    # n == 0: nothing
    assert _dense(lib, np.zeros((4, 0), np.float32), np.zeros(0, np.float32), None, None).shape == (0,)
    # v absent equals v = 1 bitwise
    a = _dense(lib, p.X2d(), p.y, None, p.z, 1.5, 0.5)
    b = _dense(lib, p.X2d(), p.y, np.ones(9, np.float32), p.z, 1.5, 0.5)
    assert np.array_equal(a, b)
    # the CSR entry points follow the same conventions
    rp, ci, vals = _dense_to_csr(p.X2d())
    out = _csr(lib, rp, ci, vals, 6, ynan, p.v, p.z, 0.0, 0.5)
    assert np.array_equal(out, 0.5 * p.z.astype(np.float64))
    out = _csr(lib, rp, ci, vals, 6, p.y, p.v, znan, 1.5, 0.0)
    assert np.array_equal(out, ref)
    empty = _csr(lib, np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32), 6, p.y,
                 np.zeros(0, np.float32), p.z, 1.0, -2.0)
    assert np.array_equal(empty, -2.0 * p.z.astype(np.float64))
    nnz0 = _csr(lib, np.zeros(5, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32), 6, p.y,
                np.ones(4, np.float32), p.z, 1.0, 0.25)
    assert np.array_equal(nnz0, 0.25 * p.z.astype(np.float64))


def check_invariants(lib):
    m, n = 40, 24
    p = datagen.dense_problem(m, n, seed=8, v="uniform01")
    X = p.X2d()
    g = np.random.default_rng(9)
    # integer-valued y so that 2 y1 - 3 y2 is exact in fp32
    y1, y2 = (g.integers(-3, 4, size=n).astype(np.float32) for _ in range(2))
    ycomb = (2 * y1 - 3 * y2).astype(np.float32)
    bnd = _dense(lib, X, np.abs(y1) * 2 + np.abs(y2) * 3, p.v, None, 1.0, 0.0, bound=True)
    # linearity in y (beta = 0)
    lhs = _dense(lib, X, ycomb, p.v)
    rhs = 2 * _dense(lib, X, y1, p.v) - 3 * _dense(lib, X, y2, p.v)
    _close(lhs, rhs, bnd, 1e-12)
    # the z term is additive: f(z) - f(beta = 0) = beta z
    full = _dense(lib, X, y1, p.v, p.z, 1.0, 0.5)
    noz = _dense(lib, X, y1, p.v, None, 1.0, 0.0)
    _close(full - noz, 0.5 * p.z.astype(np.float64), np.abs(noz) + 1.0, 1e-14)
    # symmetry of X^T diag(v) X: w . f(y) == y . f(w)
    a = float(np.dot(y2.astype(np.float64), _dense(lib, X, y1, p.v)))
    b = float(np.dot(y1.astype(np.float64), _dense(lib, X, y2, p.v)))
    assert abs(a - b) <= 1e-12 * (abs(a) + abs(b) + 1.0), (a, b)
    # y . f(y) = sum_i v_i (x_i . y)^2 >= 0 for v >= 0, and equals it
    q = float(np.dot(y1.astype(np.float64), _dense(lib, X, y1, p.v)))
    t = X.astype(np.float64) @ y1.astype(np.float64)
    assert q >= 0 and abs(q - float(np.sum(p.v * t * t))) <= 1e-12 * abs(q)
    # row permutation (rows of X with v) leaves the result unchanged
    perm = np.random.default_rng(1).permutation(m)
    base = _dense(lib, X, y1, p.v, p.z, 1.5, 0.5)
    bbase = _dense(lib, X, y1, p.v, p.z, 1.5, 0.5, bound=True)
    _close(_dense(lib, X[perm], y1, p.v[perm], p.z, 1.5, 0.5), base, bbase, 1e-13)
    # column permutation: f(X P, P^T y, P^T z) = P^T f(X, y, z)
    cp = np.random.default_rng(2).permutation(n)
    permuted = _dense(lib, np.ascontiguousarray(X[:, cp]), y1[cp], p.v, p.z[cp], 1.5, 0.5)
    _close(permuted, base[cp], bbase[cp], 1e-13)


def check_csr_dense_agree(lib):
    m, n = 120, 50
    p = datagen.dense_problem(m, n, seed=12)
    X = p.X2d().copy()
    X[np.random.default_rng(3).random((m, n)) < 0.7] = 0.0
    X[5] = 0.0                                  # an empty row
    rp, ci, vals = _dense_to_csr(X)
    a = _dense(lib, X, p.y, p.v, p.z, p.alpha, p.beta)
    b = _csr(lib, rp, ci, vals, n, p.y, p.v, p.z, p.alpha, p.beta)
    assert np.array_equal(a, b)                 # same sums in the same order, zeros added exactly
    # splitting an entry into two stored halves (exact in fp32) changes nothing
    k = int(rp[7])
    ci2 = np.insert(ci, k, ci[k])
    vals2 = np.insert(vals, k, vals[k] * 0.5)
    vals2[k + 1] = vals[k] * 0.5
    rp2 = rp.copy()
    rp2[8:] += 1
    c = _csr(lib, rp2, ci2, vals2, n, p.y, p.v, p.z, p.alpha, p.beta)
    bnd = _csr(lib, rp, ci, vals, n, p.y, p.v, p.z, p.alpha, p.beta, bound=True)
    _close(c, b, bnd, 1e-14)


def check_nan_propagation(lib):
    m, n = 10, 8
    p = datagen.dense_problem(m, n, seed=13)
    X = p.X2d().copy()
    X[4, 6] = np.nan
    out = _dense(lib, X, p.y, p.v, p.z, 1.0, 1.0)
    assert np.all(np.isnan(out))                # t_4 is NaN and reaches every column via X_4j * u_4
    # sparse: only the columns stored in the poisoned row become NaN
    Xs = np.zeros((m, n), np.float32)
    Xs[2, 1], Xs[2, 5], Xs[3, 0], Xs[3, 5], Xs[7, 2] = 1.0, 2.0, -1.0, 0.5, 3.0
    rp, ci, vals = _dense_to_csr(Xs)
    vals[0] = np.nan                            # entry (2, 1)
    out = _csr(lib, rp, ci, vals, n, p.y, p.v, p.z, 1.0, 1.0)
    assert set(np.nonzero(np.isnan(out))[0].tolist()) == {1, 5}
    # v_i == 0 does not skip row i: 0 * inf = NaN
    X = p.X2d().copy()
    X[2, 3] = np.inf
    v = p.v.copy()
    v[2] = 0.0
    out = _dense(lib, X, p.y, v, p.z, 1.0, 1.0)
    assert np.all(np.isnan(out))


def check_scipy(lib):
    p = datagen.csr_random(2000, 300, seed=21, mean_len=12.0, empty_frac=0.1, dup_frac=0.05)
    A = sp.csr_matrix((p.values.astype(np.float64), p.col_idx, p.row_ptr), shape=(p.m, p.n))
    exp = p.alpha * (A.T @ (p.v.astype(np.float64) * (A @ p.y.astype(np.float64)))) + p.beta * p.z
    out = _csr(lib, p.row_ptr, p.col_idx, p.values, p.n, p.y, p.v, p.z, p.alpha, p.beta)
    bnd = _csr(lib, p.row_ptr, p.col_idx, p.values, p.n, p.y, p.v, p.z, p.alpha, p.beta, bound=True)
    _close(out, exp, bnd, 1e-12)


def check_bound(lib):
    p = datagen.dense_problem(30, 20, seed=14)
    ref = _dense(lib, p.X2d(), p.y, p.v, p.z, -1.5, 0.5)
    bnd = _dense(lib, p.X2d(), p.y, p.v, p.z, -1.5, 0.5, bound=True)
    assert np.all(bnd >= np.abs(ref))
    # with non-negative inputs the bound is the value itself
    Xa, ya, va, za = (np.abs(a) for a in (p.X2d(), p.y, p.v, p.z))
    assert np.array_equal(_dense(lib, Xa, ya, va, za, 1.5, 0.5),
                          _dense(lib, Xa, ya, va, za, 1.5, 0.5, bound=True))
    # by hand: X = [[1, -2]], y = [3, 1], v = [-1], z = [-4, 1], alpha = -1, beta = 0.5
    # |X||y| = 5, |v| * 5 = 5, |X|^T 5 = [5, 10], 1 * [5, 10] + 0.5 * [4, 1] = [7, 10.5]
    b = _dense(lib, np.array([[1, -2]], np.float32), np.array([3, 1], np.float32),
               np.array([-1], np.float32), np.array([-4, 1], np.float32), -1.0, 0.5, bound=True)
    assert np.array_equal(b, [7.0, 10.5])


def check_csr_bound(lib):
    """The CSR normaliser D_j on its own: a hand-derived example with mixed signs everywhere, an
    empty row and a repeated column; equality with the dense normaliser of the same matrix (pinned
    by check_bound); D >= |value|; and D equal to the value when every input is non-negative."""
    for name in golden_names():
        g = read_golden(name)
        if "expected_bound" not in g:
            continue
        bnd = _csr(lib, g["row_ptr"], g["col_idx"], g["values"], g["n"], g["y"], g.get("v"), g.get("z"),
                   g["alpha"], g["beta"], bound=True)
        assert np.array_equal(bnd, g["expected_bound"]), (name, bnd, g["expected_bound"])
    # the same matrix stored densely: same sums in the same order (zeros add exactly), so the
    # CSR and dense normalisers agree bit for bit, for signed alpha, beta, v, y, z
    m, n = 90, 41
    p = datagen.dense_problem(m, n, seed=31)
    X = p.X2d().copy()
    X[np.random.default_rng(32).random((m, n)) < 0.75] = 0.0
    X[[3, 40]] = 0.0                                   # empty rows
    rp, ci, vals = _dense_to_csr(X)
    for alpha, beta, v in ((-1.25, -0.5, p.v), (0.75, 2.0, None), (1.0, 0.0, p.v)):
        z = p.z if beta != 0.0 else None
        a = _dense(lib, X, p.y, v, z, alpha, beta, bound=True)
        b = _csr(lib, rp, ci, vals, n, p.y, v, z, alpha, beta, bound=True)
        assert np.array_equal(a, b), (alpha, beta)
    # D >= |value| on an irregular matrix (empty rows, repeated columns), and D == value on
    # non-negative inputs with alpha, beta > 0
    c = datagen.csr_random(300, 70, seed=33, mean_len=6.0, empty_frac=0.2, dup_frac=0.3)
    for alpha, beta in ((-0.7, -1.5), (2.0, 0.25)):
        ref = _csr(lib, c.row_ptr, c.col_idx, c.values, 70, c.y, c.v, c.z, alpha, beta)
        bnd = _csr(lib, c.row_ptr, c.col_idx, c.values, 70, c.y, c.v, c.z, alpha, beta, bound=True)
        assert np.all(bnd >= np.abs(ref))
    pos = [np.abs(t) for t in (c.values, c.y, c.v, c.z)]
    assert np.array_equal(_csr(lib, c.row_ptr, c.col_idx, pos[0], 70, pos[1], pos[2], pos[3], 1.5, 0.5),
                          _csr(lib, c.row_ptr, c.col_idx, pos[0], 70, pos[1], pos[2], pos[3], 1.5, 0.5,
                               bound=True))


def check_thread_independence(lib):
    p = datagen.dense_problem(3001, 37, seed=15)
    c = datagen.csr_random(3001, 37, seed=15, mean_len=6.0)
    prev = lib.oracle_set_threads(0)
    try:
        lib.oracle_set_threads(1)
        a = _dense(lib, p.X2d(), p.y, p.v, p.z, p.alpha, p.beta)
        ac = _csr(lib, c.row_ptr, c.col_idx, c.values, 37, c.y, c.v, c.z, c.alpha, c.beta)
        lib.oracle_set_threads(max(prev, 4))
        b = _dense(lib, p.X2d(), p.y, p.v, p.z, p.alpha, p.beta)
        bc = _csr(lib, c.row_ptr, c.col_idx, c.values, 37, c.y, c.v, c.z, c.alpha, c.beta)
    finally:
        lib.oracle_set_threads(prev)
    assert np.array_equal(a, b) and np.array_equal(ac, bc)


def check_error_codes(lib):
    def raises(fn):
        try:
            fn()
        except oracle.OracleError:
            return True
        return False
    y = np.ones(3, np.float32)
    assert raises(lambda: _dense(lib, np.ones(6, np.float32), y, m=2, n=3, ldx=2))          # ldx < n
    assert raises(lambda: _dense(lib, np.ones((2, 3), np.float32), y, None, None, 1.0, 1.0))  # z missing
    vals = np.ones(3, np.float32)
    assert raises(lambda: _csr(lib, np.array([0, 2, 1, 3], np.int32), np.array([0, 1, 2], np.int32),
                               vals, 3, y))                                                   # decreasing
    assert raises(lambda: _csr(lib, np.array([0, 1, 2, 3], np.int32), np.array([0, 3, 2], np.int32),
                               vals, 3, y))                                                   # col >= n
    assert raises(lambda: _csr(lib, np.array([0, 1, 2, 2], np.int32), np.array([0, 1, 2], np.int32),
                               vals, 3, y))                                                   # end != nnz


# --- the two halves of the pattern (CSR): rowdot t = alpha v (X y) + beta t0, tmv out = alpha X^T u + beta z


def _rowdot(lib, rp, ci, vals, n, y, v=None, t0=None, alpha=1.0, beta=0.0, bound=False):
    return oracle.csr_rowdot(rp, ci, vals, n, y, v, t0, alpha, beta, bound=bound, lib=lib)


def _tmv(lib, rp, ci, vals, n, u, z=None, alpha=1.0, beta=0.0, bound=False):
    return oracle.csr_tmv(rp, ci, vals, n, u, z, alpha, beta, bound=bound, lib=lib)


def check_halves_golden(lib):
    g = read_golden("halves/csr_4x3_rowdot_tmv.txt")
    t = _rowdot(lib, g["row_ptr"], g["col_idx"], g["values"], g["n"], g["y"], g["v"], g["t0"],
                float(g["alpha_r"][0]), float(g["beta_r"][0]))
    assert np.array_equal(t, g["expected_rowdot"].astype(np.float64)), t
    o = _tmv(lib, g["row_ptr"], g["col_idx"], g["values"], g["n"], g["u"], g["z"], float(g["alpha_t"][0]),
             float(g["beta_t"][0]))
    assert np.array_equal(o, g["expected_tmv"].astype(np.float64)), o


def check_halves_explicit_matrix(lib):
    for m, n, seed in [(40, 30, 1), (7, 200, 2), (300, 5, 3)]:
        p = datagen.csr_random(m, n, seed=seed, mean_len=5.0, empty_frac=0.2, dup_frac=0.2)
        X = _csr_to_dense(p.row_ptr, p.col_idx, p.values, m, n)
        g = np.random.default_rng(seed)
        t0 = g.standard_normal(m).astype(np.float32)
        u = g.standard_normal(m).astype(np.float32)
        t = _rowdot(lib, p.row_ptr, p.col_idx, p.values, n, p.y, p.v, t0, 1.5, -0.25)
        expect = 1.5 * p.v.astype(np.float64) * (X @ p.y.astype(np.float64)) - 0.25 * t0
        assert np.allclose(t, expect, rtol=1e-12, atol=1e-12)
        o = _tmv(lib, p.row_ptr, p.col_idx, p.values, n, u, p.z, -0.5, 2.0)
        expect = -0.5 * (X.T @ u.astype(np.float64)) + 2.0 * p.z.astype(np.float64)
        assert np.allclose(o, expect, rtol=1e-12, atol=1e-12)


def check_halves_compose_into_the_pattern(lib):
    # small integers: every intermediate is exact, so the chain equals the full pattern bitwise
    g = np.random.default_rng(9)
    m, n = 60, 45
    X = (g.integers(-3, 4, size=(m, n)) * (g.random((m, n)) < 0.3)).astype(np.float32)
    rp, ci, vals = datagen.csr_from_dense(X)
    y = g.integers(-2, 3, size=n).astype(np.float32)
    v = g.integers(-2, 3, size=m).astype(np.float32)
    z = g.integers(-5, 6, size=n).astype(np.float32)
    u = _rowdot(lib, rp, ci, vals, n, y, v).astype(np.float32)
    assert np.array_equal(_tmv(lib, rp, ci, vals, n, u, z, 2.0, -3.0), _csr(lib, rp, ci, vals, n, y, v, z, 2.0, -3.0))


def check_halves_special_cases(lib):
    p = datagen.csr_random(20, 9, seed=4)
    nan_m = np.full(20, np.nan, np.float32)
    nan_n = np.full(9, np.nan, np.float32)
    t0 = np.arange(20, dtype=np.float32)
    z = np.arange(9, dtype=np.float32)
    # alpha == 0 reads no X, y, v or u; beta == 0 reads no t0 or z
    assert np.array_equal(_rowdot(lib, p.row_ptr, p.col_idx, p.values, 9, nan_n, nan_m, t0, 0.0, 2.0),
                          2.0 * t0.astype(np.float64))
    assert not np.isnan(_rowdot(lib, p.row_ptr, p.col_idx, p.values, 9, p.y, None, nan_m, 1.0, 0.0)).any()
    assert np.array_equal(_tmv(lib, p.row_ptr, p.col_idx, p.values, 9, nan_m, z, 0.0, -1.0), -z.astype(np.float64))
    assert not np.isnan(_tmv(lib, p.row_ptr, p.col_idx, p.values, 9, p.v, nan_n, 1.0, 0.0)).any()
    # v absent means v = 1
    assert np.array_equal(_rowdot(lib, p.row_ptr, p.col_idx, p.values, 9, p.y, None),
                          _rowdot(lib, p.row_ptr, p.col_idx, p.values, 9, p.y, np.ones(20, np.float32)))
    # malformed structure is refused
    bad = p.col_idx.copy()
    bad[0] = 9
    for fn in (lambda: _rowdot(lib, p.row_ptr, bad, p.values, 9, p.y), lambda: _tmv(lib, p.row_ptr, bad, p.values, 9, p.v)):
        try:
            fn()
        except oracle.OracleError:
            continue
        raise AssertionError("malformed CSR accepted")


def check_halves_bounds(lib):
    p = datagen.csr_random(50, 30, seed=6)
    t = _rowdot(lib, p.row_ptr, p.col_idx, p.values, 30, p.y, p.v, p.v, 1.5, -0.5)
    tb = _rowdot(lib, p.row_ptr, p.col_idx, p.values, 30, p.y, p.v, p.v, 1.5, -0.5, bound=True)
    assert (tb >= np.abs(t) - 1e-12).all()
    o = _tmv(lib, p.row_ptr, p.col_idx, p.values, 30, p.v, p.z, 1.5, -0.5)
    ob = _tmv(lib, p.row_ptr, p.col_idx, p.values, 30, p.v, p.z, 1.5, -0.5, bound=True)
    assert (ob >= np.abs(o) - 1e-12).all()
    a = [np.abs(x) for x in (p.values, p.v, p.z)]
    assert np.array_equal(_tmv(lib, p.row_ptr, p.col_idx, a[0], 30, a[1], a[2], 2.0, 3.0),
                          _tmv(lib, p.row_ptr, p.col_idx, a[0], 30, a[1], a[2], 2.0, 3.0, bound=True))


def check_bf16_worked_example(lib):
    # X = [[1.5, -2], [0.25, 3]] in bf16 (bits 0x3FC0, 0xC000, 0x3E80, 0x4040), y = (1, 2), v = (2, -1):
    # t = (1.5 - 4, 0.25 + 6) = (-2.5, 6.25); u = v t = (-5, -6.25);
    # S = X^T u = (1.5(-5) + 0.25(-6.25), -2(-5) + 3(-6.25)) = (-9.0625, -8.75);
    # out = 2 S + 0.5 z with z = (1, -1): (-17.625, -18)
    X = np.array([[0x3FC0, 0xC000], [0x3E80, 0x4040]], dtype=np.uint16)
    y = np.array([1, 2], np.float32)
    v = np.array([2, -1], np.float32)
    z = np.array([1, -1], np.float32)
    got = _dense(lib, X, y, v, z, 2.0, 0.5)
    assert np.array_equal(got, [-17.625, -18.0]), got
    # the bound: |X|^T (|v| (|X| |y|)) = (1.5 * 11 + 0.25 * 6.5, 2 * 11 + 3 * 6.5) with |X||y| = (5.5, 6.25)
    bnd = _dense(lib, X, y, v, z, 2.0, 0.5, bound=True)
    want = 2 * np.array([1.5 * 11 + 0.25 * 6.25, 2 * 11 + 3 * 6.25]) + 0.5
    assert np.array_equal(bnd, want), (bnd, want)


def check_bf16_equals_the_widened_matrix(lib):
    # bf16 X gives exactly the fp32 result of the matrix it denotes (widened here by numpy), for
    # every value class: normal, subnormal, +-0, +-inf, NaN, and a padded leading dimension
    g = np.random.default_rng(7)
    m, n, ldx = 37, 29, 33
    h = datagen.to_bf16(g.normal(0, 3, m * ldx).astype(np.float32))
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF7F], dtype=np.uint16)
    h[: specials.size] = specials
    y = g.uniform(-1, 1, n).astype(np.float32)
    v = g.uniform(-1, 1, m).astype(np.float32)
    z = g.uniform(-1, 1, n).astype(np.float32)
    wide = datagen.bf16_to_f32(h)
    for bound in (False, True):
        a = _dense(lib, h, y, v, z, 0.75, -0.5, m=m, n=n, ldx=ldx, bound=bound)
        b = _dense(lib, wide, y, v, z, 0.75, -0.5, m=m, n=n, ldx=ldx, bound=bound)
        assert np.array_equal(a, b)
    inf_nan = h.copy()
    inf_nan[3 * ldx + 4] = 0x7F80   # +inf in row 3
    inf_nan[5 * ldx + 2] = 0xFFC0   # NaN in row 5
    a = _dense(lib, inf_nan, y, v, z, 0.75, -0.5, m=m, n=n, ldx=ldx)
    b = _dense(lib, datagen.bf16_to_f32(inf_nan), y, v, z, 0.75, -0.5, m=m, n=n, ldx=ldx)
    assert np.array_equal(a, b, equal_nan=True) and np.isnan(a).any()


CHECKS = [check_golden, check_brute_force_dense, check_brute_force_csr, check_exact_integers,
          check_closed_forms, check_special_cases, check_invariants, check_csr_dense_agree,
          check_nan_propagation, check_scipy, check_bound, check_csr_bound, check_thread_independence,
          check_error_codes, check_halves_golden, check_halves_explicit_matrix,
          check_halves_compose_into_the_pattern, check_halves_special_cases, check_halves_bounds,
          check_bf16_worked_example, check_bf16_equals_the_widened_matrix]
