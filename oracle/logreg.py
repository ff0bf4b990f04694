"""CPU oracle for Newton-CG on L2-regularised logistic regression over CSR X (float64).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU baseline may
import this module; the GPU library never does, and this module imports nothing from it.

"On optimizing machine learning workloads via kernel fusion" (abstract) finds the pattern
alpha * X^T (v * (X y)) + beta * z inside common ML algorithms and ends with a whole ML
algorithm built on the fused kernel, but names no algorithm. The reading used here is the
textbook one in which the pattern is the inner step: L2-regularised logistic regression
solved by Newton's method with a conjugate-gradient inner solve and a backtracking line
search (Nocedal and Wright, "Numerical Optimization", 2nd ed.: Algorithm 7.1, line search
Newton-CG, for the outer and inner loops; Algorithm 3.1, backtracking, for the step length,
with its sufficient-decrease test evaluated on the change of f summed row by row).

The objective, for labels c_i in [0, 1] and lambda >= 0, with t = X w:

    f(w) = sum_i [ log(1 + exp(t_i)) - c_i t_i ] + (lambda / 2) |w|^2

With p = sigmoid(t) its gradient and Hessian are

    g = X^T (p - c) + lambda w,        H = X^T diag(p (1 - p)) X + lambda I,

so a Hessian-vector product H d is the pattern with alpha = 1, v = p (1 - p), y = d,
beta = lambda and z = d.

The steps below are written in that order and notation. Everything is float64; the
sparse products are scipy.sparse CSR products (a library primitive per step). The
margins t are carried from one iterate to the next (t <- t + a X s) instead of being
recomputed from w; both are exact readings of t = X w.

Status codes of a run: 0 converged (|g| <= grad_tol |g_0|), 1 iteration limit,
2 the line search found no acceptable step.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import scipy.sparse as sp

CONVERGED, ITERATION_LIMIT, LINE_SEARCH_FAILED = 0, 1, 2


def csr_matrix(row_ptr, col_idx, values, n) -> sp.csr_matrix:
    """X as a float64 scipy CSR matrix (a column stored twice in a row counts twice)."""
    rp = np.asarray(row_ptr, np.int64)
    m = rp.shape[0] - 1
    return sp.csr_matrix((np.asarray(values, np.float64), np.asarray(col_idx, np.int64), rp), shape=(m, int(n)))


def sigmoid(t):
    """1 / (1 + exp(-t)), evaluated without overflow for either sign of t."""
    t = np.asarray(t, np.float64)
    e = np.exp(-np.abs(t))
    return np.where(t >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def pointwise_loss(t, c):
    """log(1 + exp(t_i)) - c_i t_i for every row."""
    t = np.asarray(t, np.float64)
    return np.logaddexp(0.0, t) - np.asarray(c, np.float64) * t


def objective(t, c, w, lam) -> float:
    """f at the iterate whose margins are t = X w."""
    w = np.asarray(w, np.float64)
    return float(np.sum(pointwise_loss(t, c)) + 0.5 * lam * np.dot(w, w))


def objective_change(t, xs, c, w, s, lam, a) -> float:
    """f(w + a s) - f(w) for the iterate with margins t = X w and xs = X s, summed term by term
    (the change of every row's loss, then of the penalty), so that the rounding of f itself,
    which grows with the number of rows, does not swamp the small decreases near the minimiser."""
    t = np.asarray(t, np.float64)
    w = np.asarray(w, np.float64)
    rows = pointwise_loss(t + a * xs, c) - pointwise_loss(t, c)
    return float(np.sum(rows) + lam * (a * np.dot(w, s) + 0.5 * a * a * np.dot(s, s)))


def curvature_weights(p):
    """Diagonal of the Hessian's middle factor: p_i (1 - p_i)."""
    return p * (1.0 - p)


def gradient(X, p, c, w, lam):
    """g = X^T (p - c) + lambda w."""
    return X.T @ (p - np.asarray(c, np.float64)) + lam * np.asarray(w, np.float64)


def hessian_vector(X, D, lam, d):
    """H d = X^T (D * (X d)) + lambda d: the pattern with alpha 1, v = D, y = z = d, beta = lambda."""
    return X.T @ (D * (X @ d)) + lam * d


def cg_solve(hvp, g, max_cg, eps, fixed_cg):
    """Inner loop of line search Newton-CG: approximately solve H s = -g.

    Starts from s = 0 with residual r = H s + g = g and direction d = -r. Stops when
    |r| < eps (unless fixed_cg), when r vanishes exactly, after max_cg iterations, or on a
    direction of non-positive curvature (then s = -g if that happens at once, else the
    current s). Returns (s, iterations, hit_negative_curvature).
    """
    s = np.zeros_like(g)
    r = g.copy()
    d = -r
    rr = float(np.dot(r, r))
    for j in range(max_cg):
        q = hvp(d)
        kappa = float(np.dot(d, q))
        if not kappa > 0.0:
            return (-g.copy() if j == 0 else s), j + 1, True
        a = rr / kappa
        s = s + a * d
        r = r + a * q
        rr_new = float(np.dot(r, r))
        if rr_new == 0.0 or (not fixed_cg and np.sqrt(rr_new) < eps):
            return s, j + 1, False
        b = rr_new / rr
        d = -r + b * d
        rr = rr_new
    return s, max_cg, False


def backtrack(trial, f0, gs, max_backtracks, c1=1e-4, shrink=0.5):
    """Backtracking line search: the first a in 1, shrink, shrink^2, ... with
    trial(a) <= f0 + c1 a gs (sufficient decrease). Returns (a, trial(a), trials), or
    (None, None, trials) when no trial is accepted. Newton-CG passes trial(a) = f(w + a s) - f(w)
    and f0 = 0."""
    a = 1.0
    for k in range(max_backtracks):
        fa = trial(a)
        if fa <= f0 + c1 * a * gs:
            return a, fa, k + 1
        a *= shrink
    return None, None, max_backtracks


@dataclass
class NewtonResult:
    w: np.ndarray
    status: int
    newton_iterations: int
    cg_iterations: int
    line_search_trials: int
    # one entry per iterate k: loss f_k and |g_k|; for every step taken also the CG
    # iterations, the slope g_k . s_k and the accepted step length
    history: list = field(default_factory=list)


def newton_cg(row_ptr, col_idx, values, n, labels, lam, w0=None, *, max_newton=20, max_cg=50,
              grad_tol=1e-8, cg_forcing=0.5, fixed_cg=False, max_backtracks=30) -> NewtonResult:
    """Line search Newton-CG for the logistic objective above.

    At iterate k: p = sigmoid(t), f_k, g_k; stop when |g_k| <= grad_tol |g_0| or after
    max_newton steps; otherwise CG on H s = -g with the forcing tolerance
    eps_k = min(cg_forcing, sqrt(|g_k|)) |g_k|, then backtracking from a = 1 along s, then
    w <- w + a s and t <- t + a X s.
    """
    X = csr_matrix(row_ptr, col_idx, values, n)
    c = np.asarray(labels, np.float64)
    w = np.zeros(int(n)) if w0 is None else np.asarray(w0, np.float64).copy()
    t = X @ w
    hist = []
    cg_total = trials_total = 0
    g0 = None
    status = ITERATION_LIMIT
    k = 0
    while True:
        p = sigmoid(t)
        f = objective(t, c, w, lam)
        g = gradient(X, p, c, w, lam)
        gnorm = float(np.sqrt(np.dot(g, g)))
        if g0 is None:
            g0 = gnorm
        hist.append({"loss": f, "grad_norm": gnorm})
        if gnorm <= grad_tol * g0:
            status = CONVERGED
            break
        if k == max_newton:
            break
        D = curvature_weights(p)
        eps = min(cg_forcing, np.sqrt(gnorm)) * gnorm
        s, used, _ = cg_solve(lambda d: hessian_vector(X, D, lam, d), g, max_cg, eps, fixed_cg)
        cg_total += used
        xs = X @ s
        gs = float(np.dot(g, s))
        a, _, tried = backtrack(lambda a: objective_change(t, xs, c, w, s, lam, a), 0.0, gs, max_backtracks)
        trials_total += tried
        hist[-1].update({"cg": used, "gs": gs, "step": a})
        if a is None:
            status = LINE_SEARCH_FAILED
            break
        w = w + a * s
        t = t + a * xs
        k += 1
    return NewtonResult(w, status, k, cg_total, trials_total, hist)
