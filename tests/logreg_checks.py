"""Checks that pin the Newton-CG logistic-regression oracle (oracle/logreg.py) to something
other than itself.

Each ``check_*`` takes the oracle module (or a deliberately broken copy of it, see
test_oracle_logreg.py) and raises AssertionError on a mismatch. What they rest on:
a closed-form minimiser, the optimality condition evaluated with plain Python loops,
scipy's BFGS on an objective written here with dense numpy, finite differences of that
objective for the gradient and the Hessian, an exact linear solve for the CG inner loop,
the convergence rate Newton's method must show, and the line search's rule on
hand-made slopes.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.optimize

import datagen


def _problem(m, n, seed, *, lam, mean_len=3.0, soft=False):
    """Small irregular CSR (empty rows, unsorted and repeated columns) with N(0, 1)-ish values
    and labels in {0, 1} (or in [0, 1] when ``soft``)."""
    p = datagen.csr_random(m, n, seed=seed, mean_len=mean_len, values="uniform")
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    vals = (p.values * 2.0).astype(np.float32)
    labels = (g.random(m) if soft else (g.random(m) < 0.4)).astype(np.float32)
    return p.row_ptr, p.col_idx, vals, n, labels, float(lam)


def _dense(rp, ci, vals, m, n):
    X = np.zeros((m, n))
    for i in range(m):
        for k in range(rp[i], rp[i + 1]):
            X[i, ci[k]] += float(vals[k])
    return X


def _f_dense(X, c, lam):
    """The objective written with dense numpy: sum log(1 + e^t) - c t + lam/2 |w|^2."""
    c = np.asarray(c, np.float64)

    def f(w):
        t = X @ w
        return float(np.sum(np.logaddexp(0.0, t) - c * t) + 0.5 * lam * (w @ w))
    return f


def _grad_loops(rp, ci, vals, c, lam, w):
    """Gradient of the objective by plain loops over the stored entries."""
    g = [lam * float(x) for x in w]
    for i in range(len(rp) - 1):
        t = 0.0
        for k in range(rp[i], rp[i + 1]):
            t += float(vals[k]) * float(w[ci[k]])
        pr = 1.0 / (1.0 + math.exp(-t)) if t >= 0 else math.exp(t) / (1.0 + math.exp(t))
        for k in range(rp[i], rp[i + 1]):
            g[ci[k]] += float(vals[k]) * (pr - float(c[i]))
    return np.array(g)


def check_closed_form_single_feature(lr):
    # every row stores the value 2 in column 0 (some rows as 1 + 1, a repeated column); with
    # lambda = 0 the minimiser solves m sigmoid(2 w) = (number of ones): w* = logit(k / m) / 2
    m, k = 10, 3
    rp, ci, vals = [0], [], []
    for i in range(m):
        if i % 3 == 0:
            ci += [0, 0]
            vals += [1.0, 1.0]
        else:
            ci += [0]
            vals += [2.0]
        rp.append(len(ci))
    labels = np.array([1.0] * k + [0.0] * (m - k), np.float32)
    r = lr.newton_cg(np.array(rp, np.int32), np.array(ci, np.int32), np.array(vals, np.float32), 1, labels, 0.0,
                     grad_tol=1e-14, max_newton=50)
    want = math.log(k / (m - k)) / 2.0
    assert r.status == lr.CONVERGED, r.status
    assert abs(r.w[0] - want) <= 1e-10, (r.w[0], want)
    # with lambda > 0 the same objective in one variable, minimised by a bracketing scalar search
    lam = 3.0
    r = lr.newton_cg(np.array(rp, np.int32), np.array(ci, np.int32), np.array(vals, np.float32), 1, labels, lam,
                     grad_tol=1e-14, max_newton=50)
    f = lambda w: m * math.log1p(math.exp(2 * w)) - 2 * k * w + 0.5 * lam * w * w
    ref = scipy.optimize.minimize_scalar(f, bracket=(-2.0, 0.0), tol=1e-12).x
    assert abs(r.w[0] - ref) <= 1e-6, (r.w[0], ref)


def check_optimality_by_loops(lr):
    # from a far start point (which makes the line search shorten steps), the returned w has
    # a vanishing gradient when the gradient is evaluated by plain loops from w itself
    for seed, soft in ((1, False), (2, True)):
        rp, ci, vals, n, c, lam = _problem(40, 6, seed, lam=0.7, soft=soft)
        w0 = np.random.Generator(np.random.PCG64(seed)).normal(0, 8.0, n)
        r = lr.newton_cg(rp, ci, vals, n, c, lam, w0=w0, grad_tol=1e-11, max_newton=60)
        assert r.status == lr.CONVERGED, r.status
        g = _grad_loops(rp, ci, vals, c, lam, r.w)
        g0 = _grad_loops(rp, ci, vals, c, lam, w0)
        assert np.max(np.abs(g)) <= 1e-10 * np.max(np.abs(g0)), (np.max(np.abs(g)), np.max(np.abs(g0)))
        assert r.history[-1]["grad_norm"] <= 1e-11 * r.history[0]["grad_norm"]
        if not soft:
            steps = [h["step"] for h in r.history if "step" in h]
            assert min(steps) < 1.0, steps  # the fixture exercises shortened steps


def check_matches_bfgs(lr):
    # scipy's BFGS on the dense objective with finite-difference gradients finds the same w
    rp, ci, vals, n, c, lam = _problem(60, 5, 3, lam=0.5)
    X = _dense(rp, ci, vals, 60, n)
    ref = scipy.optimize.minimize(_f_dense(X, c, lam), np.zeros(n), method="BFGS",
                                  options={"gtol": 1e-9, "maxiter": 1000}).x
    r = lr.newton_cg(rp, ci, vals, n, c, lam, grad_tol=1e-12)
    assert np.max(np.abs(r.w - ref)) <= 2e-6 * max(1.0, np.max(np.abs(ref))), (r.w, ref)
    f = _f_dense(X, c, lam)
    assert abs(r.history[-1]["loss"] - f(r.w)) <= 1e-12 * abs(f(r.w))


def check_derivatives_by_differences(lr):
    # gradient and Hessian against central differences of the dense objective: directional
    # derivatives for the gradient, second differences and polarisation for H
    rp, ci, vals, n, c, lam = _problem(50, 4, 4, lam=0.9, soft=True)
    X = _dense(rp, ci, vals, 50, n)
    f = _f_dense(X, c, lam)
    Xs = lr.csr_matrix(rp, ci, vals, n)
    gen = np.random.Generator(np.random.PCG64(44))
    w = gen.normal(0, 0.7, n)
    p = lr.sigmoid(Xs @ w)
    g = lr.gradient(Xs, p, c, w, lam)
    D = lr.curvature_weights(p)
    h = 1e-4
    for _ in range(4):
        d = gen.normal(0, 1, n)
        fd = (f(w + h * d) - f(w - h * d)) / (2 * h)
        assert abs(g @ d - fd) <= 1e-6 * (1 + abs(fd)), (g @ d, fd)
    q = lambda d: (f(w + 1e-3 * d) - 2 * f(w) + f(w - 1e-3 * d)) / 1e-6  # d^T H d
    E = np.eye(n)
    H_fd = np.empty((n, n))
    for i in range(n):
        for j in range(n):
            H_fd[i, j] = (q(E[i] + E[j]) - q(E[i] - E[j])) / 4.0
    H = np.column_stack([lr.hessian_vector(Xs, D, lam, E[j]) for j in range(n)])
    assert np.max(np.abs(H - H_fd)) <= 1e-4 * np.max(np.abs(H_fd)), np.max(np.abs(H - H_fd))


def check_cg_solves_exactly(lr):
    # with n iterations and no early exit, CG solves an SPD system to rounding
    gen = np.random.Generator(np.random.PCG64(5))
    n = 7
    A = gen.normal(size=(n, n))
    H = A @ A.T + 0.5 * np.eye(n)
    g = gen.normal(size=n)
    s, used, neg = lr.cg_solve(lambda d: H @ d, g, n, 0.0, True)
    assert not neg and used <= n
    ref = np.linalg.solve(H, -g)
    assert np.max(np.abs(s - ref)) <= 1e-9 * np.max(np.abs(ref)), (s, ref)
    # with a forcing tolerance, the residual of the returned s meets it
    s, used, _ = lr.cg_solve(lambda d: H @ d, g, 50, 1e-3 * np.linalg.norm(g), False)
    assert np.linalg.norm(H @ s + g) < 1e-3 * np.linalg.norm(g)
    # a first direction of zero curvature returns the steepest-descent direction
    s, used, neg = lr.cg_solve(lambda d: np.diag([1.0, -1.0]) @ d, np.array([1.0, 1.0]), 5, 0.0, False)
    assert neg and used == 1 and np.array_equal(s, [-1.0, -1.0])


def check_newton_rate(lr):
    # Inexact Newton with the true Hessian and the forcing term min(1/2, sqrt|g|) converges with
    # order 3/2 once sqrt|g| < 1/2: |g_{k+1}| <= C |g_k|^(3/2). A wrong Hessian, or a forcing
    # term that does not shrink with |g|, converges linearly. lambda is of the order of the data
    # curvature, so a Hessian that drops it is far off.
    rp, ci, vals, n, c, lam = _problem(80, 8, 6, lam=2.0, mean_len=4.0)
    r = lr.newton_cg(rp, ci, vals, n, c, lam, w0=np.full(n, 0.5), grad_tol=1e-11, max_newton=40, max_cg=50)
    assert r.status == lr.CONVERGED and r.newton_iterations <= 11, (r.status, r.newton_iterations)
    gn = [h["grad_norm"] for h in r.history]
    fast = [(a, b) for a, b in zip(gn, gn[1:]) if a < 0.2 and b > 1e-12 * gn[0]]
    assert len(fast) >= 3, gn
    for a, b in fast:
        assert b <= 3.0 * a ** 1.5, gn


def check_descent_and_sufficient_decrease(lr):
    # every accepted step goes downhill along a descent direction and meets the 1e-4 slope rule
    rp, ci, vals, n, c, lam = _problem(60, 6, 7, lam=0.3)
    w0 = np.random.Generator(np.random.PCG64(7)).normal(0, 6.0, n)
    r = lr.newton_cg(rp, ci, vals, n, c, lam, w0=w0, grad_tol=1e-12, max_newton=60)
    h = r.history
    for k in range(len(h) - 1):
        assert h[k]["gs"] < 0
        assert h[k + 1]["loss"] <= h[k]["loss"] + 1e-4 * h[k]["step"] * h[k]["gs"] + 1e-12 * abs(h[k]["loss"])


def check_objective_change(lr):
    # the line search's f(w + a s) - f(w), summed row by row, against two evaluations of the
    # dense objective
    rp, ci, vals, n, c, lam = _problem(50, 5, 9, lam=0.8, soft=True)
    X = _dense(rp, ci, vals, 50, n)
    f = _f_dense(X, c, lam)
    gen = np.random.Generator(np.random.PCG64(9))
    w, s = gen.normal(0, 1, n), gen.normal(0, 1, n)
    for a in (1.0, 0.25, 1e-3):
        got = lr.objective_change(X @ w, X @ s, c, w, s, lam, a)
        want = f(w + a * s) - f(w)
        assert abs(got - want) <= 1e-9 * abs(want), (a, got, want)


def check_line_search_rule(lr):
    # hand-made trials: no decrease at all is never accepted; a decrease of exactly the
    # required slope is accepted at once; the step halves until the rule holds
    a, fa, k = lr.backtrack(lambda a: 0.0, 0.0, -1.0, 10)
    assert a is None and k == 10
    a, fa, k = lr.backtrack(lambda a: -1e-4 * a, 0.0, -1.0, 10)
    assert a == 1.0 and k == 1
    a, fa, k = lr.backtrack(lambda a: (a - 0.1) ** 2 - 0.01, 0.0, -0.2, 30)
    assert a == 0.125 and k == 4, (a, k)
    a, fa, k = lr.backtrack(lambda a: float("nan"), 0.0, -1.0, 5)
    assert a is None and k == 5


def check_conventions(lr):
    # fixed_cg runs exactly max_cg inner iterations; grad_tol 0 runs exactly max_newton steps;
    # a zero gradient at the start stops at once; NaN labels end with a failed line search
    rp, ci, vals, n, c, lam = _problem(50, 6, 8, lam=1.0)
    r = lr.newton_cg(rp, ci, vals, n, c, lam, grad_tol=0.0, max_newton=3, max_cg=2, fixed_cg=True)
    assert r.status == lr.ITERATION_LIMIT and r.newton_iterations == 3 and r.cg_iterations == 6
    assert len(r.history) == 4 and all(h["cg"] == 2 for h in r.history[:3])
    # the stop is the first iterate with |g_k| <= grad_tol |g_0| (relative to the start)
    r = lr.newton_cg(rp, ci, vals, n, c * 0 + 1, lam, grad_tol=1e-2, max_newton=40)
    gn = [h["grad_norm"] for h in r.history]
    assert r.status == lr.CONVERGED and gn[0] > 1.0 and gn[-1] <= 1e-2 * gn[0], gn
    assert all(x > 1e-2 * gn[0] for x in gn[:-1]), gn
    half = np.full(50, 0.5, np.float32)  # labels 1/2 at w = 0: the gradient is lambda w = 0
    r = lr.newton_cg(rp, ci, vals, n, half, lam)
    assert r.status == lr.CONVERGED and r.newton_iterations == 0 and np.all(r.w == 0)
    bad = c.copy()
    bad[3] = np.nan
    r = lr.newton_cg(rp, ci, vals, n, bad, lam, max_newton=5, max_backtracks=4)
    assert r.status == lr.LINE_SEARCH_FAILED and r.line_search_trials == 4


CHECKS = [check_closed_form_single_feature, check_optimality_by_loops, check_matches_bfgs,
          check_derivatives_by_differences, check_cg_solves_exactly, check_newton_rate,
          check_descent_and_sufficient_decrease, check_objective_change, check_line_search_rule,
          check_conventions]
