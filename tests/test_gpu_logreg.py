"""GPU Newton-CG logistic regression (xtvxy_logreg_newton_cg_f32, both engines) against the fp64
oracle of oracle/logreg.py, through the C ABI.

Two kinds of comparison:
  * a fixed schedule (grad_tol 0, fixed_cg, K Newton steps of J CG iterations): both sides take
    the same steps of the same algorithm, so the iterates, losses and gradient norms are
    compared step by step;
  * a run to a tolerance: the w the GPU returns must satisfy the optimality condition, with its
    gradient evaluated by the oracle in fp64, to about the requested tolerance.
Tolerances: the solver works in fp32 vectors with fp64 reductions. One Hessian-vector product
agrees with the oracle to about 1e-6 of its absolute-value bound (the pattern's own parity
bar is 1e-4); K steps of J CG iterations compound that to the 1e-4 relative allowed for the
iterates below; the loss is a fp64 sum of fp32 margins, good to about 1e-6 relative.
"""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
import oracle.logreg as lr
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


class LogregOnDevice:
    def __init__(self, rp, ci, vals, n, labels):
        self.n = n
        self.rp, self.ci, self.vals, self.labels = to_dev(rp), to_dev(ci), to_dev(vals), to_dev(labels)
        self.plan = None

    def solve(self, lam, w0=None, engine="fused", **kw):
        import torch
        w = torch.zeros(self.n, dtype=torch.float32, device=self.rp.device) if w0 is None else to_dev(
            np.asarray(w0, np.float32))
        if engine == "unfused" and self.plan is None:
            self.plan = xt.CsrUnfusedPlan(self.rp, self.ci, self.vals, self.n)
        w, rep, hist = xt.logreg_newton_cg(self.rp, self.ci, self.vals, self.n, self.labels, lam, w, engine=engine,
                                           unfused_plan=self.plan, **kw)
        torch.cuda.synchronize()
        return w.cpu().numpy().astype(np.float64), rep, hist


def small_problem(m, n, seed, lam, mean_len=5.0, soft=False):
    p = datagen.csr_random(m, n, seed=seed, mean_len=mean_len, values="uniform")
    g = np.random.Generator(np.random.PCG64(500 + seed))
    labels = (g.random(m) if soft else (g.random(m) < 0.45)).astype(np.float32)
    vals = (p.values * 1.5).astype(np.float32)
    return p.row_ptr, p.col_idx, vals, n, labels, lam


def oracle_gradient(rp, ci, vals, n, labels, lam, w):
    X = lr.csr_matrix(rp, ci, vals, n)
    return lr.gradient(X, lr.sigmoid(X @ w), labels, w, lam)


def compare_fixed_schedule(prob, engine, K=3, J=2, w0=None):
    """K Newton steps of J CG iterations on both sides. The schedules below keep the last step
    taken at |g| >= 5e-4 |g_0|, far above the fp32 rounding of g (a few 1e-6 |g_0| here), and
    every line-search decision of these cases clears its threshold by a factor of thousands, so
    both sides take the same decisions."""
    rp, ci, vals, n, labels, lam = prob
    note("logreg fixed schedule %s m=%d n=%d nnz=%d K=%d J=%d" % (engine, len(rp) - 1, n, len(ci), K, J))
    d = LogregOnDevice(rp, ci, vals, n, labels)
    w, rep, hist = d.solve(lam, w0, engine, max_newton=K, max_cg=J, fixed_cg=True, grad_tol=0.0)
    ref = lr.newton_cg(rp, ci, vals, n, labels, lam, w0=None if w0 is None else np.asarray(w0, np.float64),
                       max_newton=K, max_cg=J, fixed_cg=True, grad_tol=0.0)
    assert rep["status"] == ref.status and rep["newton_iterations"] == ref.newton_iterations
    assert rep["cg_iterations"] == ref.cg_iterations and rep["line_search_trials"] == ref.line_search_trials
    g0 = ref.history[0]["grad_norm"]
    for k, (a, b) in enumerate(zip(hist, ref.history)):
        assert abs(a["loss"] - b["loss"]) <= 1e-6 * abs(b["loss"]) + 1e-6, (k, a, b)
        assert abs(a["grad_norm"] - b["grad_norm"]) <= 1e-4 * g0, (k, a, b)
        if "step" in b:
            assert a["step"] == b["step"] and a["cg"] == b["cg"], (k, a, b)
    scale = max(np.max(np.abs(ref.w)), 1e-30)
    assert np.max(np.abs(w - ref.w)) <= 1e-4 * scale, np.max(np.abs(w - ref.w)) / scale
    return rep


@pytest.mark.parametrize("engine", ["fused", "unfused"])
@pytest.mark.parametrize("m,n,mean_len,lam,soft", [(3000, 40, 6.0, 1.0, False), (5000, 300, 12.0, 0.5, True),
                                                   (1200, 20000, 30.0, 2.0, False)])
def test_fixed_schedule_matches_oracle(engine, m, n, mean_len, lam, soft):
    # n = 20000 takes the many-workgroup CG update (n above one workgroup's share)
    compare_fixed_schedule(small_problem(m, n, m + n, lam, mean_len, soft), engine)


@pytest.mark.parametrize("engine", ["fused", "unfused"])
def test_fixed_schedule_reads_back_once_per_stage_or_not(engine):
    """With grad_tol == 0 the fixed CG solve is enqueued behind the gradient and both are read back
    once; a tolerance too small to stop on (1e-30) takes the path that reads the gradient first.
    Same kernels in the same order: the same steps, counts and iterates (to the run-to-run
    variation of the CSR sums' order)."""
    rp, ci, vals, n, labels, lam = small_problem(4000, 200, 21, 0.7, mean_len=8.0)
    d = LogregOnDevice(rp, ci, vals, n, labels)
    note("logreg fixed schedule read-backs %s" % engine)
    w1, rep1, hist1 = d.solve(lam, None, engine, max_newton=4, max_cg=3, fixed_cg=True, grad_tol=0.0)
    w2, rep2, hist2 = d.solve(lam, None, engine, max_newton=4, max_cg=3, fixed_cg=True, grad_tol=1e-30)
    for key in ("status", "newton_iterations", "cg_iterations", "line_search_trials"):
        assert rep1[key] == rep2[key], key
    def same(x, y):  # rows after the last step hold NaN for the CG and line-search fields
        return (x is None and y is None) or x == y or (np.isnan(x) and np.isnan(y))

    for a, b in zip(hist1, hist2):
        assert abs(a["loss"] - b["loss"]) <= 1e-7 * abs(b["loss"]), (a, b)  # the sums' order varies
        assert same(a.get("cg"), b.get("cg")) and same(a.get("step"), b.get("step")), (a, b)
    assert np.max(np.abs(w1 - w2)) <= 1e-5 * max(np.max(np.abs(w2)), 1e-30)


@pytest.mark.parametrize("engine", ["fused", "unfused"])
def test_fixed_schedule_from_a_far_start_backtracks(engine):
    prob = small_problem(2000, 30, 11, 0.3, mean_len=4.0)
    w0 = np.random.Generator(np.random.PCG64(3)).normal(0, 6.0, 30)
    rep = compare_fixed_schedule(prob, engine, K=4, J=2, w0=w0)
    assert rep["line_search_trials"] > rep["newton_iterations"]  # some step was shortened


@pytest.mark.parametrize("engine", ["fused", "unfused"])
def test_converges_to_the_optimum(engine):
    rp, ci, vals, n, labels, lam = small_problem(20000, 500, 5, 1.0, mean_len=20.0)
    note("logreg converge %s" % engine)
    d = LogregOnDevice(rp, ci, vals, n, labels)
    w, rep, hist = d.solve(lam, None, engine, grad_tol=1e-5, max_newton=30)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED, rep
    g = oracle_gradient(rp, ci, vals, n, labels, lam, w)
    assert np.linalg.norm(g) <= 3e-5 * rep["grad_norm0"], (np.linalg.norm(g), rep)
    ref = lr.newton_cg(rp, ci, vals, n, labels, lam, grad_tol=1e-10)
    assert np.max(np.abs(w - ref.w)) <= 1e-4 * np.max(np.abs(ref.w))
    assert abs(rep["loss"] - ref.history[-1]["loss"]) <= 1e-6 * abs(ref.history[-1]["loss"])


def test_degenerate_shapes():
    # no rows: f = lambda/2 |w|^2, minimised at w = 0 in one exact Newton step
    rp = np.zeros(1, np.int32)
    d = LogregOnDevice(rp, np.zeros(0, np.int32), np.zeros(0, np.float32), 6, np.zeros(0, np.float32))
    note("logreg no rows")
    w, rep, _ = d.solve(2.0, np.arange(6, dtype=np.float32) - 2.5, grad_tol=1e-6)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED and rep["newton_iterations"] == 1
    assert np.max(np.abs(w)) <= 1e-6
    # no stored entries: t = 0, the gradient is X^T (1/2 - c) + lambda w = lambda w
    rp = np.zeros(9, np.int32)
    d = LogregOnDevice(rp, np.zeros(0, np.int32), np.zeros(0, np.float32), 3, np.ones(8, np.float32))
    note("logreg no entries")
    w, rep, hist = d.solve(1.0, np.ones(3, np.float32), grad_tol=1e-6)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED and np.max(np.abs(w)) <= 1e-6
    assert abs(hist[0]["loss"] - (8 * np.log(2.0) + 1.5)) <= 1e-6
    # no columns: nothing to fit, converged at once
    rp = np.zeros(5, np.int32)
    d = LogregOnDevice(rp, np.zeros(0, np.int32), np.zeros(0, np.float32), 0, np.ones(4, np.float32))
    note("logreg no columns")
    _, rep, hist = d.solve(1.0, None)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED and rep["newton_iterations"] == 0
    assert abs(rep["loss"] - 4 * np.log(2.0)) <= 1e-6


def test_labels_at_one_half_are_already_optimal():
    rp, ci, vals, n, labels, lam = small_problem(500, 20, 2, 1.0)
    d = LogregOnDevice(rp, ci, vals, n, np.full(500, 0.5, np.float32))
    note("logreg labels 1/2")
    w, rep, _ = d.solve(lam, None)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED and rep["newton_iterations"] == 0 and np.all(w == 0)


def test_nan_label_ends_in_a_failed_line_search():
    rp, ci, vals, n, labels, lam = small_problem(500, 20, 3, 1.0)
    labels = labels.copy()
    labels[7] = np.nan
    d = LogregOnDevice(rp, ci, vals, n, labels)
    note("logreg NaN label")
    _, rep, _ = d.solve(lam, None, max_newton=5, max_backtracks=4)
    ref = lr.newton_cg(rp, ci, vals, n, labels, lam, max_newton=5, max_backtracks=4)
    assert rep["status"] == ref.status == xt.XTVXY_LOGREG_LINE_SEARCH_FAILED
    assert rep["line_search_trials"] == ref.line_search_trials == 4


def test_separable_data_without_penalty_stops_at_the_limit():
    # one feature that separates the labels perfectly: with lambda = 0 the loss has no minimiser
    m = 200
    rp = np.arange(m + 1, dtype=np.int32)
    ci = np.zeros(m, np.int32)
    vals = np.where(np.arange(m) % 2 == 0, 1.0, -1.0).astype(np.float32)
    labels = (vals > 0).astype(np.float32)
    d = LogregOnDevice(rp, ci, vals, 1, labels)
    note("logreg separable")
    w, rep, _ = d.solve(0.0, None, max_newton=8, grad_tol=0.0)
    assert rep["status"] in (xt.XTVXY_LOGREG_ITERATION_LIMIT, xt.XTVXY_LOGREG_LINE_SEARCH_FAILED)
    assert np.isfinite(w[0]) and w[0] > 3.0 and rep["loss"] < rep["loss0"]


@pytest.mark.parametrize("engine", ["fused", "unfused"])
def test_full_size_workload(engine):
    # the 10,000,000 x 1000 logistic workload, both engines, checked by the optimality condition
    P = datagen.LOGISTIC_WORKLOADS["logreg_csr_10000000x1000"]()
    X = P.X
    d = LogregOnDevice(X.row_ptr, X.col_idx, X.values, X.n, P.labels)
    note("logreg full size %s" % engine)
    w, rep, hist = d.solve(P.lam, None, engine, grad_tol=1e-4, max_newton=20)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED, rep
    g = oracle_gradient(X.row_ptr, X.col_idx, X.values, X.n, P.labels, P.lam, w)
    assert np.linalg.norm(g) <= 3e-4 * rep["grad_norm0"], (np.linalg.norm(g), rep)
    # every accepted step decreased the loss
    losses = [h["loss"] for h in hist]
    assert all(b < a for a, b in zip(losses, losses[1:])), losses
