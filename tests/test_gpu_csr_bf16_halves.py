"""GPU parity of the two halves of the pattern (xtvxy_csr_bf16_rowdot, xtvxy_csr_bf16_tmv) and of the
Newton-CG solver (xtvxy_logreg_newton_cg_bf16) with CSR values stored as bf16, through the C ABI,
against the fp64 oracle run on the values the bf16 bit patterns denote (widened exactly by numpy).
The arithmetic is the fp32 path's, so the tolerances are the fp32 tests' own."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
import oracle.logreg as lr
from gpu_util import CsrOnDevice, note, to_dev
from test_gpu_csr_halves import aux, half_plans, rowdot_case, tmv_case
from test_gpu_logreg import LogregOnDevice, oracle_gradient

pytestmark = pytest.mark.gpu


def bf16_pair(p):
    """(the bf16 problem, the same problem with its values widened to fp32): the first goes to the
    device, the second to the oracle."""
    b = datagen.csr_values_bf16(p, (p.name or "csr") + " bf16")
    w = datagen.CsrProblem(b.m, b.n, b.row_ptr, b.col_idx, b.values_f32(), b.y, b.v, b.z, b.alpha, b.beta,
                           b.name + " widened", dict(b.info))
    return b, w


def test_values_reach_the_device_as_bf16():
    import torch
    b, w = bf16_pair(datagen.csr_random(100, 30, seed=1, mean_len=4.0))
    d = CsrOnDevice(b)
    assert d.vals.dtype == torch.bfloat16 and w.values.dtype == np.float32
    assert np.array_equal(w.values.view(np.uint32) >> 16, b.values.astype(np.uint32))  # widening is exact


@pytest.mark.parametrize("m,n,mean_len", [(1, 1, 1.0), (5, 7, 3.0), (3000, 64, 6.0), (3000, 1000, 40.0),
                                          (2500, 20000, 9.0), (700, 300000, 30.0)])
def test_halves_on_irregular_matrices(m, n, mean_len):
    b, w = bf16_pair(datagen.csr_random(m, n, seed=m + n + 1, mean_len=mean_len, empty_frac=0.2, dup_frac=0.1))
    d = CsrOnDevice(b)
    t0, u = aux(w, 1)
    rowdot_case(w, d, t0, 1.25, -0.5, what="bf16")
    tmv_case(w, d, u, -0.75, 0.5, what="bf16")


@pytest.mark.parametrize("m,n,mean_len", [(2000, 500, 9.0), (500, 30000, 30.0)])
def test_halves_every_variant(m, n, mean_len):
    b, w = bf16_pair(datagen.csr_random(m, n, seed=78, mean_len=mean_len, empty_frac=0.1, dup_frac=0.05))
    d = CsrOnDevice(b)
    t0, u = aux(w, 2)
    for plan in half_plans(m, n, b.nnz):
        rowdot_case(w, d, t0, 0.5, 2.0, plan=plan, what="bf16 forced")
        tmv_case(w, d, u, 1.5, -1.0, plan=plan, what="bf16 forced")


def test_halves_at_misaligned_values():
    # values starting 1..3 entries into their buffer: 2-, 4- and 6-byte offsets from a 16-byte start
    b, w = bf16_pair(datagen.csr_random(1500, 3000, seed=5, mean_len=11.0, empty_frac=0.1))
    t0, u = aux(w, 3)
    for off in (1, 2, 3):
        d = CsrOnDevice(b, entry_offset=off)
        rowdot_case(w, d, t0, 1.0, 0.5, what="bf16 offset %d" % off)
        tmv_case(w, d, u, 1.0, 0.5, what="bf16 offset %d" % off)


def test_halves_compose_into_the_fused_pattern():
    import torch
    b, w = bf16_pair(datagen.WORKLOADS["csr_10000000x1000_logistic_hvp"](m=200_000))
    d = CsrOnDevice(b)
    note("bf16 halves compose")
    t = xt.csr_rowdot(d.rp, d.ci, d.vals, b.n, d.y, d.v)
    out = xt.csr_tmv(d.rp, d.ci, d.vals, b.n, t, d.z, b.alpha, b.beta)
    fused = xt.csr(d.rp, d.ci, d.vals, b.n, d.y, d.v, d.z, b.alpha, b.beta)
    torch.cuda.synchronize()
    import oracle
    ref = oracle.csr(w.row_ptr, w.col_idx, w.values, w.n, w.y, w.v, w.z, w.alpha, w.beta)
    bnd = oracle.csr(w.row_ptr, w.col_idx, w.values, w.n, w.y, w.v, w.z, w.alpha, w.beta, bound=True)
    from gpu_util import assert_parity
    assert_parity(out.cpu().numpy(), ref, bnd, "bf16 rowdot then tmv")
    assert_parity(fused.cpu().numpy(), ref, bnd, "bf16 fused")


@pytest.mark.parametrize("name", ["csr_10000000x1000_logistic_hvp", "csr_5000000x1000000_zipf"])
def test_halves_full_size(name):
    b, w = bf16_pair(datagen.WORKLOADS[name]())
    d = CsrOnDevice(b)
    t0, u = aux(w, 5)
    rowdot_case(w, d, t0, 1.0, 0.5, what="bf16")
    tmv_case(w, d, u, 0.7, 0.3 if w.z is not None else 0.0, what="bf16")


# ---------------------------------------------------------------------------------------------
# the solver


def small_bf16_problem(m, n, seed, lam, mean_len=5.0, soft=False):
    p = datagen.csr_random(m, n, seed=seed, mean_len=mean_len, values="uniform")
    g = np.random.Generator(np.random.PCG64(900 + seed))
    labels = (g.random(m) if soft else (g.random(m) < 0.45)).astype(np.float32)
    vals = datagen.to_bf16((p.values * 1.5).astype(np.float32))
    return p.row_ptr, p.col_idx, vals, n, labels, lam


@pytest.mark.parametrize("m,n,mean_len,lam,soft", [(3000, 40, 6.0, 1.0, False), (5000, 300, 12.0, 0.5, True),
                                                   (1200, 20000, 30.0, 2.0, False)])
def test_solver_fixed_schedule_matches_oracle(m, n, mean_len, lam, soft):
    """K Newton steps of J CG iterations on both sides, the oracle on the widened values; the bars
    are those of the fp32 solver's test of the same schedule."""
    rp, ci, vals, n, labels, lam = small_bf16_problem(m, n, m + n, lam, mean_len, soft)
    K, J = 3, 2
    note("logreg bf16 fixed schedule m=%d n=%d nnz=%d" % (m, n, len(ci)))
    d = LogregOnDevice(rp, ci, vals, n, labels)
    w, rep, hist = d.solve(lam, None, "fused", max_newton=K, max_cg=J, fixed_cg=True, grad_tol=0.0)
    ref = lr.newton_cg(rp, ci, datagen.bf16_to_f32(vals), n, labels, lam, max_newton=K, max_cg=J, fixed_cg=True,
                       grad_tol=0.0)
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


def test_solver_agrees_with_the_fp32_solver_on_the_widened_values():
    rp, ci, vals, n, labels, lam = small_bf16_problem(8000, 400, 17, 0.8, mean_len=15.0)
    note("logreg bf16 vs fp32")
    wb, repb, _ = LogregOnDevice(rp, ci, vals, n, labels).solve(lam, None, grad_tol=1e-6, max_newton=30)
    wf, repf, _ = LogregOnDevice(rp, ci, datagen.bf16_to_f32(vals), n, labels).solve(lam, None, grad_tol=1e-6,
                                                                                    max_newton=30)
    assert repb["status"] == repf["status"] == xt.XTVXY_LOGREG_CONVERGED
    assert np.max(np.abs(wb - wf)) <= 1e-4 * np.max(np.abs(wf))
    assert abs(repb["loss"] - repf["loss"]) <= 1e-6 * abs(repf["loss"])


def test_solver_converges_to_the_optimum():
    rp, ci, vals, n, labels, lam = small_bf16_problem(20000, 500, 6, 1.0, mean_len=20.0)
    note("logreg bf16 converge")
    w, rep, _ = LogregOnDevice(rp, ci, vals, n, labels).solve(lam, None, grad_tol=1e-5, max_newton=30)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED, rep
    g = oracle_gradient(rp, ci, datagen.bf16_to_f32(vals), n, labels, lam, w)
    assert np.linalg.norm(g) <= 3e-5 * rep["grad_norm0"], (np.linalg.norm(g), rep)


def test_solver_refuses_the_unfused_engine():
    rp, ci, vals, n, labels, lam = small_bf16_problem(100, 10, 2, 1.0)
    d = LogregOnDevice(rp, ci, vals, n, labels)
    with pytest.raises(ValueError, match="fused engine only"):
        xt.logreg_newton_cg(d.rp, d.ci, d.vals, n, d.labels, lam, engine="unfused")


def test_solver_full_size_workload():
    # the 10,000,000 x 1000 logistic workload with its values rounded to bf16
    P = datagen.LOGISTIC_WORKLOADS["logreg_csr_10000000x1000"]()
    X = P.X
    vals = datagen.to_bf16(X.values)
    d = LogregOnDevice(X.row_ptr, X.col_idx, vals, X.n, P.labels)
    note("logreg bf16 full size")
    w, rep, hist = d.solve(P.lam, None, grad_tol=1e-4, max_newton=20)
    assert rep["status"] == xt.XTVXY_LOGREG_CONVERGED, rep
    g = oracle_gradient(X.row_ptr, X.col_idx, datagen.bf16_to_f32(vals), X.n, P.labels, P.lam, w)
    assert np.linalg.norm(g) <= 3e-4 * rep["grad_norm0"], (np.linalg.norm(g), rep)
    losses = [h["loss"] for h in hist]
    assert all(b < a for a, b in zip(losses, losses[1:])), losses
