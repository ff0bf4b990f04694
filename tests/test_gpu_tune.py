"""GPU: the empirical tuner (xtvxy_*_tune) and its cache, through the C ABI. The plans it picks are
run again through the _ex entry points and checked against the oracle."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import CsrOnDevice, DenseOnDevice, assert_parity, csr_oracle, dense_oracle, note

pytestmark = pytest.mark.gpu


def check_report(rep):
    assert rep["candidates"] > 1 and rep["from_cache"] == 0
    # the best plan is the fastest of the final round, which includes the model's plan
    assert 0 < rep["best_seconds"] <= rep["model_seconds"]


@pytest.mark.parametrize("m,n", [(30000, 256), (3000, 3000), (512, 20000)])
def test_dense_tune_picks_a_correct_plan_and_caches_it(m, n, tmp_path):
    import torch
    p = datagen.dense_problem(m, n, seed=m + n, z="uniform", beta=0.5)
    d = DenseOnDevice(p)
    X2 = d.X.view(m, n)
    xt.xtvxy_tune_cache_clear()
    note("dense tune m=%d n=%d" % (m, n))
    rep = xt.dense_tune(X2, d.y, d.v, d.z, p.alpha, p.beta, repeats=3)
    check_report(rep)
    ref, bnd = dense_oracle(p)
    best = xt.xtvxy_launch_params(**rep["best"])
    assert_parity(d.run(plan=best), ref, bnd, "dense tuned plan")
    again = xt.dense_tune(X2, d.y, d.v, d.z, p.alpha, p.beta, repeats=3)
    assert again["from_cache"] == 1 and again["best"] == rep["best"]
    aligned = 1 if d.X.data_ptr() % 16 == 0 else 0
    found_rep, found = xt.xtvxy_tune_cache_lookup(0, m, n, n, aligned)
    assert found and found_rep.best.as_dict() == rep["best"]
    path = str(tmp_path / "cache.txt")
    xt.xtvxy_tune_cache_save(path)
    xt.xtvxy_tune_cache_clear()
    assert not xt.xtvxy_tune_cache_lookup(0, m, n, n, aligned)[1]
    xt.xtvxy_tune_cache_load(path)
    found_rep, found = xt.xtvxy_tune_cache_lookup(0, m, n, n, aligned)
    assert found and found_rep.best.as_dict() == rep["best"]
    torch.cuda.synchronize()


@pytest.mark.parametrize("m,n,mean_len", [(20000, 2000, 12.0), (20000, 200000, 20.0)])
def test_csr_tune_picks_a_correct_plan(m, n, mean_len):
    p = datagen.csr_random(m, n, seed=m + n, mean_len=mean_len, beta=0.5)
    d = CsrOnDevice(p)
    xt.xtvxy_tune_cache_clear()
    note("csr tune m=%d n=%d" % (m, n))
    rep = xt.csr_tune(d.rp, d.ci, d.vals, n, d.y, d.v, d.z, p.alpha, p.beta, repeats=3)
    check_report(rep)
    ref, bnd = csr_oracle(p)
    best = xt.xtvxy_launch_params(**rep["best"])
    assert_parity(d.run(plan=best), ref, bnd, "csr tuned plan")
    if n > 8192:  # a wide matrix offers windows, atomics and bins to choose from
        assert rep["candidates"] >= 20
    xt.xtvxy_tune_cache_clear()


@pytest.mark.parametrize("x_dtype,kind", [("bf16", 2), ("f16", 3)])
def test_dense_tune_on_16_bit_x(x_dtype, kind):
    p = datagen.dense_problem(3000, 3000, seed=77, x_dtype=x_dtype, z="uniform", beta=0.5)
    d = DenseOnDevice(p)
    xt.xtvxy_tune_cache_clear()
    note("dense tune %s" % x_dtype)
    rep = xt.dense_tune(d.X.view(p.m, p.n), d.y, d.v, d.z, p.alpha, p.beta, repeats=3)
    check_report(rep)
    ref, bnd = dense_oracle(p)
    assert_parity(d.run(plan=xt.xtvxy_launch_params(**rep["best"])), ref, bnd, "dense %s tuned plan" % x_dtype)
    aligned = 1 if d.X.data_ptr() % 16 == 0 else 0
    found_rep, found = xt.xtvxy_tune_cache_lookup(kind, p.m, p.n, p.n, aligned)
    assert found and found_rep.best.as_dict() == rep["best"]
    assert not xt.xtvxy_tune_cache_lookup(0 if kind != 0 else 2, p.m, p.n, p.n, aligned)[1]  # kinds kept apart
    xt.xtvxy_tune_cache_clear()


def test_csr_tune_on_bf16_values():
    p = datagen.csr_values_bf16(datagen.csr_random(20000, 200000, seed=5, mean_len=20.0, beta=0.5))
    d = CsrOnDevice(p)
    xt.xtvxy_tune_cache_clear()
    note("csr tune bf16 values")
    rep = xt.csr_tune(d.rp, d.ci, d.vals, p.n, d.y, d.v, d.z, p.alpha, p.beta, repeats=3)
    check_report(rep)
    assert rep["best"]["kernel"] != xt.XTVXY_CSR_ROWS
    ref, bnd = csr_oracle(p)
    assert_parity(d.run(plan=xt.xtvxy_launch_params(**rep["best"])), ref, bnd, "csr bf16 tuned plan")
    aligned = 1 if d.vals.data_ptr() % 16 == 0 and d.ci.data_ptr() % 16 == 0 else 0
    assert xt.xtvxy_tune_cache_lookup(4, p.m, p.n, p.nnz, aligned)[1]
    assert not xt.xtvxy_tune_cache_lookup(1, p.m, p.n, p.nnz, aligned)[1]
    xt.xtvxy_tune_cache_clear()
