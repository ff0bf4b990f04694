"""GPU parity of the unfused library comparator (rocBLAS / rocSPARSE + one elementwise kernel)."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import CsrOnDevice, DenseOnDevice, assert_parity, csr_oracle, dense_oracle, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,v,beta", [(2048, 128, "uniform", 0.5), (20000, 256, None, 0.0), (300, 8192, "uniform", 1.0),
                                        (64, 20000, "uniform01", -1.0), (1, 1, "uniform", 0.5)])
def test_dense_comparator(m, n, v, beta):
    p = datagen.dense_problem(m, n, seed=m + n, v=v, z="uniform", beta=beta)
    note("dense unfused m=%d n=%d" % (m, n))
    got = DenseOnDevice(p).run(unfused=True)
    ref, bnd = dense_oracle(p)
    assert_parity(got, ref, bnd, "dense unfused")


def test_dense_comparator_in_place_and_quick_returns():
    p = datagen.dense_problem(500, 300, seed=3)
    d = DenseOnDevice(p)
    separate = d.run(unfused=True)
    z_orig = d.z
    zz = d.z.clone()
    d.z = zz
    assert np.array_equal(d.run(unfused=True, out=zz), separate)
    d.z = z_orig
    assert np.array_equal(d.run(unfused=True, alpha=0.0, beta=0.5), (np.float32(0.5) * p.z).astype(np.float32))


@pytest.mark.parametrize("m,n,mean_len", [(3000, 1000, 10.0), (2000, 50000, 30.0), (10, 5, 2.0)])
@pytest.mark.parametrize("beta", [0.0, 0.75])
def test_csr_comparator(m, n, mean_len, beta):
    import torch
    p = datagen.csr_random(m, n, seed=m + n, mean_len=mean_len, beta=beta)
    d = CsrOnDevice(p)
    note("csr unfused m=%d n=%d" % (m, n))
    plan = xt.CsrUnfusedPlan(d.rp, d.ci, d.vals, n)
    out = torch.full((n,), float("nan"), device="cuda")  # beta == 0 must not read out
    plan(d.y, d.v, d.z if beta else None, p.alpha, beta, out=out)
    torch.cuda.synchronize()
    ref, bnd = csr_oracle(datagen.CsrProblem(m, n, p.row_ptr, p.col_idx, p.values, p.y, p.v,
                                             p.z if beta else None, p.alpha, beta))
    assert_parity(out.cpu().numpy(), ref, bnd, "csr unfused")
    plan.close()
