"""GPU parity of the dense path with X stored as bf16 (xtvxy_dense_bf16) against the fp64 oracle run
on the same bf16 matrix (each element widened exactly), through the C ABI. The tolerance is the
fp32 path's: the arithmetic is the same fp32, only X's storage is narrower."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import DenseOnDevice, assert_parity, dense_oracle, note

pytestmark = pytest.mark.gpu


def check(p, plan=None, X_offset=0, what=""):
    note("dense bf16 %s m=%d n=%d ldx=%d plan=%s" % (what or p.name, p.m, p.n, p.ldx,
                                                    None if plan is None else plan.as_dict()))
    d = DenseOnDevice(p, X_offset)
    got = d.run(plan=plan)
    ref, bnd = dense_oracle(p)
    return assert_parity(got, ref, bnd, "bf16 %s m=%d n=%d" % (what or p.name, p.m, p.n))


WIDTHS = [1, 3, 8, 64, 100, 256, 264, 512, 1000, 1024, 2040, 2048, 2056, 3000, 8184, 8192, 8200, 20000]


# every width with 1 and 70 rows, and with 1000 rows while the matrix stays within 8e6 elements
SHAPES = [(m, n) for m in (1, 70, 1000) for n in WIDTHS if m * n <= 8_000_000]


@pytest.mark.parametrize("m,n", SHAPES)
def test_shapes(m, n):
    check(datagen.dense_problem(m, n, seed=m * 31 + n, x_dtype="bf16", z="uniform", beta=0.5))


def test_padded_and_unaligned_rows():
    # ldx not a multiple of 8 and an X that starts 2 elements past a 16-byte boundary: 2-byte loads
    check(datagen.dense_problem(500, 96, seed=1, ldx=100, x_dtype="bf16"), what="ldx 100")
    check(datagen.dense_problem(500, 96, seed=2, ldx=104, x_dtype="bf16"), what="ldx 104")
    check(datagen.dense_problem(400, 256, seed=3, x_dtype="bf16"), X_offset=2, what="unaligned")


def forced_plans(m, n, aligned=True):
    """Every bf16 kernel variant that can cover width n, with a few grid sizes."""
    plans = []
    vecs = [8, 1] if aligned and n % 8 == 0 else [1]
    for vec in vecs:
        for chunks in (1, 2, 4):
            lanes = 1
            while lanes * vec * chunks < n and lanes < 64:
                lanes *= 2
            if lanes * vec * chunks >= n:
                for grid in (1, 5, 64):
                    plans.append(dict(kernel=xt.XTVXY_DENSE_WAVE_ROWS, vec=vec, chunks=chunks, lanes_per_row=lanes,
                                      grid=grid, group=1))
        for chunks in ((1, 2, 4) if vec == 8 else (1, 2, 4, 8)):
            if 256 * vec * chunks >= n:
                for grid in (1, 7, 300):
                    plans.append(dict(kernel=xt.XTVXY_DENSE_BLOCK_ROWS, vec=vec, chunks=chunks, grid=grid, group=1))
            group = -(-n // (256 * vec * chunks))
            if 1 <= group <= 16:
                for units in (1, 3, 16):
                    plans.append(dict(kernel=xt.XTVXY_DENSE_GROUP_ROWS, vec=vec, chunks=chunks, grid=group * units,
                                      group=group))
    return [xt.xtvxy_dense_bf16_plan_complete(m, n, n, xt.xtvxy_launch_params(block_threads=256, **d)) for d in plans]


@pytest.mark.parametrize("m,n", [(333, 8), (257, 104), (300, 256), (129, 1000), (77, 2048), (45, 6000), (20, 30000)])
def test_every_kernel_variant(m, n):
    p = datagen.dense_problem(m, n, seed=11 + n, x_dtype="bf16", z="uniform", beta=-0.5)
    ref, bnd = dense_oracle(p)
    d = DenseOnDevice(p)
    plans = forced_plans(m, n)
    assert plans
    for plan in plans:
        note("forced bf16 %s" % plan.as_dict())
        assert_parity(d.run(plan=plan), ref, bnd, "bf16 forced %s" % plan.as_dict())


def test_special_values_propagate():
    p = datagen.dense_problem(64, 256, seed=5, x_dtype="bf16", z="uniform", beta=0.5)
    X = p.X.copy()
    X[3 * 256 + 7] = 0x7FC0   # NaN in row 3, column 7
    X[9 * 256 + 100] = 0x7F80  # +inf in row 9, column 100
    p.X = X
    d = DenseOnDevice(p)
    got = d.run()
    ref, _ = dense_oracle(p)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).any()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.allclose(got[fin], ref[fin], rtol=1e-4, atol=1e-3)


def test_model_plans_use_16_byte_loads_of_8():
    for m, n, kernel in ((1000, 256, xt.XTVXY_DENSE_WAVE_ROWS), (1000, 4096, xt.XTVXY_DENSE_BLOCK_ROWS),
                         (100, 65536, xt.XTVXY_DENSE_GROUP_ROWS)):
        p = xt.xtvxy_dense_bf16_plan(m, n, n, 1)
        assert p.vec == 8 and p.kernel == kernel, p.as_dict()


@pytest.mark.parametrize("name", ["dense_1000000x256_normal_equations_bf16", "dense_65536x8192_bf16",
                                  "dense_8192x65536_bf16"])
def test_full_size_workloads(name):
    check(datagen.WORKLOADS[name]())
