"""GPU parity of the dense path with X stored as IEEE fp16 (xtvxy_dense_f16) against the fp64 oracle
run on the same matrix widened exactly to fp32 (by numpy), through the C ABI. The tolerance is the
fp32 path's: the arithmetic is the same fp32, only X's storage is narrower."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import DenseOnDevice, assert_parity, dense_oracle, note
from test_gpu_dense_bf16 import forced_plans

pytestmark = pytest.mark.gpu


def check(p, plan=None, X_offset=0, what=""):
    note("dense f16 %s m=%d n=%d ldx=%d plan=%s" % (what or p.name, p.m, p.n, p.ldx,
                                                   None if plan is None else plan.as_dict()))
    d = DenseOnDevice(p, X_offset)
    got = d.run(plan=plan)
    ref, bnd = dense_oracle(p)
    return assert_parity(got, ref, bnd, "f16 %s m=%d n=%d" % (what or p.name, p.m, p.n))


def test_x_is_fp16_on_the_device():
    import torch
    p = datagen.dense_problem(10, 16, seed=1, x_dtype="f16")
    assert p.X.dtype == np.float16 and DenseOnDevice(p).X.dtype == torch.float16


@pytest.mark.parametrize("m,n", [(1, 1), (70, 3), (70, 64), (1000, 100), (1000, 256), (1000, 1000), (70, 2056),
                                 (1000, 8192), (70, 8200), (70, 20000), (7, 100000)])
def test_shapes(m, n):
    check(datagen.dense_problem(m, n, seed=m * 37 + n, x_dtype="f16", z="uniform", beta=0.5))


def test_padded_and_unaligned_rows():
    check(datagen.dense_problem(500, 96, seed=1, ldx=100, x_dtype="f16"), what="ldx 100")
    check(datagen.dense_problem(400, 256, seed=3, x_dtype="f16"), X_offset=2, what="unaligned")


@pytest.mark.parametrize("m,n", [(257, 104), (129, 1000), (45, 6000), (20, 30000)])
def test_every_kernel_variant(m, n):
    # the bf16 plans: the same 2 bytes per element, the same layouts
    p = datagen.dense_problem(m, n, seed=13 + n, x_dtype="f16", z="uniform", beta=-0.5)
    ref, bnd = dense_oracle(p)
    d = DenseOnDevice(p)
    for plan in forced_plans(m, n):
        note("forced f16 %s" % plan.as_dict())
        assert_parity(d.run(plan=plan), ref, bnd, "f16 forced %s" % plan.as_dict())


def test_subnormals_and_special_values():
    # fp16 subnormals widen to normal fp32 numbers; NaN and inf stay what they are
    p = datagen.dense_problem(64, 256, seed=5, x_dtype="f16", z="uniform", beta=0.5)
    bits = p.X.view(np.uint16).copy()
    bits[0:256:3] = 0x0001    # 2^-24, the smallest subnormal
    bits[256:512:5] = 0x83FF  # the largest negative subnormal
    bits[3 * 256 + 7] = 0x7E00   # NaN in row 3, column 7
    bits[9 * 256 + 100] = 0x7C00  # +inf in row 9, column 100
    p.X = bits.view(np.float16)
    assert p.X_f32()[0] == np.float32(2.0 ** -24)
    d = DenseOnDevice(p)
    got = d.run()
    ref, _ = dense_oracle(p)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).any()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.allclose(got[fin], ref[fin], rtol=1e-4, atol=1e-3)


def test_exact_integers_bitwise():
    # small integers are exact in fp16 and every partial sum stays below 2^24
    g = np.random.default_rng(7)
    m, n = 300, 520
    X = g.integers(-3, 4, size=(m, n)).astype(np.float32)
    y, v, z = (g.integers(-2, 3, size=s).astype(np.float32) for s in (n, m, n))
    p = datagen.DenseProblem(m, n, n, X.ravel().astype(np.float16), y, v, z, 1.5, 0.5, "integers", "f16")
    S = X.astype(np.int64).T @ (v.astype(np.int64) * (X.astype(np.int64) @ y.astype(np.int64)))
    want = (1.5 * S + 0.5 * z).astype(np.float32)
    d = DenseOnDevice(p)
    for plan in [None] + forced_plans(m, n)[::4]:
        note("f16 exact integers %s" % (None if plan is None else plan.as_dict()))
        assert np.array_equal(d.run(plan=plan), want)


@pytest.mark.parametrize("name", ["dense_1000000x256_normal_equations_f16", "dense_65536x8192_f16",
                                  "dense_8192x65536_f16"])
def test_full_size_workloads(name):
    check(datagen.WORKLOADS[name]())
