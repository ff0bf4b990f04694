"""GPU parity of the fused dense path against the fp64 oracle (runs through the C ABI)."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import DenseOnDevice, assert_parity, dense_oracle, note

pytestmark = pytest.mark.gpu


def check(p, plan=None, X_offset=0, what=""):
    note("dense %s m=%d n=%d ldx=%d plan=%s" % (what or p.name, p.m, p.n, p.ldx,
                                               None if plan is None else plan.as_dict()))
    d = DenseOnDevice(p, X_offset)
    got = d.run(plan=plan)
    ref, bnd = dense_oracle(p)
    return assert_parity(got, ref, bnd, "%s m=%d n=%d" % (what or p.name, p.m, p.n))


def test_small_workload_2048x128():
    check(datagen.WORKLOADS["dense_2048x128"]())


WIDTHS = [1, 2, 3, 4, 5, 31, 64, 100, 128, 255, 256, 257, 511, 512, 600, 1000, 1023, 1024, 1025, 2048, 3000,
          4096, 5000, 8191, 8192, 8193, 12000, 16385, 20000]


# (m, n) pairs of the width sweep: every width with 1, 3 and 70 rows, and with 1000 rows while the
# matrix stays within 8e6 elements (the wider ones are covered by the smaller m)
SHAPES = [(m, n) for m in (1, 3, 70, 1000) for n in WIDTHS if m * n <= 8_000_000]


@pytest.mark.parametrize("m,n", SHAPES)
def test_shapes(m, n):
    check(datagen.dense_problem(m, n, seed=m * 7919 + n))


def test_normal_equations_instance_scaled():
    # v absent, beta 0, N(0, 1) data: the normal-equations recipe at 50k rows
    check(datagen.WORKLOADS["dense_1000000x256_normal_equations"](m=50_000))


def forced_plans(m, n, aligned=True):
    """Every kernel variant that can cover width n, with a few grid sizes."""
    plans = []
    vecs = [4, 1] if aligned and n % 4 == 0 else [1]
    for vec in vecs:
        for chunks in (1, 2, 4):
            lanes = 1
            while lanes * vec * chunks < n and lanes < 64:
                lanes *= 2
            if lanes * vec * chunks >= n:
                for grid in (1, 5, 64):
                    plans.append(dict(kernel=xt.XTVXY_DENSE_WAVE_ROWS, vec=vec, chunks=chunks, lanes_per_row=lanes,
                                      grid=grid, group=1))
        for chunks in (1, 2, 4, 8):
            if 256 * vec * chunks >= n:
                for grid in (1, 7, 300):
                    plans.append(dict(kernel=xt.XTVXY_DENSE_BLOCK_ROWS, vec=vec, chunks=chunks, grid=grid, group=1))
            group = -(-n // (256 * vec * chunks))
            if 1 <= group <= 16:
                for units in (1, 3, 16):
                    plans.append(dict(kernel=xt.XTVXY_DENSE_GROUP_ROWS, vec=vec, chunks=chunks, grid=group * units,
                                      group=group))
    out = []
    for d in plans:
        lp = xt.xtvxy_launch_params(block_threads=256, **d)
        out.append(xt.xtvxy_dense_f32_plan_complete(m, n, n, lp))
    return out


@pytest.mark.parametrize("m,n", [(333, 4), (257, 100), (300, 256), (129, 700), (77, 1500), (45, 3001)])
def test_every_kernel_variant(m, n):
    p = datagen.dense_problem(m, n, seed=11 + n)
    ref, bnd = dense_oracle(p)
    d = DenseOnDevice(p)
    plans = forced_plans(m, n)
    assert plans
    for plan in plans:
        note("forced %s" % plan.as_dict())
        got = d.run(plan=plan)
        assert_parity(got, ref, bnd, "forced %s" % plan.as_dict())


@pytest.mark.parametrize("m,n,ldx", [(50, 100, 103), (50, 100, 104), (40, 1030, 1031), (9, 9000, 9004),
                                     (33, 3, 5)])
def test_padded_leading_dimension(m, n, ldx):
    # padding columns hold NaN: any read of them would poison the result
    check(datagen.dense_problem(m, n, seed=3, ldx=ldx), what="ldx")


@pytest.mark.parametrize("n", [256, 2048, 9000])
def test_unaligned_X(n):
    # X starts 4 bytes past a 16-byte boundary: the model must fall back to 4-byte loads
    p = datagen.dense_problem(70, n, seed=5)
    plan = xt.xtvxy_dense_f32_plan(70, n, n, 0)
    assert plan.vec == 1
    check(p, X_offset=1, what="unaligned")


@pytest.mark.parametrize("m,n", [(2048, 128), (600, 1000), (64, 8192), (16, 20000)])
def test_exact_integers_bitwise(m, n):
    g = np.random.default_rng(m + n)
    X = g.integers(-1, 2, size=(m, n)).astype(np.float32)
    y, v, z = (g.integers(-1, 2, size=s).astype(np.float32) for s in (n, m, n))
    p = datagen.DenseProblem(m, n, n, X.ravel(), y, v, z, 1.5, 0.5, "integers")
    note("exact integers m=%d n=%d" % (m, n))
    got = DenseOnDevice(p).run()
    S = X.astype(np.int64).T @ (v.astype(np.int64) * (X.astype(np.int64) @ y.astype(np.int64)))
    expected = (1.5 * S + 0.5 * z).astype(np.float32)
    assert np.array_equal(got, expected)


@pytest.mark.parametrize("n", [128, 256, 5000, 20000])
def test_v_absent_equals_ones_and_runs_are_reproducible(n):
    p = datagen.dense_problem(500, n, seed=21, v=None)
    d = DenseOnDevice(p)
    note("v absent n=%d" % n)
    a = d.run()
    b = d.run(v=d.y.new_ones(500))
    c = d.run()
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("n", [256, 5000, 20000])
def test_out_aliases_z(n):
    p = datagen.dense_problem(300, n, seed=22)
    d = DenseOnDevice(p)
    note("out == z n=%d" % n)
    separate = d.run()
    zz = d.z.clone()
    d2 = DenseOnDevice(p)
    d2.z = zz
    inplace = d2.run(out=zz)
    assert np.array_equal(separate, inplace)


def test_quick_returns_and_special_scalars():
    import torch
    p = datagen.dense_problem(40, 300, seed=23)
    d = DenseOnDevice(p)
    d.X.view(40, 300)[3, 7] = float("nan")
    note("alpha == 0")
    out = d.run(alpha=0.0, beta=0.5)
    assert np.array_equal(out, (np.float32(0.5) * p.z).astype(np.float32))
    out = d.run(alpha=0.0, beta=0.0)
    assert np.array_equal(out, np.zeros(300, np.float32))
    # beta == 0: z not read even when it holds NaN
    p2 = datagen.dense_problem(40, 300, seed=24)
    d2 = DenseOnDevice(p2)
    ref = d2.run(beta=0.0)
    d2.z = torch.full_like(d2.z, float("nan"))
    out = d2.run(beta=0.0)
    assert np.array_equal(out, ref) and np.all(np.isfinite(out))
    # m == 0 and n == 0
    p3 = datagen.dense_problem(0, 50, seed=25)
    assert np.array_equal(DenseOnDevice(p3).run(), (np.float32(p3.beta) * p3.z).astype(np.float32))
    p4 = datagen.dense_problem(5, 0, seed=26, ldx=1)
    assert DenseOnDevice(p4).run().shape == (0,)


@pytest.mark.parametrize("n", [100, 3000, 10000])
def test_nan_and_inf_propagate_like_the_formula(n):
    p = datagen.dense_problem(64, n, seed=27)
    X = p.X.copy()
    X[5 * n + n // 2] = np.nan
    q = datagen.DenseProblem(64, n, n, X, p.y, p.v, p.z, p.alpha, p.beta)
    note("NaN n=%d" % n)
    assert np.all(np.isnan(DenseOnDevice(q).run()))
    X = p.X.copy()
    X[9 * n + 1] = np.inf
    v = p.v.copy()
    v[9] = 0.0
    q = datagen.DenseProblem(64, n, n, X, p.y, v, p.z, p.alpha, p.beta)
    assert np.all(np.isnan(DenseOnDevice(q).run()))


@pytest.fixture(scope="module")
def full_normal_equations():
    return datagen.WORKLOADS["dense_1000000x256_normal_equations"]()


def test_full_size_normal_equations_1000000x256(full_normal_equations):
    check(full_normal_equations)


def test_full_size_65536x8192():
    check(datagen.WORKLOADS["dense_65536x8192"]())


def test_full_size_8192x65536_column_slices():
    p = datagen.WORKLOADS["dense_8192x65536"]()
    plan = xt.xtvxy_dense_f32_plan(p.m, p.n, p.ldx, 1)
    assert plan.kernel == xt.XTVXY_DENSE_GROUP_ROWS
    check(p)


def test_group_wait_failure_is_visible():
    # The failure path of the group-row kernel's bounded wait, forced from the host: every wait
    # looks for a step tag that no member publishes and gives up after 4 polls, so every kernel
    # still ends normally; the call must then deliver NaN in every element, and the next call with
    # the hook off must be correct again.
    m, n = 96, 20000
    p = datagen.dense_problem(m, n, seed=41)
    ref, bnd = dense_oracle(p)
    d = DenseOnDevice(p)
    plan = xt.xtvxy_dense_f32_plan_complete(m, n, n, xt.xtvxy_launch_params(
        kernel=xt.XTVXY_DENSE_GROUP_ROWS, block_threads=256, vec=4, chunks=8, group=3, grid=12))
    note("group-row wait failure forced, plan %s" % plan.as_dict())
    xt.xtvxy_test_group_wait(4, 1)
    try:
        failed = d.run(plan=plan)
    finally:
        xt.xtvxy_test_group_wait(0, 0)
    assert np.isnan(failed).all()
    note("group-row plan again, hook off")
    assert_parity(d.run(plan=plan), ref, bnd, "after the forced failure")


def test_group_rows_on_two_streams_at_once():
    # Two group-row calls on two streams with nothing ordering them, each grid as large as the
    # device holds: the library runs group-row launches of a device one after another, so every
    # member of each call finds a slot and both results are correct.
    import torch
    m, n = 1024, 40000
    probs = [datagen.dense_problem(m, n, seed=s) for s in (44, 45)]
    refs = [dense_oracle(p) for p in probs]
    ds = [DenseOnDevice(p) for p in probs]
    plan = xt.xtvxy_dense_f32_plan(m, n, n, 1)
    assert plan.kernel == xt.XTVXY_DENSE_GROUP_ROWS
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    note("group rows on two streams, plan %s" % plan.as_dict())
    outs = []
    for _ in range(3):
        for p, d, s in zip(probs, ds, streams):
            outs.append(xt.dense(d.X, d.y, d.v, d.z, p.alpha, p.beta, m=m, n=n, ldx=n, stream=s))
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        ref, bnd = refs[k % 2]
        assert_parity(o.cpu().numpy(), ref, bnd, "stream %d, call %d" % (k % 2, k // 2))


def test_helpers_on_a_non_current_stream():
    # the tensor helpers allocate their workspace (and out) on the current stream and launch on
    # the caller's: the allocations are recorded on that stream, so the caching allocator cannot
    # hand them to other work while the kernels still use them
    import torch
    p = datagen.dense_problem(4000, 3000, seed=42)
    ref, bnd = dense_oracle(p)
    d = DenseOnDevice(p)
    s = torch.cuda.Stream()
    note("dense on a side stream")
    with torch.cuda.stream(torch.cuda.current_stream()):
        outs = [xt.dense(d.X, d.y, d.v, d.z, p.alpha, p.beta, m=p.m, n=p.n, ldx=p.ldx, stream=s) for _ in range(3)]
        junk = [torch.full((1 << 22,), float("nan"), device=d.X.device) for _ in range(8)]  # reuse pressure
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    for o in outs:
        assert_parity(o.cpu().numpy(), ref, bnd, "side stream")


def test_workspace_query_for_widths_only_aligned_X_supports():
    # beyond 262,144 columns only 16-byte loads (an aligned X) give a plan: the workspace query
    # must return that plan's size instead of failing on the unaligned one
    m, n = 16, 300_000
    need = xt.xtvxy_dense_f32_workspace_size(m, n, n)
    assert need == xt.xtvxy_dense_f32_plan(m, n, n, 1).workspace_bytes
    check(datagen.dense_problem(m, n, seed=43), what="aligned-only width")
