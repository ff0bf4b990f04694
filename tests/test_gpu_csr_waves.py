"""GPU parity of the wavefront CSR kernel (plan kernel XTVXY_CSR_WAVES) against the fp64 oracle,
through the C ABI with forced plans: irregular rows, rows longer than a wavefront's tile,
stretches of empty rows, ragged entry tails and misaligned arrays, every window and cold mode."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import CsrOnDevice, assert_parity, csr_oracle, note

pytestmark = pytest.mark.gpu

LDS = 163840


def wave_plan(m, n, nnz, blk=1024, grid=64, window=0, y_window=0, bin_columns=0):
    lp = xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_WAVES, block_threads=blk, entries_per_thread=8, grid=grid,
                                vec=1, chunks=1, group=1, lds_window=window, y_window=y_window,
                                bin_columns=bin_columns)
    return xt.xtvxy_csr_f32_plan_complete(m, n, nnz, lp)


def wave_plans(m, n, nnz):
    """Output windows from none to all of n, y from global memory, LDS or split, both workgroup
    sizes, a few grids, and the columns outside the window by atomics or in bins of 1024."""
    out = []
    for w in sorted({0, min(n, 7), min(n, 4096), min(n, 20000)}):
        for yw in sorted({0, min(n, 300), min(n, 8000)}):
            if (w + yw) * 4 + 60000 > LDS:
                continue
            for blk in (512, 1024):
                for grid in (1, 7, 256):
                    for bc in ((0, 1024) if w < n else (0,)):
                        bins = -(-(n - w) // bc) if bc else 0
                        if bins > 512:
                            continue
                        out.append(wave_plan(m, n, nnz, blk, grid, w, yw, bc))
    return out


def check(p, plan, what=""):
    note("csr waves %s m=%d n=%d nnz=%d plan=%s" % (what or p.name, p.m, p.n, p.nnz, plan.as_dict()))
    got = CsrOnDevice(p).run(plan=plan)
    ref, bnd = csr_oracle(p)
    return assert_parity(got, ref, bnd, "%s m=%d n=%d" % (what or p.name, p.m, p.n))


@pytest.mark.parametrize("m,n,mean_len", [(1, 1, 1.0), (100, 3, 6.0), (3000, 1000, 9.0), (500, 30000, 30.0),
                                          (2500, 20000, 40.0), (4000, 70000, 6.0)])
def test_every_variant(m, n, mean_len):
    p = datagen.csr_random(m, n, seed=m + n, mean_len=mean_len, empty_frac=0.2, dup_frac=0.1)
    ref, bnd = csr_oracle(p)
    d = CsrOnDevice(p)
    for plan in wave_plans(m, n, p.nnz):
        note("waves forced m=%d n=%d %s" % (m, n, plan.as_dict()))
        assert_parity(d.run(plan=plan), ref, bnd, "waves forced %s" % plan.as_dict())


@pytest.mark.parametrize("entry_offset", [0, 1, 3])
def test_entry_tails_and_misaligned_arrays(entry_offset):
    cases = []
    for nnz in range(1, 10):
        rng = np.random.default_rng(200 + nnz)
        m, n = 3, 11
        rows = np.sort(rng.integers(0, m, nnz))
        rp = np.zeros(m + 1, np.int32)
        rp[1:] = np.cumsum(np.bincount(rows, minlength=m))
        ci = np.concatenate([np.sort(rng.choice(n, int(c), replace=False)) for c in np.diff(rp)]).astype(np.int32)
        vals = rng.uniform(-1, 1, nnz).astype(np.float32)
        y, v, z = (rng.uniform(-1, 1, k).astype(np.float32) for k in (n, m, n))
        cases.append(datagen.CsrProblem(m, n, rp, ci, vals, y, v, z, 0.9, 0.4, "nnz=%d" % nnz))
    p = datagen.csr_random(5001, 3000, seed=78, mean_len=9.0, empty_frac=0.1)
    if p.nnz % 4 == 0:
        p = datagen.csr_random(5002, 3000, seed=78, mean_len=9.0, empty_frac=0.1)
    assert p.nnz % 4 != 0
    cases.append(p)
    for q in cases:
        ref, bnd = csr_oracle(q)
        d = CsrOnDevice(q, entry_offset=entry_offset)
        for plan in wave_plans(q.m, q.n, q.nnz)[::5]:
            note("waves tails nnz=%d offset=%d plan=%s" % (q.nnz, entry_offset, plan.as_dict()))
            assert_parity(d.run(plan=plan), ref, bnd, "nnz=%d offset=%d" % (q.nnz, entry_offset))


def test_rows_longer_than_a_tile():
    # rows of 510..9000 entries (a wavefront's tile holds 512 slots) between short and empty rows
    g = np.random.default_rng(15)
    m, n = 200, 12000
    lens = g.integers(0, 5, size=m)
    lens[[3, 17, 40, 63, 64, 65, 120, 199]] = [3000, 9000, 509, 510, 511, 512, 513, 5000]
    rp = np.zeros(m + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    cols = np.concatenate([np.sort(g.choice(n, size=L, replace=False)) for L in lens]).astype(np.int32)
    p = datagen.CsrProblem(m, n, rp.astype(np.int32), cols, datagen.uniform(int(rp[-1]), 3, "vals"),
                           datagen.uniform(n, 3, "y"), datagen.uniform(m, 3, "v"), datagen.uniform(n, 3, "z"),
                           1.25, -0.5, "long rows")
    for plan in wave_plans(m, n, p.nnz)[::3]:
        check(p, plan, what="waves long rows")


def test_long_runs_of_empty_rows():
    m, n = 20000, 300
    g = np.random.default_rng(16)
    lens = np.zeros(m, np.int64)
    lens[::2999] = g.integers(1, 40, size=lens[::2999].size)
    lens[-1] = 0
    rp = np.zeros(m + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    cols = g.integers(0, n, size=int(rp[-1])).astype(np.int32)
    p = datagen.CsrProblem(m, n, rp.astype(np.int32), cols, datagen.uniform(int(rp[-1]), 4, "vals"),
                           datagen.uniform(n, 4, "y"), datagen.uniform(m, 4, "v"), None, 2.0, 0.0, "sparse rows")
    for plan in wave_plans(m, n, p.nnz)[::3]:
        check(p, plan, what="waves sparse rows")


def test_exact_integers_bitwise():
    g = np.random.default_rng(13)
    m, n = 5000, 700
    X = (g.integers(-1, 2, size=(m, n)) * (g.random((m, n)) < 0.05)).astype(np.float32)
    rp, ci, vals = datagen.csr_from_dense(X)
    y, v, z = (g.integers(-1, 2, size=s).astype(np.float32) for s in (n, m, n))
    p = datagen.CsrProblem(m, n, rp, ci, vals, y, v, z, 1.5, 0.5, "integers")
    S = X.astype(np.int64).T @ (v.astype(np.int64) * (X.astype(np.int64) @ y.astype(np.int64)))
    want = (1.5 * S + 0.5 * z).astype(np.float32)
    d = CsrOnDevice(p)
    for plan in (wave_plan(m, n, p.nnz, 1024, 256, n, n), wave_plan(m, n, p.nnz, 512, 64, 100, 0, 1024),
                 wave_plan(m, n, p.nnz, 1024, 7, 0, 300, 0)):
        note("waves exact integers %s" % plan.as_dict())
        assert np.array_equal(d.run(plan=plan), want)


def test_binned_spills_and_long_rows():
    # most entries fall in a few bins, so a wavefront's tile hands a bin more items than a chunk
    # holds; rows longer than a tile are binned in slices
    g = np.random.default_rng(22)
    m, n = 3000, 300000
    lens = g.integers(0, 30, size=m)
    lens[[10, 500, 2999]] = [5000, 2100, 9000]
    rp = np.zeros(m + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    hot = g.random(int(rp[-1])) < 0.7
    cols = np.where(hot, g.integers(2048, 4096, size=hot.size), g.integers(0, n, size=hot.size))
    row_of = np.repeat(np.arange(m), lens)
    cols = cols[np.lexsort((cols, row_of))]
    p = datagen.CsrProblem(m, n, rp.astype(np.int32), cols.astype(np.int32), datagen.uniform(int(rp[-1]), 22, "vals"),
                           datagen.uniform(n, 22, "y"), datagen.uniform(m, 22, "v"), datagen.uniform(n, 22, "z"),
                           0.75, 0.5, "binned spills")
    for window, bc, grid, yw, blk in [(0, 1024, 64, 0, 1024), (1000, 1024, 7, 3000, 512), (100, 2048, 256, 0, 512),
                                      (16000, 32768, 1, 8000, 1024), (9000, 16384, 5, 3000, 1024)]:
        check(p, wave_plan(m, n, p.nnz, blk, grid, window, yw, bc), what="waves binned w=%d bc=%d" % (window, bc))


def test_zipf_scaled():
    p = datagen.WORKLOADS["csr_5000000x1000000_zipf"](m=100_000, n=200_000)
    for plan in (wave_plan(p.m, p.n, p.nnz, 1024, 256, 28000, 0, 16384),
                 wave_plan(p.m, p.n, p.nnz, 512, 512, 12000, 2000, 16384)):
        check(p, plan, what="waves zipf")


def test_full_size_zipf_5000000x1000000():
    p = datagen.WORKLOADS["csr_5000000x1000000_zipf"]()
    check(p, wave_plan(p.m, p.n, p.nnz, 1024, 256, 28000, 0, 16384), what="waves zipf full")


@pytest.mark.parametrize("m,n,mean_len,longest", [(200_000, 1000, 10.0, None), (100_000, 4000, 40.0, None),
                                                  (150_000, 2000, 12.0, 600)])
def test_plan_from_the_longest_row(m, n, mean_len, longest):
    # xtvxy_csr_f32_plan_rows: three workgroups per CU when every row fits a tile and rows hold 8 or
    # more entries on average (the first two matrices), the model's plan when a row is longer than
    # a tile (the third, with one row made 600 entries long)
    p = datagen.csr_random(m, n, seed=m + n + 7, mean_len=mean_len, empty_frac=0.05, dup_frac=0.05)
    if longest:
        rl = np.diff(p.row_ptr).astype(np.int64)
        rl[m // 2] = longest
        rp = np.zeros(m + 1, dtype=np.int64)
        np.cumsum(rl, out=rp[1:])
        g = np.random.default_rng(3)
        cols = g.integers(0, n, size=int(rp[-1])).astype(np.int32)
        vals = g.uniform(-1, 1, size=int(rp[-1])).astype(np.float32)
        p = datagen.CsrProblem(m, n, rp.astype(np.int32), cols, vals, p.y, p.v, p.z, p.alpha, p.beta, "long row")
    lr = int(np.diff(p.row_ptr).max())
    plan = xt.xtvxy_csr_f32_plan_rows(p.m, p.n, p.nnz, lr)
    model = xt.xtvxy_csr_f32_plan(p.m, p.n, p.nnz)
    cus = xt.xtvxy_get_device_info().compute_units
    assert plan.kernel == xt.XTVXY_CSR_WAVES
    if lr + 3 <= 512 and p.nnz >= 8 * p.m and model.grid > 3 * cus:
        assert plan.grid == 3 * cus
    else:
        assert plan.grid == model.grid
    check(p, plan, "plan from the longest row (%d)" % lr)
