"""GPU parity of the fused CSR path against the fp64 oracle (runs through the C ABI)."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import CsrOnDevice, DenseOnDevice, assert_parity, csr_oracle, dense_oracle, note

pytestmark = pytest.mark.gpu


def check(p, plan=None, what=""):
    note("csr %s m=%d n=%d nnz=%d plan=%s" % (what or p.name, p.m, p.n, p.nnz,
                                             None if plan is None else plan.as_dict()))
    got = CsrOnDevice(p).run(plan=plan)
    ref, bnd = csr_oracle(p)
    return assert_parity(got, ref, bnd, "%s m=%d n=%d" % (what or p.name, p.m, p.n))


@pytest.mark.parametrize("m,n", [(1, 1), (5, 7), (100, 3), (100, 1000), (3000, 64), (3000, 1000), (2500, 20000),
                                 (4000, 70000), (700, 300000)])
@pytest.mark.parametrize("mean_len", [1.0, 6.0, 40.0])
def test_irregular_matrices(m, n, mean_len):
    check(datagen.csr_random(m, n, seed=m + n + int(mean_len), mean_len=mean_len, empty_frac=0.2, dup_frac=0.1),
          what="random")


def forced_plans(m, n, nnz):
    """Output windows from none to all of n, y gathered from global memory, from LDS or split,
    each tile size, a few grids, and the columns outside the window by atomics or in bins."""
    fixed = 32768  # more than the kernel's own LDS for any workgroup and tile size
    windows = sorted({0, min(n, 7), min(n, 4096), n if n * 4 + fixed <= 163840 else min(n, 30000)})
    out = []
    for w in windows:
        for yw in sorted({0, min(n, 300), n}):
            if (w + yw) * 4 + fixed > 163840:
                continue
            for blk, ept in ((256, 4), (256, 8), (512, 8)):
                for grid in (1, 7, 256):
                    # columns outside the window: global atomics, or bins of 1024 columns
                    for bc in ((0, 1024) if w < n else (0,)):
                        lp = xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_TILES, block_threads=blk,
                                                    entries_per_thread=ept, grid=grid, vec=1, chunks=1, group=1,
                                                    lds_window=w, y_window=yw, bin_columns=bc)
                        out.append(xt.xtvxy_csr_f32_plan_complete(m, n, nnz, lp))
    return out


def binned_plan(m, n, nnz, window, bin_columns, grid=64, ept=8, y_window=0, blk=256):
    lp = xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_TILES, block_threads=blk, entries_per_thread=ept, grid=grid,
                                vec=1, chunks=1, group=1, lds_window=window, y_window=y_window,
                                bin_columns=bin_columns)
    return xt.xtvxy_csr_f32_plan_complete(m, n, nnz, lp)


@pytest.mark.parametrize("m,n,mean_len", [(2000, 500, 9.0), (500, 30000, 30.0)])
def test_every_kernel_variant(m, n, mean_len):
    p = datagen.csr_random(m, n, seed=31, mean_len=mean_len, empty_frac=0.1, dup_frac=0.05)
    ref, bnd = csr_oracle(p)
    d = CsrOnDevice(p)
    for plan in forced_plans(m, n, p.nnz):
        note("forced %s" % plan.as_dict())
        assert_parity(d.run(plan=plan), ref, bnd, "forced %s" % plan.as_dict())


@pytest.mark.parametrize("entry_offset", [0, 1, 3])
def test_entry_tails_and_misaligned_arrays(entry_offset):
    """nnz of every residue mod 4 (1 to 9 entries, and a matrix of several tiles), with col_idx and
    values 16-byte aligned or not: the entries after the last whole quad, and the element-wise
    loads of misaligned arrays, under every kernel variant."""
    cases = []
    for nnz in range(1, 10):
        rng = np.random.default_rng(100 + nnz)
        m, n = 3, 11
        rows = np.sort(rng.integers(0, m, nnz))
        rp = np.zeros(m + 1, np.int32)
        rp[1:] = np.cumsum(np.bincount(rows, minlength=m))
        ci = np.concatenate([np.sort(rng.choice(n, int(c), replace=False)) for c in np.diff(rp)]).astype(np.int32)
        vals = rng.uniform(-1, 1, nnz).astype(np.float32)
        y, v, z = (rng.uniform(-1, 1, k).astype(np.float32) for k in (n, m, n))
        cases.append(datagen.CsrProblem(m, n, rp, ci, vals, y, v, z, 0.9, 0.4, "nnz=%d" % nnz))
    p = datagen.csr_random(5000, 3000, seed=77, mean_len=9.0, empty_frac=0.1)
    if p.nnz % 4 == 0:  # keep a ragged last quad
        p = datagen.csr_random(5001, 3000, seed=77, mean_len=9.0, empty_frac=0.1)
    assert p.nnz % 4 != 0
    cases.append(p)
    for q in cases:
        ref, bnd = csr_oracle(q)
        d = CsrOnDevice(q, entry_offset=entry_offset)
        for plan in [None] + forced_plans(q.m, q.n, q.nnz)[::5]:
            note("tails nnz=%d offset=%d plan=%s" % (q.nnz, entry_offset, None if plan is None else plan.as_dict()))
            assert_parity(d.run(plan=plan), ref, bnd, "nnz=%d offset=%d" % (q.nnz, entry_offset))


def test_rows_longer_than_a_tile():
    # rows of 3000..9000 entries (more than one 2048-entry tile) between short and empty rows
    g = np.random.default_rng(5)
    m, n = 64, 12000
    lens = g.integers(0, 5, size=m)
    lens[[3, 17, 40, 63]] = [3000, 9000, 2049, 5000]
    rp = np.zeros(m + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    cols = np.concatenate([np.sort(g.choice(n, size=L, replace=False)) for L in lens]).astype(np.int32)
    p = datagen.CsrProblem(m, n, rp.astype(np.int32), cols, datagen.uniform(int(rp[-1]), 1, "vals"),
                           datagen.uniform(n, 1, "y"), datagen.uniform(m, 1, "v"), datagen.uniform(n, 1, "z"),
                           1.25, -0.5, "long rows")
    check(p)
    for plan in forced_plans(m, n, p.nnz)[::4]:
        check(p, plan=plan, what="long rows forced")


def test_long_runs_of_empty_rows():
    # stretches of empty rows longer than the rows a tile can stage
    m, n = 20000, 300
    g = np.random.default_rng(6)
    lens = np.zeros(m, np.int64)
    lens[::2999] = g.integers(1, 40, size=lens[::2999].size)
    lens[-1] = 0
    rp = np.zeros(m + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    cols = g.integers(0, n, size=int(rp[-1])).astype(np.int32)
    p = datagen.CsrProblem(m, n, rp.astype(np.int32), cols, datagen.uniform(int(rp[-1]), 2, "vals"),
                           datagen.uniform(n, 2, "y"), datagen.uniform(m, 2, "v"), None, 2.0, 0.0, "sparse rows")
    check(p)
    for plan in forced_plans(m, n, p.nnz)[::3]:
        check(p, plan=plan, what="sparse rows forced")


@pytest.mark.parametrize("n", [50, 900, 40000])
def test_csr_agrees_with_dense_on_the_same_matrix(n):
    m = 300
    p = datagen.dense_problem(m, n, seed=41)
    X = p.X2d().copy()
    X[np.random.default_rng(1).random((m, n)) < 0.9] = 0.0
    rp, ci, vals = datagen.csr_from_dense(X)
    q = datagen.CsrProblem(m, n, rp, ci, vals, p.y, p.v, p.z, p.alpha, p.beta, "from dense")
    pd = datagen.DenseProblem(m, n, n, X.ravel().copy(), p.y, p.v, p.z, p.alpha, p.beta, "dense twin")
    note("csr vs dense n=%d" % n)
    got_csr = CsrOnDevice(q).run()
    got_dense = DenseOnDevice(pd).run()
    ref, bnd = dense_oracle(pd)
    assert_parity(got_csr, ref, bnd, "csr")
    assert_parity(got_dense, ref, bnd, "dense")


def test_exact_integers_bitwise():
    g = np.random.default_rng(3)
    m, n = 5000, 700
    X = (g.integers(-1, 2, size=(m, n)) * (g.random((m, n)) < 0.05)).astype(np.float32)
    rp, ci, vals = datagen.csr_from_dense(X)
    y, v, z = (g.integers(-1, 2, size=s).astype(np.float32) for s in (n, m, n))
    p = datagen.CsrProblem(m, n, rp, ci, vals, y, v, z, 1.5, 0.5, "integers")
    note("csr exact integers")
    got = CsrOnDevice(p).run()
    S = X.astype(np.int64).T @ (v.astype(np.int64) * (X.astype(np.int64) @ y.astype(np.int64)))
    assert np.array_equal(got, (1.5 * S + 0.5 * z).astype(np.float32))


def test_special_cases():
    import torch
    p = datagen.csr_random(200, 50, seed=7)
    d = CsrOnDevice(p)
    note("csr alpha == 0")
    assert np.array_equal(d.run(alpha=0.0, beta=0.5), (np.float32(0.5) * p.z).astype(np.float32))
    # beta == 0: z is not read even when it holds NaN (CSR sums are atomic-ordered, so compare
    # with the oracle to the tolerance rather than bitwise with another run)
    d.z = torch.full_like(d.z, float("nan"))
    out = d.run(beta=0.0)
    q0 = datagen.CsrProblem(p.m, p.n, p.row_ptr, p.col_idx, p.values, p.y, p.v, None, p.alpha, 0.0)
    ref, bnd = csr_oracle(q0)
    assert np.all(np.isfinite(out))
    assert_parity(out, ref, bnd, "beta == 0")
    empty = datagen.CsrProblem(4, 50, np.zeros(5, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32),
                               p.y, np.ones(4, np.float32), p.z, 1.0, -2.0, "no entries")
    assert np.array_equal(CsrOnDevice(empty).run(), (np.float32(-2.0) * p.z).astype(np.float32))
    # NaN in one stored entry reaches exactly the columns of its row
    X = np.zeros((10, 8), np.float32)
    X[2, 1], X[2, 5], X[3, 0], X[3, 5], X[7, 2] = 1.0, 2.0, -1.0, 0.5, 3.0
    rp, ci, vals = datagen.csr_from_dense(X)
    vals[0] = np.nan
    q = datagen.CsrProblem(10, 8, rp, ci, vals, p.y[:8].copy(), np.ones(10, np.float32), p.z[:8].copy(), 1.0, 1.0)
    out = CsrOnDevice(q).run()
    assert set(np.nonzero(np.isnan(out))[0].tolist()) == {1, 5}


def test_structure_check():
    import torch
    p = datagen.csr_random(100, 20, seed=8)
    d = CsrOnDevice(p)
    note("csr_check")
    assert xt.csr_check(d.rp, d.ci, 20) == 0
    bad = d.ci.clone()
    bad[3] = 20
    assert xt.csr_check(d.rp, bad, 20) == 3
    rp = d.rp.clone()
    a, b = int(rp[10].item()), int(rp[11].item())
    rp[10], rp[11] = b + 1, a  # row_ptr decreases from position 10 to 11
    assert xt.csr_check(rp, d.ci, 20) >= 2
    rp = d.rp.clone()
    rp[-1] -= 1
    assert xt.csr_check(rp, d.ci, 20) >= 1


def test_logistic_hvp_scaled():
    check(datagen.WORKLOADS["csr_10000000x1000_logistic_hvp"](m=300_000))


def test_zipf_scaled():
    check(datagen.WORKLOADS["csr_5000000x1000000_zipf"](m=100_000, n=200_000))


def test_zipf_permuted_columns_scaled():
    check(datagen.WORKLOADS["csr_5000000x1000000_zipf"](m=100_000, n=200_000, permute_columns=True),
          what="zipf permuted")


def test_full_size_logistic_hvp_10000000x1000():
    check(datagen.WORKLOADS["csr_10000000x1000_logistic_hvp"]())


def test_full_size_zipf_5000000x1000000():
    check(datagen.WORKLOADS["csr_5000000x1000000_zipf"]())


def test_repeated_calls_reuse_a_workspace():
    import torch
    p = datagen.csr_random(5000, 900, seed=9, mean_len=12.0)
    d = CsrOnDevice(p)
    ws = torch.empty(xt.xtvxy_csr_f32_workspace_size(p.m, p.n, p.nnz), dtype=torch.uint8, device="cuda")
    ref, bnd = csr_oracle(p)
    note("csr workspace reuse")
    for _ in range(3):
        out = xt.csr(d.rp, d.ci, d.vals, p.n, d.y, d.v, d.z, p.alpha, p.beta, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), ref, bnd, "reuse")


def test_binned_many_bins_spills_and_long_rows():
    # 293 bins of 1024 columns; most entries fall in a few bins, so a tile hands a bin more
    # items than one 512-item chunk holds; some rows are longer than a tile (binned in slices)
    g = np.random.default_rng(12)
    m, n = 3000, 300000
    lens = g.integers(0, 30, size=m)
    lens[[10, 500, 2999]] = [5000, 2100, 9000]
    rp = np.zeros(m + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    hot = g.random(int(rp[-1])) < 0.7
    cols = np.where(hot, g.integers(2048, 4096, size=hot.size), g.integers(0, n, size=hot.size))
    row_of = np.repeat(np.arange(m), lens)
    cols = cols[np.lexsort((cols, row_of))]  # sorted within rows (repeats allowed: each one counts)
    p = datagen.CsrProblem(m, n, rp.astype(np.int32), cols.astype(np.int32), datagen.uniform(int(rp[-1]), 12, "vals"),
                           datagen.uniform(n, 12, "y"), datagen.uniform(m, 12, "v"), datagen.uniform(n, 12, "z"),
                           0.75, 0.5, "binned spills")
    for window, bc, grid, ept, yw, blk in [(0, 1024, 64, 8, 0, 256), (1000, 1024, 7, 4, 3000, 256),
                                           (100, 2048, 256, 8, 0, 512), (16000, 32768, 1, 8, 16000, 256),
                                           (9000, 16384, 5, 8, 3000, 512)]:
        check(p, plan=binned_plan(m, n, p.nnz, window, bc, grid, ept, yw, blk),
              what="binned w=%d bc=%d yw=%d blk=%d" % (window, bc, yw, blk))


def test_binned_workspace_reuse_and_shrinking_input():
    import torch
    p = datagen.WORKLOADS["csr_5000000x1000000_zipf"](m=20_000, n=100_000)
    plan = binned_plan(p.m, p.n, p.nnz, 2000, 4096, grid=128)
    ws = torch.full((plan.workspace_bytes,), 255, dtype=torch.uint8, device="cuda")  # dirty workspace
    d = CsrOnDevice(p)
    ref, bnd = csr_oracle(p)
    note("csr binned workspace reuse")
    for _ in range(2):
        out = xt.csr(d.rp, d.ci, d.vals, p.n, d.y, d.v, d.z, p.alpha, p.beta, plan=plan, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), ref, bnd, "binned reuse")
    # then a smaller matrix in the same workspace
    q = datagen.csr_random(3000, 100_000, seed=13, mean_len=20.0)
    plan_q = binned_plan(q.m, q.n, q.nnz, 2000, 4096, grid=128)
    assert plan_q.workspace_bytes <= ws.numel()
    dq = CsrOnDevice(q)
    out = xt.csr(dq.rp, dq.ci, dq.vals, q.n, dq.y, dq.v, dq.z, q.alpha, q.beta, plan=plan_q, workspace=ws)
    torch.cuda.synchronize()
    ref_q, bnd_q = csr_oracle(q)
    assert_parity(out.cpu().numpy(), ref_q, bnd_q, "binned smaller")


def test_torch_sparse_csr_tensor_input():
    # the convenience wrapper over torch.sparse_csr_tensor passes the tensor's own arrays
    import torch
    p = datagen.csr_random(3000, 700, seed=77, mean_len=9.0, empty_frac=0.1, dup_frac=0.05)
    ref, bnd = csr_oracle(p)
    X = torch.sparse_csr_tensor(torch.from_numpy(p.row_ptr).cuda(), torch.from_numpy(p.col_idx).cuda(),
                                torch.from_numpy(p.values).cuda(), size=(p.m, p.n))
    d = CsrOnDevice(p)
    note("csr from torch.sparse_csr_tensor m=%d n=%d nnz=%d" % (p.m, p.n, p.nnz))
    got = xt.csr_tensor(X, d.y, d.v, d.z, p.alpha, p.beta)
    torch.cuda.synchronize()
    assert_parity(got.cpu().numpy(), ref, bnd, "sparse_csr_tensor")
    with pytest.raises(ValueError):
        xt.csr_tensor(X.to_dense(), d.y)
    X64 = torch.sparse_csr_tensor(torch.from_numpy(p.row_ptr.astype(np.int64)).cuda(),
                                  torch.from_numpy(p.col_idx.astype(np.int64)).cuda(),
                                  torch.from_numpy(p.values).cuda(), size=(p.m, p.n))
    with pytest.raises(ValueError):
        xt.csr_tensor(X64, d.y)
