"""The synthetic workload generators: determinism and the distributions they promise (no GPU)."""
import numpy as np

import datagen


def test_deterministic_and_thread_independent(monkeypatch):
    a = datagen.csr_zipf(2000, 5000, seed=3, alpha=0.7, beta=0.3)
    b = datagen.csr_zipf(2000, 5000, seed=3, alpha=0.7, beta=0.3)
    for k in ("row_ptr", "col_idx", "values", "y", "v", "z"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    c = datagen.csr_zipf(2000, 5000, seed=4)
    assert not np.array_equal(a.values[:100], c.values[:100])
    d1 = datagen.dense_problem(300, 40, seed=1, x="normal")
    d2 = datagen.dense_problem(300, 40, seed=1, x="normal")
    assert np.array_equal(d1.X, d2.X)


def test_uniform_and_normal_moments():
    u = datagen.uniform(1_000_000, 0, "u")
    assert u.min() >= -1 and u.max() < 1 and abs(u.mean()) < 3e-3 and abs(u.var() - 1 / 3) < 3e-3
    assert np.all(u * 2 ** 23 == np.round(u * 2 ** 23))        # 24-bit grid, exact in fp32
    g = datagen.normal(1_000_000, 0, "g")
    assert abs(g.mean()) < 5e-3 and abs(g.std() - 1) < 5e-3
    assert abs(np.mean(g ** 4) - 3) < 0.05                         # Gaussian kurtosis


def test_bernoulli_density_and_structure():
    m, n, p = 200_000, 1000, 0.01
    c = datagen.csr_bernoulli(m, n, p, seed=0)
    total = m * n
    sigma = np.sqrt(total * p * (1 - p))
    assert abs(c.nnz - total * p) < 4 * sigma
    rl = np.diff(c.row_ptr)
    # row lengths ~ Binomial(1000, 0.01): mean 10, variance 9.9, P(empty) = 0.99^1000
    assert abs(rl.mean() - 10) < 0.05 and abs(rl.var() - 9.9) < 0.3
    assert abs((rl == 0).mean() - 0.99 ** 1000) < 4 * np.sqrt(0.99 ** 1000 / m)
    # columns sorted and distinct within rows, in range, spread uniformly
    rows = np.repeat(np.arange(m), rl)
    key = rows.astype(np.int64) * n + c.col_idx
    assert np.all(np.diff(key) > 0)
    counts = np.bincount(c.col_idx, minlength=n)
    assert counts.std() < 4 * np.sqrt(c.nnz / n)
    # v = p(1 - p) lies in (0, 1/4]
    assert c.v.min() > 0 and c.v.max() <= 0.25


def test_zipf_rows_and_columns():
    m, n = 200_000, 1_000_000
    c = datagen.csr_zipf(m, n, seed=0)
    rl = np.diff(c.row_ptr)
    # truncated Zipf(1.5) on 1..2726: mean 40.003
    k = np.arange(1, 2727, dtype=np.float64)
    pk = k ** -1.5 / np.sum(k ** -1.5)
    mean = float(np.sum(k * pk))
    sd = float(np.sqrt(np.sum(k * k * pk) - mean ** 2))
    assert abs(mean - 40.003) < 1e-3
    assert abs(rl.mean() - mean) < 4 * sd / np.sqrt(m)
    assert rl.min() >= 1 and rl.max() <= 2726
    assert abs((rl == 1).mean() - pk[0]) < 4 * np.sqrt(pk[0] / m)
    # columns distinct and sorted within each row
    rows = np.repeat(np.arange(m), rl)
    key = rows.astype(np.int64) * n + c.col_idx
    assert np.all(np.diff(key) > 0)
    # column popularity decays like rank^-1.2 in the tail where rows rarely saturate
    counts = np.bincount(c.col_idx, minlength=n).astype(np.float64)
    r = np.arange(1000, 100_000)
    slope = np.polyfit(np.log(r + 1.0), np.log(counts[r] + 0.5), 1)[0]
    assert abs(slope + 1.2) < 0.08, slope


def test_zipf_permuted_columns_keep_the_structure():
    a = datagen.csr_zipf(5000, 20000, seed=2)
    b = datagen.csr_zipf(5000, 20000, seed=2, permute_columns=True)
    assert np.array_equal(a.row_ptr, b.row_ptr)
    assert a.col_idx.sum() != b.col_idx.sum()
    ca = np.sort(np.bincount(a.col_idx, minlength=20000))
    cb = np.sort(np.bincount(b.col_idx, minlength=20000))
    assert np.array_equal(ca, cb)          # same popularity profile, relabelled columns


def test_dense_padding_is_nan():
    p = datagen.dense_problem(4, 3, seed=0, ldx=5)
    X = p.X.reshape(4, 5)
    assert np.all(np.isnan(X[:, 3:])) and np.all(np.isfinite(X[:, :3]))


def test_logistic_bf16_workload_rounds_the_values_only():
    P = datagen.LOGISTIC_WORKLOADS["logreg_csr_10000000x1000"](m=20_000)
    B = datagen.LOGISTIC_WORKLOADS["logreg_csr_10000000x1000_bf16"](m=20_000)
    assert B.X.values_dtype == "bf16" and B.X.values.dtype == np.uint16
    assert np.array_equal(B.labels, P.labels) and B.lam == P.lam
    assert np.array_equal(B.X.row_ptr, P.X.row_ptr) and np.array_equal(B.X.col_idx, P.X.col_idx)
    assert np.array_equal(B.X.values, datagen.to_bf16(P.X.values))
    # rounding to nearest bf16: within half a unit of the last of 8 significant bits
    assert np.all(np.abs(B.X.values_f32() - P.X.values) <= np.abs(P.X.values) * 2.0 ** -8)


def test_logistic_labels():
    P = datagen.LOGISTIC_WORKLOADS["logreg_csr_10000000x1000"](m=200_000)
    Q = datagen.LOGISTIC_WORKLOADS["logreg_csr_10000000x1000"](m=200_000)
    assert np.array_equal(P.labels, Q.labels) and P.lam == 1.0
    assert set(np.unique(P.labels)) <= {0.0, 1.0}
    # the planted w ~ N(0, 0.01) is symmetric, so P(c = 1) = 1/2; rows whose curvature weight
    # v = p(1 - p) is lowest have |p - 1/2| largest, and their labels follow the sign of p - 1/2
    m = P.X.m
    assert abs(P.labels.mean() - 0.5) < 4 * np.sqrt(0.25 / m)
    w = datagen.normal(P.X.n, 0, "w", 0.0, 0.1).astype(np.float64)
    rows = np.repeat(np.arange(m), np.diff(P.X.row_ptr))
    eta = np.bincount(rows, weights=P.X.values.astype(np.float64) * w[P.X.col_idx], minlength=m)
    p = 1.0 / (1.0 + np.exp(-eta))
    assert np.allclose(P.X.v, p * (1 - p), rtol=1e-6, atol=0)
    # calibration: among rows with p in a bin, the label frequency matches the bin's mean p
    for lo, hi in ((0.3, 0.45), (0.55, 0.7)):
        sel = (p >= lo) & (p < hi)
        k = int(sel.sum())
        assert k > 1000 and abs(P.labels[sel].mean() - p[sel].mean()) < 4 * np.sqrt(0.25 / k)


def test_bf16_rounding():
    # ties go to the even neighbour; other values to the nearest; bf16 values round-trip exactly
    f = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -(1.0 + 2.0 ** -8),
                  np.finfo(np.float32).max, np.inf, -0.0], dtype=np.float32)
    h = datagen.to_bf16(f)
    assert list(h) == [0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x7F80, 0x7F80, 0x8000], [hex(x) for x in h]
    g = datagen.bf16_to_f32(np.arange(0, 0x7F80, 7, dtype=np.uint16))
    assert np.array_equal(datagen.to_bf16(g), np.arange(0, 0x7F80, 7, dtype=np.uint16))
    n = datagen.to_bf16(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all(np.isnan(datagen.bf16_to_f32(n)))
    p = datagen.dense_problem(20, 8, seed=3, x_dtype="bf16", ldx=9)
    q = datagen.dense_problem(20, 8, seed=3, ldx=9)
    assert p.X.dtype == np.uint16 and np.array_equal(p.X, datagen.to_bf16(q.X))


def test_f16_storage_rounds_to_nearest_even_and_widens_exactly():
    # the generator rounds the fp32 draw to IEEE fp16 once; the bit patterns below are fixed by the
    # binary16 format: signed zeros, the smallest and largest subnormals, the smallest normal, 1,
    # -2, the largest finite value and the infinities
    bits = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0xC000, 0x7BFF, 0x7C00, 0xFC00], np.uint16)
    want = np.array([0.0, -0.0, 2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14, 1.0, -2.0, 65504.0, np.inf, -np.inf],
                    np.float32)
    p = datagen.DenseProblem(1, 10, 10, bits.view(np.float16), np.zeros(10, np.float32), None, None, 1.0, 0.0,
                             "f16 patterns", "f16")
    got = p.X_f32()
    assert got.dtype == np.float32 and np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    # ties to even: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10, 1 + 3 * 2^-11 between 1 + 2^-10 and 1 + 2^-9
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -12], np.float32)
    assert np.array_equal(x.astype(np.float16).astype(np.float32),
                          np.array([1.0, 1 + 2.0 ** -9, 1.0], np.float32))
    q = datagen.dense_problem(20, 8, seed=3, x_dtype="f16", ldx=9)
    r = datagen.dense_problem(20, 8, seed=3, x_dtype="f32", ldx=9)
    assert q.X.dtype == np.float16
    assert np.array_equal(q.X2d().astype(np.float32), r.X2d().astype(np.float16).astype(np.float32))
