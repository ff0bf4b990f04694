"""GPU parity of the CSR path with bf16 values (xtvxy_csr_bf16*, through the C ABI) against the fp64
oracle on the values the bf16 bit patterns denote (widened exactly by numpy): the tile and wavefront
kernels under every layout, tails and misaligned arrays, exact integers bitwise, analysed calls, and
the two full-size CSR workloads."""
import numpy as np
import pytest

import datagen
import dense_linear_algebra_alpha_amd as xt
from gpu_util import CsrOnDevice, assert_parity, csr_oracle, note
from test_gpu_csr import forced_plans
from test_gpu_csr_waves import wave_plans

pytestmark = pytest.mark.gpu


def bf16(p, name=""):
    return datagen.csr_values_bf16(p, name or (p.name or "csr") + " bf16")


def check(p, plan=None, what="", entry_offset=0):
    note("csr bf16 %s m=%d n=%d nnz=%d offset=%d plan=%s" % (what or p.name, p.m, p.n, p.nnz, entry_offset,
                                                           None if plan is None else plan.as_dict()))
    got = CsrOnDevice(p, entry_offset=entry_offset).run(plan=plan)
    ref, bnd = csr_oracle(p)
    return assert_parity(got, ref, bnd, "%s m=%d n=%d" % (what or p.name, p.m, p.n))


def test_values_are_bf16_bit_patterns():
    p = bf16(datagen.csr_random(300, 50, seed=1, mean_len=5.0))
    d = CsrOnDevice(p)
    import torch
    assert d.vals.dtype == torch.bfloat16 and p.values.dtype == np.uint16


@pytest.mark.parametrize("m,n", [(1, 1), (5, 7), (100, 1000), (3000, 64), (2500, 20000), (700, 300000)])
@pytest.mark.parametrize("mean_len", [1.0, 6.0, 40.0])
def test_irregular_matrices(m, n, mean_len):
    check(bf16(datagen.csr_random(m, n, seed=m + n + int(mean_len), mean_len=mean_len, empty_frac=0.2,
                                  dup_frac=0.1)), what="random")


@pytest.mark.parametrize("m,n,mean_len", [(2000, 500, 9.0), (500, 30000, 30.0)])
def test_every_tile_variant(m, n, mean_len):
    p = bf16(datagen.csr_random(m, n, seed=31, mean_len=mean_len, empty_frac=0.1, dup_frac=0.05))
    ref, bnd = csr_oracle(p)
    d = CsrOnDevice(p)
    for plan in forced_plans(m, n, p.nnz):
        note("bf16 tiles forced %s" % plan.as_dict())
        assert_parity(d.run(plan=plan), ref, bnd, "bf16 tiles forced %s" % plan.as_dict())


@pytest.mark.parametrize("m,n,mean_len", [(3000, 700, 12.0), (400, 30000, 60.0)])
def test_every_wavefront_variant(m, n, mean_len):
    p = bf16(datagen.csr_random(m, n, seed=32, mean_len=mean_len, empty_frac=0.1, dup_frac=0.05))
    ref, bnd = csr_oracle(p)
    d = CsrOnDevice(p)
    plans = wave_plans(m, n, p.nnz)
    for blk in (256, 512):  # the smaller workgroups too (the model's choice for narrow matrices)
        lp = xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_WAVES, block_threads=blk, entries_per_thread=8, grid=96,
                                    vec=1, chunks=1, group=1, lds_window=min(n, 4096), y_window=min(n, 4096))
        plans.append(xt.xtvxy_csr_f32_plan_complete(m, n, p.nnz, lp))
    for plan in plans:
        note("bf16 waves forced %s" % plan.as_dict())
        assert_parity(d.run(plan=plan), ref, bnd, "bf16 waves forced %s" % plan.as_dict())


@pytest.mark.parametrize("entry_offset", [0, 1, 2, 3, 4])
def test_entry_tails_and_misaligned_values(entry_offset):
    """nnz of every residue mod 4, with col_idx and values shifted by 0-4 elements: offsets 0 and 4
    keep the vector loads (values 8-byte, col_idx 16-byte aligned), 1-3 take the element loads."""
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
        cases.append(bf16(datagen.CsrProblem(m, n, rp, ci, vals, y, v, z, 0.9, 0.4, "nnz=%d" % nnz)))
    p = datagen.csr_random(5001, 3000, seed=77, mean_len=9.0, empty_frac=0.1)
    assert p.nnz % 4 != 0
    cases.append(bf16(p))
    for q in cases:
        ref, bnd = csr_oracle(q)
        d = CsrOnDevice(q, entry_offset=entry_offset)
        plans = [None] + forced_plans(q.m, q.n, q.nnz)[::7] + wave_plans(q.m, q.n, q.nnz)[::9]
        for plan in plans:
            note("bf16 tails nnz=%d offset=%d plan=%s" % (q.nnz, entry_offset,
                                                         None if plan is None else plan.as_dict()))
            assert_parity(d.run(plan=plan), ref, bnd, "bf16 nnz=%d offset=%d" % (q.nnz, entry_offset))


def test_exact_integers_bitwise():
    # small integers are exact in bf16, and every partial sum is an integer below 2^24: the result
    # is the integer formula, bit for bit, under every kernel and layout
    g = np.random.default_rng(14)
    m, n = 5000, 700
    X = (g.integers(-3, 4, size=(m, n)) * (g.random((m, n)) < 0.05)).astype(np.float32)
    rp, ci, vals = datagen.csr_from_dense(X)
    y, v, z = (g.integers(-1, 2, size=s).astype(np.float32) for s in (n, m, n))
    p = bf16(datagen.CsrProblem(m, n, rp, ci, vals, y, v, z, 1.5, 0.5, "integers"))
    assert np.array_equal(p.values_f32(), vals)
    S = X.astype(np.int64).T @ (v.astype(np.int64) * (X.astype(np.int64) @ y.astype(np.int64)))
    want = (1.5 * S + 0.5 * z).astype(np.float32)
    d = CsrOnDevice(p)
    plans = [None] + forced_plans(m, n, p.nnz)[::6] + wave_plans(m, n, p.nnz)[::6]
    for plan in plans:
        note("bf16 exact integers %s" % (None if plan is None else plan.as_dict()))
        assert np.array_equal(d.run(plan=plan), want)


def test_special_scalars_and_nan():
    p = bf16(datagen.csr_random(2000, 900, seed=5, mean_len=8.0))
    d = CsrOnDevice(p)
    ref, bnd = csr_oracle(p)
    note("bf16 out == z, alpha 0, beta 0")
    out = d.z.clone()
    got = xt.csr(d.rp, d.ci, d.vals, p.n, d.y, d.v, out, p.alpha, p.beta, out=out)
    import torch
    torch.cuda.synchronize()
    assert_parity(got.cpu().numpy(), ref, bnd, "out == z")
    zero = xt.csr(d.rp, d.ci, d.vals, p.n, d.y, d.v, d.z, 0.0, 2.0)
    torch.cuda.synchronize()
    assert np.array_equal(zero.cpu().numpy(), (np.float32(2.0) * p.z).astype(np.float32))
    # a NaN value reaches exactly the columns its row shares
    q = bf16(datagen.csr_random(300, 200, seed=6, mean_len=4.0, empty_frac=0.0))
    q.values = q.values.copy()
    q.values[0] = 0x7FC0  # bf16 NaN
    got = CsrOnDevice(q).run()
    ref, _ = csr_oracle(q)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).any()


def test_analysed_calls():
    import torch
    for permute in (False, True):
        p = bf16(datagen.WORKLOADS["csr_5000000x1000000_zipf"](m=100_000, n=200_000, permute_columns=permute))
        ref, bnd = csr_oracle(p)
        d = CsrOnDevice(p)
        an = xt.CsrAnalysis(d.rp, d.ci, p.n)
        note("bf16 analysed zipf permute=%s plan=%s" % (permute, an.plan().as_dict()))
        got = an(d.vals, d.y, d.v, d.z, p.alpha, p.beta)
        torch.cuda.synchronize()
        assert_parity(got.cpu().numpy(), ref, bnd, "bf16 analysed permute=%s" % permute)
        for kernel, blk in ((xt.XTVXY_CSR_TILES, 256), (xt.XTVXY_CSR_WAVES, 512)):
            lp = xt.xtvxy_launch_params(kernel=kernel, block_threads=blk, entries_per_thread=8, grid=200, vec=1,
                                        chunks=1, group=1, lds_window=4096, y_window=1024, bin_columns=16384)
            plan = an.complete(lp)
            note("bf16 analysed forced %s" % plan.as_dict())
            got = an(d.vals, d.y, d.v, d.z, p.alpha, p.beta, plan=plan)
            torch.cuda.synchronize()
            assert_parity(got.cpu().numpy(), ref, bnd, "bf16 analysed forced %s" % plan.as_dict())
        # the row-class kernel takes fp32 values only
        lp = xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_ROWS, block_threads=256, entries_per_thread=8, grid=200,
                                    vec=1, chunks=1, group=1, lds_window=4096, y_window=1024, bin_columns=16384)
        plan = an.complete(lp)
        with pytest.raises(xt.XtvxyError):
            an(d.vals, d.y, d.v, d.z, p.alpha, p.beta, plan=plan)
        an.close()


def test_matches_fp32_on_the_widened_values():
    # the same call on fp32 values equal to the widened bf16 ones: both within the bar of the same
    # oracle, and close to each other (only the order of fp32 additions may differ)
    p = bf16(datagen.csr_random(20000, 5000, seed=9, mean_len=20.0))
    q = datagen.CsrProblem(p.m, p.n, p.row_ptr, p.col_idx, p.values_f32(), p.y, p.v, p.z, p.alpha, p.beta, "f32")
    ref, bnd = csr_oracle(p)
    note("bf16 against fp32 on the widened values")
    a = CsrOnDevice(p).run()
    b = CsrOnDevice(q).run()
    assert_parity(a, ref, bnd, "bf16")
    assert_parity(b, ref, bnd, "fp32 widened")


def test_torch_sparse_csr_tensor_with_bf16_values():
    import torch
    p = bf16(datagen.csr_random(3000, 700, seed=78, mean_len=9.0, empty_frac=0.1, dup_frac=0.05))
    ref, bnd = csr_oracle(p)
    d = CsrOnDevice(p)
    X = torch.sparse_csr_tensor(d.rp, d.ci, d.vals, size=(p.m, p.n))
    assert X.values().dtype == torch.bfloat16
    note("bf16 csr from torch.sparse_csr_tensor m=%d n=%d nnz=%d" % (p.m, p.n, p.nnz))
    got = xt.csr_tensor(X, d.y, d.v, d.z, p.alpha, p.beta)
    torch.cuda.synchronize()
    assert_parity(got.cpu().numpy(), ref, bnd, "bf16 sparse_csr_tensor")


@pytest.mark.parametrize("name", ["csr_10000000x1000_logistic_hvp_bf16", "csr_5000000x1000000_zipf_bf16"])
def test_full_size(name):
    import torch
    p = datagen.WORKLOADS[name]()
    ref, bnd = csr_oracle(p)
    d = CsrOnDevice(p)
    note("bf16 full size %s plain" % name)
    assert_parity(d.run(), ref, bnd, name)
    an = xt.CsrAnalysis(d.rp, d.ci, p.n)
    note("bf16 full size %s analysed plan=%s" % (name, an.plan().as_dict()))
    got = an(d.vals, d.y, d.v, d.z, p.alpha, p.beta)
    torch.cuda.synchronize()
    assert_parity(got.cpu().numpy(), ref, bnd, name + " analysed")
    an.close()
