"""The C ABI without a GPU: exports, host-side argument checks, and the launch model.

Every call here returns before the library touches the HIP runtime (argument
errors are detected first), or is a pure host computation (plans for a stated
device description). No kernel is launched.
"""
import ctypes
import os
import re

import pytest

import dense_linear_algebra_alpha_amd as xt
from dense_linear_algebra_alpha_amd import _abi, build

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "xtvxy.h")

MI355X = xt.xtvxy_device_info(compute_units=256, lds_bytes=163840, l2_bytes=4 << 20, xcds=8,
                              hbm_bytes_per_s=8.0e12)


@pytest.fixture(scope="module")
def lib():
    if build.sources_newer_than_library():
        build.build()
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xtvxy_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 18
    for name in names:
        assert hasattr(lib, name), name
    # and the binding wraps each of them under the same name
    for name in names:
        assert hasattr(xt, name), name


def test_status_strings(lib):
    assert xt.xtvxy_status_string(0) == "XTVXY_SUCCESS"
    assert xt.xtvxy_status_string(4) == "XTVXY_ERROR_WORKSPACE"
    assert xt.xtvxy_status_string(99) == "XTVXY_UNKNOWN_STATUS"


FAKE = 1 << 40  # an address that is never dereferenced: every call below fails its host checks first


def dense_status(m=8, n=8, alpha=1.0, X=FAKE, ldx=8, v=None, y=FAKE + 4096, beta=0.0, z=None, out=FAKE + 8192,
                 ws=None, ws_bytes=0, fn="xtvxy_dense_f32"):
    return getattr(_abi.load(), fn)(m, n, alpha, X, ldx, v, y, beta, z, out, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["xtvxy_dense_f32", "xtvxy_dense_f32_unfused_reference"])
def test_dense_argument_errors(lib, fn):
    assert dense_status(m=-1, fn=fn) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert dense_status(n=-2, fn=fn) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert dense_status(ldx=7, fn=fn) == _abi.XTVXY_ERROR_INVALID_VALUE          # ldx < n
    assert dense_status(n=0, ldx=0, fn=fn) == _abi.XTVXY_ERROR_INVALID_VALUE     # ldx < 1
    assert dense_status(m=1 << 60, ldx=1 << 10, fn=fn) == _abi.XTVXY_ERROR_INVALID_VALUE  # bytes overflow
    assert dense_status(y=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert dense_status(out=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert dense_status(X=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert dense_status(beta=0.5, z=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    # out overlapping X, y, v, or z (other than out == z) is rejected
    assert dense_status(out=FAKE + 16, fn=fn) == _abi.XTVXY_ERROR_ALIASING
    assert dense_status(out=FAKE + 4096 + 4, fn=fn) == _abi.XTVXY_ERROR_ALIASING
    assert dense_status(v=FAKE + 8192 + 8, fn=fn) == _abi.XTVXY_ERROR_ALIASING
    assert dense_status(beta=1.0, z=FAKE + 8192 + 4, fn=fn) == _abi.XTVXY_ERROR_ALIASING
    # n == 0 is a successful no-op that touches nothing
    assert dense_status(n=0, ldx=1, fn=fn) == _abi.XTVXY_SUCCESS


def test_dense_explicit_comparator_argument_errors(lib):
    def explicit(m=8, n=8, X=FAKE, ldx=8, Xt=FAKE + (1 << 20), ldxt=8, y=FAKE + 4096, out=FAKE + 8192, ws=None, wsb=0):
        return lib.xtvxy_dense_f32_unfused_reference_explicit(m, n, 1.0, X, ldx, Xt, ldxt, None, y, 0.0, None, out, ws,
                                                              wsb, None)
    assert explicit(m=-1) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert explicit(ldx=7) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert explicit(ldxt=7) == _abi.XTVXY_ERROR_INVALID_VALUE      # ldxt < m
    assert explicit(Xt=None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert explicit(X=None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert explicit(out=FAKE + (1 << 20) + 64) == _abi.XTVXY_ERROR_ALIASING  # out inside Xt
    assert explicit(out=FAKE + 16) == _abi.XTVXY_ERROR_ALIASING             # out inside X
    assert explicit() == _abi.XTVXY_ERROR_WORKSPACE                          # no workspace for t
    assert explicit(n=0, ldx=1) == _abi.XTVXY_SUCCESS
    tr = lib.xtvxy_dense_f32_transpose
    assert tr(-1, 8, FAKE, 8, FAKE + (1 << 20), 8, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert tr(8, 8, FAKE, 7, FAKE + (1 << 20), 8, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert tr(8, 8, FAKE, 8, FAKE + (1 << 20), 7, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert tr(8, 8, None, 8, FAKE + (1 << 20), 8, None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert tr(8, 8, FAKE, 8, FAKE + 128, 8, None) == _abi.XTVXY_ERROR_ALIASING
    assert tr(0, 8, None, 8, None, 1, None) == _abi.XTVXY_SUCCESS
    assert tr(1 << 32, 8, FAKE, 8, FAKE + (1 << 20), 1 << 32, None) == _abi.XTVXY_ERROR_UNSUPPORTED


def csr_status(m=8, n=8, nnz=16, alpha=1.0, rp=FAKE, ci=FAKE + 1024, vals=FAKE + 2048, v=None, y=FAKE + 4096,
               beta=0.0, z=None, out=FAKE + 8192, fn="xtvxy_csr_f32"):
    return getattr(_abi.load(), fn)(m, n, nnz, alpha, rp, ci, vals, v, y, beta, z, out, None, 0, None)


@pytest.mark.parametrize("fn", ["xtvxy_csr_f32", "xtvxy_csr_bf16"])
def test_csr_argument_errors(lib, fn):
    assert csr_status(m=-1, fn=fn) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert csr_status(nnz=-1, fn=fn) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert csr_status(nnz=1 << 31, fn=fn) == _abi.XTVXY_ERROR_UNSUPPORTED
    assert csr_status(m=1 << 31, fn=fn) == _abi.XTVXY_ERROR_UNSUPPORTED
    assert csr_status(rp=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert csr_status(ci=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert csr_status(vals=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert csr_status(y=None, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert csr_status(beta=2.0, fn=fn) == _abi.XTVXY_ERROR_NULL_POINTER
    assert csr_status(out=FAKE + 1024 + 60, fn=fn) == _abi.XTVXY_ERROR_ALIASING        # overlaps col_idx
    assert csr_status(out=FAKE + 4, fn=fn) == _abi.XTVXY_ERROR_ALIASING                # overlaps row_ptr
    assert csr_status(out=FAKE + 2048 + 28, fn=fn) == _abi.XTVXY_ERROR_ALIASING        # overlaps values
    assert csr_status(n=0, fn=fn) == _abi.XTVXY_SUCCESS
    st = lib.xtvxy_csr_check(4, 4, 4, None, FAKE, FAKE, None)
    assert st == _abi.XTVXY_ERROR_NULL_POINTER


def test_csr_bf16_values_span_two_bytes_each(lib):
    # 16 values end 64 bytes after their start as fp32 but 32 bytes after it as bf16: an out that
    # starts 40 bytes in overlaps the fp32 values only (the bf16 call then fails later, with no GPU)
    assert csr_status(out=FAKE + 2048 + 40) == _abi.XTVXY_ERROR_ALIASING
    assert csr_status(out=FAKE + 2048 + 40, fn="xtvxy_csr_bf16") != _abi.XTVXY_ERROR_ALIASING


def test_query_argument_errors(lib):
    b = ctypes.c_size_t()
    assert lib.xtvxy_dense_f32_workspace_size(4, 8, 4, ctypes.byref(b)) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert lib.xtvxy_dense_f32_workspace_size(4, 8, 8, None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert lib.xtvxy_csr_f32_workspace_size(-1, 8, 8, ctypes.byref(b)) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert lib.xtvxy_dense_f32_unfused_reference_workspace_size(100, 8, ctypes.byref(b)) == 0
    assert b.value >= 400 and b.value % 256 == 0
    assert lib.xtvxy_csr_f32_unfused_plan_create(4, 4, 4, None, FAKE, FAKE, None, None) == \
        _abi.XTVXY_ERROR_NULL_POINTER
    h = ctypes.c_void_p()
    assert lib.xtvxy_csr_f32_unfused_plan_create_ex(4, 4, 4, FAKE, FAKE, FAKE, 7, None, ctypes.byref(h)) == \
        _abi.XTVXY_ERROR_INVALID_VALUE
    assert lib.xtvxy_csr_f32_unfused_plan_create_ex(4, 4, 4, None, FAKE, FAKE, 1, None, ctypes.byref(h)) == \
        _abi.XTVXY_ERROR_NULL_POINTER


def test_probe_argument_errors(lib):
    assert lib.xtvxy_read_probe(None, 16, 1, FAKE, None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert lib.xtvxy_read_probe(FAKE, 15, 1, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert lib.xtvxy_read_probe(FAKE + 4, 16, 1, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert lib.xtvxy_read_probe(FAKE, 16, 0, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    tp = lib.xtvxy_tile_stream_probe
    assert tp(None, FAKE, 2048, 1, 0, FAKE, None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert tp(FAKE, FAKE, 2047, 1, 0, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE   # not whole tiles
    assert tp(FAKE, FAKE, 4096, 3, 0, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE   # not a multiple of grid
    assert tp(FAKE + 4, FAKE, 2048, 1, 0, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert tp(FAKE, FAKE, 2048, 1, 2, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert tp(FAKE, FAKE, 0, 1, 0, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    probe = lib.xtvxy_scatter_probe
    assert probe(_abi.XTVXY_PROBE_GATHERS, None, 64, 16, 8, 0, 1, FAKE, None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert probe(_abi.XTVXY_PROBE_GATHERS, FAKE, 64, 16, 8, 0, 1, None, None) == _abi.XTVXY_ERROR_NULL_POINTER
    for kind in (-1, 4):
        assert probe(kind, FAKE, 1 << 20, 16, 8, 0, 1, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert probe(_abi.XTVXY_PROBE_GATHERS, FAKE, 64, 0, 8, 0, 1, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert probe(_abi.XTVXY_PROBE_GATHERS, FAKE, 64, 16, 8, 2, 1, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert probe(_abi.XTVXY_PROBE_GATHERS, FAKE, 64, 16, 8, 0, 0, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert probe(_abi.XTVXY_PROBE_GATHERS, FAKE + 4, 64, 16, 8, 0, 1, FAKE, None) == _abi.XTVXY_ERROR_INVALID_VALUE
    # the buffer must cover what the kind indexes: n floats, n 8-byte items, 8 copies of n floats
    assert probe(_abi.XTVXY_PROBE_GATHERS, FAKE, 63, 16, 8, 0, 1, FAKE, None) == _abi.XTVXY_ERROR_WORKSPACE
    assert probe(_abi.XTVXY_PROBE_ATOMIC_DEVICE, FAKE, 63, 16, 8, 0, 1, FAKE, None) == _abi.XTVXY_ERROR_WORKSPACE
    assert probe(_abi.XTVXY_PROBE_ITEM_STORES, FAKE, 127, 16, 8, 0, 1, FAKE, None) == _abi.XTVXY_ERROR_WORKSPACE
    assert probe(_abi.XTVXY_PROBE_ATOMIC_PER_XCD, FAKE, 511, 16, 8, 0, 1, FAKE, None) == \
        _abi.XTVXY_ERROR_WORKSPACE
    # no updates: nothing to launch
    assert probe(_abi.XTVXY_PROBE_ATOMIC_PER_XCD, FAKE, 512, 16, 0, 1, 1, FAKE, None) == _abi.XTVXY_SUCCESS


SHAPES = [(2048, 128), (1_000_000, 256), (65_536, 8192), (8192, 65_536), (1, 1), (7, 3), (100, 1000),
          (5, 1025), (3, 8193), (1000, 200_000)]


@pytest.mark.parametrize("m,n", SHAPES)
@pytest.mark.parametrize("aligned", [1, 0])
def test_dense_model_plans_cover_the_problem(lib, m, n, aligned):
    p = xt.xtvxy_dense_f32_plan(m, n, n, aligned, MI355X)
    assert p.block_threads == 256 and p.grid >= 1
    assert p.vec == (4 if aligned and n % 4 == 0 else 1)
    if p.kernel == xt.XTVXY_DENSE_WAVE_ROWS:
        assert p.lanes_per_row * p.vec * p.chunks >= n and p.lanes_per_row <= 64 and p.group == 1
        units = p.grid
    elif p.kernel == xt.XTVXY_DENSE_BLOCK_ROWS:
        assert 256 * p.vec * p.chunks >= n and p.group == 1
        units = p.grid
    else:
        assert p.kernel == xt.XTVXY_DENSE_GROUP_ROWS
        assert p.group * 256 * p.vec * p.chunks >= n and p.grid % p.group == 0
        units = p.grid // p.group
    assert p.rows_per_unit * units >= m and (p.rows_per_unit - 1) * units < m + p.rows_per_unit
    assert p.workspace_bytes >= units * n * 4 and p.workspace_bytes % 256 == 0
    assert p.predicted_seconds > 0


def test_dense_model_picks_the_row_layout_by_width(lib):
    assert xt.xtvxy_dense_f32_plan(2048, 128, 128, 1, MI355X).kernel == xt.XTVXY_DENSE_WAVE_ROWS
    assert xt.xtvxy_dense_f32_plan(2048, 128, 128, 1, MI355X).lanes_per_row == 32
    assert xt.xtvxy_dense_f32_plan(10**6, 256, 256, 1, MI355X).lanes_per_row == 64
    assert xt.xtvxy_dense_f32_plan(65536, 8192, 8192, 1, MI355X).kernel == xt.XTVXY_DENSE_BLOCK_ROWS
    p = xt.xtvxy_dense_f32_plan(8192, 65536, 65536, 1, MI355X)
    assert p.kernel == xt.XTVXY_DENSE_GROUP_ROWS and p.group == 8
    # the model's estimate is close to the bandwidth bound on the big shapes
    p = xt.xtvxy_dense_f32_plan(10**6, 256, 256, 1, MI355X)
    assert 1.024e9 / 8.0e12 < p.predicted_seconds < 1.024e9 / 8.0e12 / 0.8


def test_plan_complete_rejects_plans_that_do_not_cover(lib):
    p = xt.xtvxy_dense_f32_plan(1000, 256, 256, 1, MI355X)
    q = xt.xtvxy_launch_params.from_buffer_copy(p)
    q.lanes_per_row = 16  # 16 lanes * 4 * 1 = 64 columns < 256
    with pytest.raises(xt.XtvxyError):
        xt.xtvxy_dense_f32_plan_complete(1000, 256, 256, q, MI355X)
    q = xt.xtvxy_launch_params.from_buffer_copy(p)
    q.lanes_per_row = 48  # not a power of two
    with pytest.raises(xt.XtvxyError):
        xt.xtvxy_dense_f32_plan_complete(1000, 256, 256, q, MI355X)
    q = xt.xtvxy_launch_params.from_buffer_copy(p)
    q.grid, q.rows_per_unit = 64, 0
    xt.xtvxy_dense_f32_plan_complete(1000, 256, 256, q, MI355X)
    assert q.rows_per_unit == 16 and q.workspace_bytes == 64 * 256 * 4


@pytest.mark.parametrize("m,n,nnz", [(10_000_000, 1000, 100_000_000), (5_000_000, 1_000_000, 200_000_000),
                                     (1_000_000, 1000, 100_000_000), (100_000, 8192, 20_000_000),
                                     (10, 5, 7), (1, 1, 1)])
def test_csr_model_plans(lib, m, n, nnz):
    p = xt.xtvxy_csr_f32_plan(m, n, nnz, MI355X)
    # narrow matrices of at most 128 entries per row on average take the wavefront kernel, the
    # rest workgroup tiles
    waves = n * 8 <= 64 * 1024 and nnz <= 128 * m
    assert p.kernel == (xt.XTVXY_CSR_WAVES if waves else xt.XTVXY_CSR_TILES)
    assert p.grid >= 1 and p.entries_per_thread in (4, 8, 16)
    assert 0 < p.lds_window <= n and p.workspace_bytes >= p.grid * p.lds_window * 4
    lds = (p.lds_window + p.y_window) * 4
    assert lds <= 64 * 1024
    if p.lds_window < n and p.bin_columns == 0:
        assert p.workspace_bytes >= p.grid * p.lds_window * 4 + n * 4
    if p.bin_columns:
        # binned: two workgroups per CU still fit, and the pool holds every stored entry
        bins = -(-(n - p.lds_window) // p.bin_columns)
        assert bins <= 512 and p.bin_columns & (p.bin_columns - 1) == 0
        assert p.kernel == xt.XTVXY_CSR_TILES
        static = 29 * p.block_threads + 256 + 4 * p.block_threads * p.entries_per_thread
        assert (2048 // p.block_threads) // 2 * (lds + bins * 32 + static) <= MI355X.lds_bytes
        assert p.workspace_bytes >= nnz * 8


def test_csr_wave_plans(lib):
    """The wavefront kernel: 256, 512 or 1024 threads of 8 entries; its LDS (windows, 512 bytes of
    marks and 256 of u per wavefront, a word per thread, 24 bytes per bin and wavefront) must fit;
    its bin pool leaves room for one partly filled chunk per (wavefront, bin)."""
    def lp(blk, window, y_window, bc, grid=64, ept=8):
        return xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_WAVES, block_threads=blk, entries_per_thread=ept, grid=grid,
                                      vec=1, chunks=1, group=1, lds_window=window, y_window=y_window, bin_columns=bc)
    for blk in (256, 512, 1024):
        q = xt.xtvxy_csr_f32_plan_complete(1000, 900, 9000, lp(blk, 900, 900, 0), MI355X)
        assert q.kernel == xt.XTVXY_CSR_WAVES and q.workspace_bytes == 64 * 900 * 4
    for blk, ept in ((128, 8), (256, 4), (2048, 8)):
        with pytest.raises(xt.XtvxyError):
            xt.xtvxy_csr_f32_plan_complete(1000, 900, 9000, lp(blk, 900, 900, 0, ept=ept), MI355X)
    # the largest window that fits beside the 1024-thread workgroup's static LDS (16 KiB)
    static = 16 * (512 + 256) + 4 * 1024
    w = (MI355X.lds_bytes - static) // 4
    xt.xtvxy_csr_f32_plan_complete(1000, 10**6, 10**6, lp(1024, w, 0, 0), MI355X)
    with pytest.raises(xt.XtvxyError):
        xt.xtvxy_csr_f32_plan_complete(1000, 10**6, 10**6, lp(1024, w + 2, 0, 0), MI355X)
    # binned: 60 bins of 16384 columns, 24 bytes per bin and wavefront
    n, w = 1_000_000, 20000
    bins = -(-(n - w) // 16384)
    q = xt.xtvxy_csr_f32_plan_complete(5_000_000, n, 2 * 10**8, lp(1024, w, 0, 16384, grid=256), MI355X)
    chunks = -(-2 * 10**8 // 512) + 256 * 16 * bins
    assert q.workspace_bytes >= chunks * 512 * 8
    with pytest.raises(xt.XtvxyError):  # the bin state of 16 wavefronts no longer fits
        xt.xtvxy_csr_f32_plan_complete(5_000_000, n, 2 * 10**8,
                                       lp(1024, (MI355X.lds_bytes - static - 16 * 24 * bins) // 4 + 2, 0, 16384),
                                       MI355X)


def test_csr_plan_rows(lib):
    """Three workgroups per CU for the wavefront kernel when every row fits its 512-slot tiles and
    rows hold 8 or more entries on average; the model's plan otherwise."""
    base = xt.xtvxy_csr_f32_plan(10_000_000, 1000, 100_000_000, MI355X)
    assert base.kernel == xt.XTVXY_CSR_WAVES and base.grid == 4 * 256
    p = xt.xtvxy_csr_f32_plan_rows(10_000_000, 1000, 100_000_000, 40, MI355X)
    assert p.kernel == xt.XTVXY_CSR_WAVES and p.grid == 3 * 256 and p.workspace_bytes == 768 * 1000 * 4
    assert xt.xtvxy_csr_f32_plan_rows(10_000_000, 1000, 100_000_000, 509, MI355X).grid == 768
    for m, n, nnz, longest in ((10_000_000, 1000, 100_000_000, 510),  # a row longer than a tile
                               (10_000_000, 1000, 50_000_000, 40),    # 5 entries per row
                               (5_000_000, 1_000_000, 200_000_000, 2726)):  # wide: workgroup tiles
        q = xt.xtvxy_csr_f32_plan_rows(m, n, nnz, longest, MI355X)
        r = xt.xtvxy_csr_f32_plan(m, n, nnz, MI355X)
        assert (q.kernel, q.grid, q.lds_window, q.y_window, q.bin_columns) == (r.kernel, r.grid, r.lds_window,
                                                                               r.y_window, r.bin_columns)
    for longest in (-1, 100_000_001):
        with pytest.raises(xt.XtvxyError):
            xt.xtvxy_csr_f32_plan_rows(10_000_000, 1000, 100_000_000, longest, MI355X)


def test_csr_model_bins_the_wide_zipf_matrix_and_not_the_narrow_one(lib):
    assert xt.xtvxy_csr_f32_plan(5_000_000, 1_000_000, 200_000_000, MI355X).bin_columns == 16384
    assert xt.xtvxy_csr_f32_plan(10_000_000, 1000, 100_000_000, MI355X).bin_columns == 0


def test_csr_plan_complete_checks_the_bins(lib):
    def lp(window, bc):
        return xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_TILES, block_threads=256, entries_per_thread=8, grid=64,
                                      vec=1, chunks=1, group=1, lds_window=window, y_window=0, bin_columns=bc)
    n = 1000 + 512 * 1024
    q = xt.xtvxy_csr_f32_plan_complete(1000, n, 10**6, lp(1000, 1024), MI355X)  # exactly 512 bins
    assert q.workspace_bytes >= 10**6 * 8
    for bad in (lp(999, 1024), lp(1000, 1000), lp(1000, 512), lp(1000, 65536)):
        with pytest.raises(xt.XtvxyError):
            xt.xtvxy_csr_f32_plan_complete(1000, n, 10**6, bad, MI355X)
    # a window that covers every column needs no bins
    q = xt.xtvxy_csr_f32_plan_complete(1000, 500, 10**4, lp(500, 1024), MI355X)
    assert q.bin_columns == 0 and q.workspace_bytes == 64 * 500 * 4


def test_struct_layouts_match_the_header(tmp_path):
    # sizeof / offsetof of every ABI struct as a C compiler lays them out, against the ctypes mirrors
    structs = {"xtvxy_device_info": xt.xtvxy_device_info, "xtvxy_launch_params": xt.xtvxy_launch_params,
               "xtvxy_logreg_options": xt.xtvxy_logreg_options, "xtvxy_logreg_report": xt.xtvxy_logreg_report,
               "xtvxy_tune_report": xt.xtvxy_tune_report}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "xtvxy.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append('  printf("%s %%zu\\n", sizeof(%s));' % (cname, cname))
        for field, _ in cls._fields_:
            cfield = "lambda" if field == "lambda_" else field
            lines.append('  printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, field, cname, cfield))
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.dirname(HEADER), "-I/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for field, _ in cls._fields_:
            assert int(got["%s.%s" % (cname, field)]) == getattr(cls, field).offset, (cname, field)


def logreg_status(m=8, n=4, nnz=16, rp=FAKE, ci=FAKE + 1024, vals=FAKE + 2048, labels=FAKE + 4096, w=FAKE + 8192,
                  opt=None, plan=None, ws=FAKE + 65536, ws_bytes=1 << 20, history=None, rows=0, **kw):
    o = xt.xtvxy_logreg_options(1.0, 5, 10, 30, 1e-6, 0.5, 0, xt.XTVXY_LOGREG_FUSED)
    for k, v in kw.items():
        setattr(o, k, v)
    return _abi.load().xtvxy_logreg_newton_cg_f32(m, n, nnz, rp, ci, vals, labels, w,
                                                  ctypes.byref(o) if opt is None else opt, plan, ws, ws_bytes,
                                                  None, None, history, rows)


def test_logreg_argument_errors(lib):
    E = _abi
    assert logreg_status(m=-1) == E.XTVXY_ERROR_INVALID_VALUE
    assert logreg_status(rows=-1) == E.XTVXY_ERROR_INVALID_VALUE
    assert logreg_status(nnz=1 << 31) == E.XTVXY_ERROR_UNSUPPORTED
    assert lib.xtvxy_logreg_newton_cg_f32(8, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1, None, None,
                                          None, 0) == E.XTVXY_ERROR_NULL_POINTER  # no options
    for field, bad in (("lambda_", -1.0), ("lambda_", float("inf")), ("lambda_", float("nan")), ("max_newton", -1),
                       ("max_cg", 0), ("max_backtracks", 0), ("grad_tol", -1e-3), ("grad_tol", float("nan")),
                       ("cg_forcing", 0.0), ("cg_forcing", 1.5), ("engine", 2)):
        assert logreg_status(**{field: bad}) == E.XTVXY_ERROR_INVALID_VALUE, field
    assert logreg_status(rp=None) == E.XTVXY_ERROR_NULL_POINTER
    assert logreg_status(ci=None) == E.XTVXY_ERROR_NULL_POINTER
    assert logreg_status(labels=None) == E.XTVXY_ERROR_NULL_POINTER
    assert logreg_status(w=None) == E.XTVXY_ERROR_NULL_POINTER
    assert logreg_status(rows=3) == E.XTVXY_ERROR_NULL_POINTER                  # history rows without history
    assert logreg_status(engine=xt.XTVXY_LOGREG_UNFUSED) == E.XTVXY_ERROR_NULL_POINTER  # no comparator plan
    assert logreg_status(ws=None) == E.XTVXY_ERROR_WORKSPACE
    assert logreg_status(ws=FAKE + 65536 + 64) == E.XTVXY_ERROR_WORKSPACE     # not 256-byte aligned
    b = ctypes.c_size_t()
    assert lib.xtvxy_logreg_newton_cg_f32_workspace_size(-1, 4, 4, ctypes.byref(b)) == E.XTVXY_ERROR_INVALID_VALUE
    assert lib.xtvxy_logreg_newton_cg_f32_workspace_size(4, 4, 4, None) == E.XTVXY_ERROR_NULL_POINTER


def logreg_bf16_status(m=8, n=4, nnz=16, vals=FAKE + 2048, ws=FAKE + 65536, **kw):
    o = xt.xtvxy_logreg_options(1.0, 5, 10, 30, 1e-6, 0.5, 0, xt.XTVXY_LOGREG_FUSED)
    for k, v in kw.items():
        setattr(o, k, v)
    return _abi.load().xtvxy_logreg_newton_cg_bf16(m, n, nnz, FAKE, FAKE + 1024, vals, FAKE + 4096, FAKE + 8192,
                                                   ctypes.byref(o), ws, 1 << 20, None, None, None, 0)


def test_logreg_bf16_argument_errors(lib):
    E = _abi
    assert logreg_bf16_status(engine=xt.XTVXY_LOGREG_UNFUSED) == E.XTVXY_ERROR_INVALID_VALUE  # fused engine only
    assert logreg_bf16_status(m=-1) == E.XTVXY_ERROR_INVALID_VALUE
    assert logreg_bf16_status(max_cg=0) == E.XTVXY_ERROR_INVALID_VALUE
    assert logreg_bf16_status(vals=None) == E.XTVXY_ERROR_NULL_POINTER
    assert logreg_bf16_status(ws=None) == E.XTVXY_ERROR_WORKSPACE


@pytest.mark.parametrize("fn", ["xtvxy_csr_f32_rowdot", "xtvxy_csr_bf16_rowdot"])
def test_rowdot_argument_errors(lib, fn):
    f = getattr(lib, fn)
    # m n nnz alpha row_ptr col_idx values v y beta t0 t stream
    ok = [8, 8, 16, 1.0, FAKE, FAKE + 1024, FAKE + 2048, None, FAKE + 4096, 0.0, None, FAKE + 8192, None]
    def st(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert st(a0=-1) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert st(a2=1 << 31) == _abi.XTVXY_ERROR_UNSUPPORTED
    assert st(a6=None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert st(a9=1.0) == _abi.XTVXY_ERROR_NULL_POINTER          # beta != 0 without t0
    assert st(a11=FAKE + 2048 + 16) == _abi.XTVXY_ERROR_ALIASING  # t overlaps the values


@pytest.mark.parametrize("fn", ["xtvxy_csr_f32_tmv", "xtvxy_csr_bf16_tmv"])
def test_tmv_argument_errors(lib, fn):
    f = getattr(lib, fn)
    # m n nnz alpha row_ptr col_idx values u beta z out workspace bytes stream
    ok = [8, 8, 16, 1.0, FAKE, FAKE + 1024, FAKE + 2048, FAKE + 4096, 0.0, None, FAKE + 8192, None, 0, None]
    def st(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert st(a1=-1) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert st(a6=None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert st(a7=None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert st(a8=1.0) == _abi.XTVXY_ERROR_NULL_POINTER           # beta != 0 without z
    assert st(a10=FAKE + 2048 + 16) == _abi.XTVXY_ERROR_ALIASING  # out overlaps the values


def test_tune_argument_errors(lib):
    rep = xt.xtvxy_tune_report()
    assert lib.xtvxy_dense_f32_tune(8, 8, 1.0, FAKE, 8, None, FAKE + 4096, 0.0, None, FAKE + 8192, 10, None,
                                    None) == _abi.XTVXY_ERROR_NULL_POINTER
    assert lib.xtvxy_dense_f32_tune(8, 8, 1.0, FAKE, 8, None, FAKE + 4096, 0.0, None, FAKE + 8192, 0, None,
                                    ctypes.byref(rep)) == _abi.XTVXY_ERROR_INVALID_VALUE  # repeats
    assert lib.xtvxy_dense_f32_tune(8, 8, 1.0, FAKE, 7, None, FAKE + 4096, 0.0, None, FAKE + 8192, 5, None,
                                    ctypes.byref(rep)) == _abi.XTVXY_ERROR_INVALID_VALUE  # ldx < n
    # alpha = 0: the call reads no X, nothing to tune
    assert lib.xtvxy_dense_f32_tune(8, 8, 0.0, FAKE, 8, None, FAKE + 4096, 0.0, None, FAKE + 8192, 5, None,
                                    ctypes.byref(rep)) == _abi.XTVXY_ERROR_INVALID_VALUE
    assert lib.xtvxy_csr_f32_tune(8, 8, 16, 1.0, None, FAKE, FAKE, None, FAKE + 4096, 0.0, None, FAKE + 8192, 5,
                                  None, ctypes.byref(rep)) == _abi.XTVXY_ERROR_NULL_POINTER
    assert lib.xtvxy_csr_f32_tune(8, 8, 0, 1.0, FAKE, None, None, None, FAKE + 4096, 0.0, None, FAKE + 8192, 5,
                                  None, ctypes.byref(rep)) == _abi.XTVXY_ERROR_INVALID_VALUE  # nnz = 0
    # the fp16 dense and bf16 CSR tuners check as the others do (bf16 values span 2 bytes each)
    assert lib.xtvxy_dense_f16_tune(8, 8, 1.0, FAKE, 8, None, FAKE + 4096, 0.0, None, FAKE + 8192, 0, None,
                                    ctypes.byref(rep)) == _abi.XTVXY_ERROR_INVALID_VALUE  # repeats
    assert lib.xtvxy_dense_f16_tune(8, 8, 0.0, FAKE, 8, None, FAKE + 4096, 0.0, None, FAKE + 8192, 5, None,
                                    ctypes.byref(rep)) == _abi.XTVXY_ERROR_INVALID_VALUE  # nothing to tune
    assert lib.xtvxy_csr_bf16_tune(8, 8, 16, 1.0, None, FAKE, FAKE, None, FAKE + 4096, 0.0, None, FAKE + 8192, 5,
                                   None, ctypes.byref(rep)) == _abi.XTVXY_ERROR_NULL_POINTER
    assert lib.xtvxy_csr_bf16_tune(8, 8, 16, 1.0, FAKE, FAKE + 1024, FAKE + 2048, None, FAKE + 4096, 0.0, None,
                                   FAKE + 2048 + 28, 5, None, ctypes.byref(rep)) == _abi.XTVXY_ERROR_ALIASING
    found = ctypes.c_int32()
    for kind in (-1, 5):
        assert lib.xtvxy_tune_cache_lookup(kind, 1, 1, 1, 0, ctypes.byref(rep), ctypes.byref(found)) == \
            _abi.XTVXY_ERROR_INVALID_VALUE
    for kind in range(5):  # nothing tuned yet: found = 0
        assert lib.xtvxy_tune_cache_lookup(kind, 1, 1, 1, 0, ctypes.byref(rep), ctypes.byref(found)) in \
            (_abi.XTVXY_SUCCESS, _abi.XTVXY_ERROR_LAUNCH)  # no device here: the key cannot be made


def test_tune_cache_file_round_trip(lib, tmp_path):
    # a hand-written cache line loads, saves back unchanged, and a malformed file changes nothing
    plan = "11 1 256 0 1 1 1024 0 8 1000 1000 0 4096000"
    model = "11 1 256 0 1 1 1024 0 8 1000 1000 0 4096000"
    line = "gfx950:256 1 10000000 1000 100006237 1 %s %s 2.140000000e-04 2.150000000e-04 24" % (plan, model)
    src = tmp_path / "in.txt"
    src.write_text("# comment\n" + line + "\n")
    xt.xtvxy_tune_cache_clear()
    xt.xtvxy_tune_cache_load(str(src))
    out = tmp_path / "out.txt"
    xt.xtvxy_tune_cache_save(str(out))
    body = [l for l in out.read_text().splitlines() if not l.startswith("#")]
    assert body == [line]
    bad = tmp_path / "bad.txt"
    bad.write_text(line + "\n" + "gfx950:256 1 5 5\n")
    with pytest.raises(xt.XtvxyError):
        xt.xtvxy_tune_cache_load(str(bad))
    with pytest.raises(xt.XtvxyError):
        xt.xtvxy_tune_cache_load(str(tmp_path / "missing.txt"))
    xt.xtvxy_tune_cache_clear()
    xt.xtvxy_tune_cache_save(str(out))
    assert [l for l in out.read_text().splitlines() if not l.startswith("#")] == []


def test_bf16_plans_and_checks(lib):
    # model plans for bf16 X: 16-byte loads of 8 elements when aligned; the layout thresholds double
    p = xt.xtvxy_dense_bf16_plan(1000, 256, 256, 1, MI355X)
    assert (p.kernel, p.vec, p.lanes_per_row, p.chunks) == (xt.XTVXY_DENSE_WAVE_ROWS, 8, 32, 1)
    p = xt.xtvxy_dense_bf16_plan(1000, 2048, 2048, 1, MI355X)
    assert (p.kernel, p.vec, p.chunks) == (xt.XTVXY_DENSE_WAVE_ROWS, 8, 4)
    p = xt.xtvxy_dense_bf16_plan(1000, 8192, 8192, 1, MI355X)
    assert (p.kernel, p.vec, p.chunks) == (xt.XTVXY_DENSE_BLOCK_ROWS, 8, 4)
    p = xt.xtvxy_dense_bf16_plan(1000, 65536, 65536, 1, MI355X)
    assert (p.kernel, p.vec, p.group, p.chunks) == (xt.XTVXY_DENSE_GROUP_ROWS, 8, 8, 4)
    assert xt.xtvxy_dense_bf16_plan(1000, 256, 260, 1, MI355X).vec == 1   # ldx % 8 != 0
    assert xt.xtvxy_dense_bf16_plan(1000, 256, 256, 0, MI355X).vec == 1   # X not 16-byte aligned
    # the fp32 model keeps 4-element loads; the bf16 one predicts half the X time
    f = xt.xtvxy_dense_f32_plan(1_000_000, 256, 256, 1, MI355X)
    h = xt.xtvxy_dense_bf16_plan(1_000_000, 256, 256, 1, MI355X)
    assert f.vec == 4 and h.predicted_seconds < 0.6 * f.predicted_seconds
    # forced plans: vec 4 is not a bf16 width, vec 8 needs n % 8 == 0, and 8 chunks of 8 are refused
    bad = [dict(kernel=xt.XTVXY_DENSE_WAVE_ROWS, vec=4, chunks=1, lanes_per_row=64, grid=8, group=1),
           dict(kernel=xt.XTVXY_DENSE_BLOCK_ROWS, vec=8, chunks=8, grid=8, group=1)]
    for d in bad:
        with pytest.raises(xt.XtvxyError):
            xt.xtvxy_dense_bf16_plan_complete(100, 256, 256, xt.xtvxy_launch_params(block_threads=256, **d), MI355X)
    with pytest.raises(xt.XtvxyError):
        xt.xtvxy_dense_bf16_plan_complete(100, 260, 260, xt.xtvxy_launch_params(
            block_threads=256, kernel=xt.XTVXY_DENSE_BLOCK_ROWS, vec=8, chunks=1, grid=8, group=1), MI355X)
    # the aliasing check measures X in 2-byte elements: out just past X's last byte is fine
    st = lib.xtvxy_dense_bf16(8, 8, 1.0, FAKE, 8, None, FAKE + 4096, 0.0, None, FAKE + 126, None, 0, None)
    assert st == _abi.XTVXY_ERROR_ALIASING      # X spans 128 bytes: out at +126 overlaps
    st = lib.xtvxy_dense_bf16(8, 0, 1.0, FAKE, 1, None, FAKE + 4096, 0.0, None, FAKE + 128, None, 0, None)
    assert st == _abi.XTVXY_SUCCESS              # n == 0
