"""The measurement probes on the GPU: every update of the scatter probe lands (exact integer counts
in fp32), per XCD copy or in one copy, and the gathers, the streaming read and the tile-stream read
write nothing."""
import pytest

import dense_linear_algebra_alpha_amd as xt
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [xt.XTVXY_PROBE_ATOMIC_PER_XCD, xt.XTVXY_PROBE_ATOMIC_DEVICE])
@pytest.mark.parametrize("skew", [0, 1])
def test_scatter_probe_atomics_count_every_update(kind, skew):
    import torch
    n, items = 4096, 1_000_003
    note("scatter probe kind=%d skew=%d n=%d items=%d" % (kind, skew, n, items))
    copies = 8 if kind == xt.XTVXY_PROBE_ATOMIC_PER_XCD else 1
    buf = torch.zeros(copies * n, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    xt.xtvxy_scatter_probe(kind, buf.data_ptr(), buf.numel() * 4, n, items, skew, 512, sink.data_ptr(), None)
    torch.cuda.synchronize()
    per_column = buf.view(copies, n).sum(0).double()
    assert float(per_column.sum()) == items
    assert bool((per_column == per_column.round()).all())
    if skew:  # a quarter of the updates on the first 1.6% of the columns
        assert float(per_column[: int(0.016 * n) + 1].sum()) >= 0.24 * items
    else:
        assert float(per_column.max()) < 2 * items / n


def test_scatter_probe_stores_and_gathers():
    import torch
    n, items = 1 << 16, 1 << 20
    note("scatter probe stores and gathers n=%d items=%d" % (n, items))
    pool = torch.full((2 * n,), -1, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    xt.xtvxy_scatter_probe(xt.XTVXY_PROBE_ITEM_STORES, pool.data_ptr(), pool.numel() * 4, n, items, 0, 256,
                           sink.data_ptr(), None)
    y = torch.zeros(n, dtype=torch.float32, device="cuda")
    xt.xtvxy_scatter_probe(xt.XTVXY_PROBE_GATHERS, y.data_ptr(), n * 4, n, items, 1, 256, sink.data_ptr(), None)
    big = torch.zeros(1 << 22, dtype=torch.float32, device="cuda")
    xt.xtvxy_read_probe(big.data_ptr(), big.numel() * 4, 1024, sink.data_ptr(), None)
    torch.cuda.synchronize()
    items_view = pool.view(n, 2).cpu()
    written = items_view[:, 1] == 1
    # every written slot holds {k, 1} with k < items; with 16 updates per slot on average nearly all are written
    assert int(written.sum()) > 0.99 * n
    assert bool(((items_view[written, 0] >= 0) & (items_view[written, 0] < items)).all())
    assert bool((items_view[~written] == -1).all())
    assert float(sink[0]) == 0.0


@pytest.mark.parametrize("interleave", [0, 1])
def test_tile_stream_probe_reads_and_writes_nothing(interleave):
    import torch
    grid = 64
    entries = grid * 2048 * 3  # three tiles per wavefront
    note("tile stream probe grid=%d entries=%d interleave=%d" % (grid, entries, interleave))
    a = torch.zeros(entries, dtype=torch.int32, device="cuda")
    b = torch.zeros(entries, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    xt.xtvxy_tile_stream_probe(a.data_ptr(), b.data_ptr(), entries, grid, interleave, sink.data_ptr(), None)
    torch.cuda.synchronize()
    assert float(sink[0]) == 0.0
    with pytest.raises(xt.XtvxyError):  # not a whole number of tiles per wavefront
        xt.xtvxy_tile_stream_probe(a.data_ptr(), b.data_ptr(), entries - 4, grid, interleave, sink.data_ptr(), None)
