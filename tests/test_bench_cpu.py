"""bench.py pieces that need no GPU: the one-GPU guard and the plan override."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import dense_linear_algebra_alpha_amd as xt  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_plan_override_replaces_fields_and_rejects_unknown_ones():
    p = xt.xtvxy_launch_params(kernel=xt.XTVXY_CSR_TILES, block_threads=512, entries_per_thread=8, grid=512)
    assert bench.override(p, None) is False
    assert bench.override(p, json.dumps({"bin_columns": 0, "lds_window": 16384, "block_threads": 256})) is True
    assert (p.bin_columns, p.lds_window, p.block_threads, p.grid) == (0, 16384, 256, 512)
    with pytest.raises(SystemExit):
        bench.override(p, json.dumps({"no_such_field": 1}))


def test_algorithmic_bytes_count_each_operand_once():
    import datagen
    d = datagen.dense_problem(10, 4, seed=1)
    assert bench.algorithmic_bytes(d) == 4 * 10 * 4 + 4 * 10 + 4 * 4 + 4 * 4 + 4 * 4  # X, v, y, z, out
    c = datagen.csr_random(10, 7, seed=2)
    expect = 8 * c.nnz + 4 * 11 + 4 * 7 + 4 * 7 + (4 * 10 if c.v is not None else 0) + (4 * 7 if c.beta else 0)
    assert bench.algorithmic_bytes(c) == expect


def test_newton_iteration_bytes():
    m, n, nnz = 100, 7, 1000
    rows = 4 * (m + 1) + 8 * nnz
    # link 24m; gradient and each HVP: rows + 4m + 12n; X s: rows + 4n + 4m; trials 12m each
    assert bench.logreg_iteration_bytes(m, n, nnz, 0, 0) == 24 * m + (rows + 4 * m + 12 * n) + (rows + 4 * n + 4 * m)
    assert bench.logreg_iteration_bytes(m, n, nnz, 3, 2) - bench.logreg_iteration_bytes(m, n, nnz, 0, 0) == \
        3 * (rows + 4 * m + 12 * n) + 2 * 12 * m


def test_algorithmic_bytes_of_bf16_storage():
    import datagen
    d = datagen.dense_problem(10, 8, seed=1, x_dtype="bf16")
    assert bench.algorithmic_bytes(d) == 2 * 10 * 8 + 4 * 10 + 4 * 8 + 4 * 8 + 4 * 8  # X in 2 bytes per element
