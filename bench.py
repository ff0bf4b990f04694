#!/usr/bin/env python3
"""Benchmark of the fused out = alpha * X^T (v .* (X y)) + beta * z on one GPU.

One step is one call of the fused path (main fused kernel + aggregation) on a
batch of synthetic input already resident in HBM. Default workload: dense
65,536 x 8192 fp32 X ~ U(-1, 1), v ~ U(0, 1), y, z ~ U(-1, 1), alpha = beta = 1 —
the largest configuration (2 GiB of X) — with the other measured configurations
(dense 1,000,000 x 256 normal equations, the CSR logistic Hessian-vector product,
the CSR Zipf matrix and its column-permuted form) carried on the same line under
``other_configs``. Prints one JSON line with:
  value            effective GB/s = algorithmic bytes per step / wall time per step
  call_ms          median, p10, p90 of per-call times (HIP events around each call)
  roofline         the main fused kernel's algorithmic bytes / its mean duration
                   (HIP events recorded around it on the call's stream) vs 8 TB/s
  peaks            the published 8 TB/s, the device properties' theoretical peak and
                   the measured streaming-read ceiling, with the kernel's fraction of each
  speedup_vs_unfused  wall time of the rocBLAS/rocSPARSE chain / fused wall time
  speedup_vs_unfused_explicit_transpose
                   the same chain with X^T kept as a second matrix (made once, outside the
                   timed region), so that both products take the library's fast path
  cpu_baseline     the CPU oracle on the host cores (same algorithmic-bytes formula)
Algorithmic bytes: every operand once — dense 4mn (X) + 4m (v, if given) + 4n (y)
+ 4n (z, if beta != 0) + 4n (out); CSR 8 nnz + 4(m + 1) + 4m (v) + 4n (y) + 4n (z)
+ 4n (out).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused X^T(v⊙Xy) effective GB/s, % of HBM peak, speedup vs unfused GEMV"
DEFAULT_WORKLOAD = "dense_65536x8192"
# the other configurations measured by a default run (each timed with --also-steps calls)
ALSO_DEFAULT = ["dense_1000000x256_normal_equations", "csr_10000000x1000_logistic_hvp", "csr_5000000x1000000_zipf",
                "csr_5000000x1000000_zipf_permuted"]
# workloads whose oracle is also timed on one host thread
SINGLE_THREAD_CPU = ("dense_2048x128", "dense_1000000x256_normal_equations")
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E peak


def algorithmic_bytes(p) -> int:
    if hasattr(p, "col_idx"):
        vb = 2 if getattr(p, "values_dtype", "f32") == "bf16" else 4  # bf16 values: 2 bytes each
        b = (vb + 4) * p.nnz + 4 * (p.m + 1) + 4 * p.n + 4 * p.n
        b += 4 * p.m if p.v is not None else 0
    else:
        xb = 2 if getattr(p, "x_dtype", "f32") in ("bf16", "f16") else 4  # 16-bit X: 2 bytes per element
        b = xb * p.m * p.n + 4 * p.n + 4 * p.n
        b += 4 * p.m if p.v is not None else 0
    b += 4 * p.n if p.beta != 0 else 0
    return b


class HipEvents:
    """hipEvent_t pairs from libamdhip64 (the events the library records around its main kernel).
    They are created without the system-scope fence HIP otherwise puts on a record: the timing
    is on the device, and the fence would add several microseconds to every call."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventSynchronize(b) != 0 or self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def kernel_sources_hash(kind: str) -> str:
    csrc = os.path.join(ROOT, "dense_linear_algebra_alpha_amd", "csrc")
    files = ["device_util.h", "internal.h"] + {"csr": ["csr_common.h", "csr.hip"],
                                                "csr_waves": ["csr_common.h", "csr_waves.hip"],
                                                "csr_rows": ["csr_common.h", "csr_rows.hip"]}.get(kind, ["dense.hip"])
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_name(plan) -> str:
    """Name of the main fused kernel a plan launches (dense_block_rows serves both block paths;
    dense_group_rows is its group-row form)."""
    import dense_linear_algebra_alpha_amd as xt
    names = {xt.XTVXY_DENSE_WAVE_ROWS: "dense_wave_rows", xt.XTVXY_DENSE_BLOCK_ROWS: "dense_block_rows",
             xt.XTVXY_DENSE_GROUP_ROWS: "dense_group_rows", xt.XTVXY_CSR_TILES: "csr_fused",
             xt.XTVXY_CSR_WAVES: "csr_waves", xt.XTVXY_CSR_ROWS: "csr_rows"}
    return names.get(plan.kernel, "kernel%d" % plan.kernel)


def load_traffic(workload: str, kernel: str, kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE,
    each scaled by what it reads on a plain copy of known size), when it was taken on this source."""
    path = os.path.join(ROOT, "profiles", "%s__%s.counters.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha256") != kernel_sources_hash(kind):
        return None
    fetch = c["fetch_kib_per_dispatch"] * 1024.0 * c.get("fetch_scale", 1.0)
    write = c["write_kib_per_dispatch"] * 1024.0 * c.get("write_scale", 1.0)
    return fetch + write


def override(plan, text):
    """Replace fields of the model's plan with those of a JSON object (--plan); True when forced."""
    if not text:
        return False
    for k, val in json.loads(text).items():
        if k not in dict(plan._fields_):
            raise SystemExit("unknown plan field %s" % k)
        setattr(plan, k, val)
    return True


def cpu_baseline(p, budget_s: float, threads=None, min_runs=3):
    """The oracle, as it is, on the host cores: repeated runs of the full workload for ~budget_s."""
    import numpy as np

    import oracle
    threads = oracle.set_threads(threads or len(os.sched_getaffinity(0)))
    runs = []
    vals = p.values_f32() if hasattr(p, "col_idx") else None  # bf16 values widened (exactly) once
    X = None if hasattr(p, "col_idx") else (p.X.astype(np.float32) if p.x_dtype == "f16" else p.X)  # fp16: widened
    t_end = time.perf_counter() + budget_s
    while len(runs) < min_runs or (time.perf_counter() < t_end and len(runs) < 200):
        t0 = time.perf_counter()
        if hasattr(p, "col_idx"):
            oracle.csr(p.row_ptr, p.col_idx, vals, p.n, p.y, p.v, p.z, p.alpha, p.beta)
        else:
            oracle.dense(X, p.y, p.v, p.z, p.alpha, p.beta, m=p.m, n=p.n, ldx=p.ldx)
        runs.append(time.perf_counter() - t0)
    med = statistics.median(runs)
    oracle.set_threads(len(os.sched_getaffinity(0)))
    return {"value": round(algorithmic_bytes(p) / med / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": "the full workload, %d runs (median %.3f s each)" % (len(runs), med),
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentiles(ms):
    """median, p10, p90 and mean of a list of per-call times (ms)."""
    q = sorted(ms)

    def pct(f):
        k = (len(q) - 1) * f
        lo, hi = int(k), min(int(k) + 1, len(q) - 1)
        return q[lo] + (q[hi] - q[lo]) * (k - lo)
    return {"median": round(pct(0.5), 5), "p10": round(pct(0.1), 5), "p90": round(pct(0.9), 5),
            "mean": round(statistics.mean(q), 5)}


def stream_read_ceiling(xt, torch, dev, nbytes=2 << 30, reps=20):
    """GB/s of the library's streaming-read probe over a 2 GiB buffer: the best of `reps` timed
    launches after 5 warmup launches (HIP events on the current stream)."""
    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream().cuda_stream or None
    grid = 8 * xt.xtvxy_get_device_info().compute_units
    for _ in range(5):
        xt.xtvxy_read_probe(buf.data_ptr(), nbytes, grid, sink.data_ptr(), sh)
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(reps)]
    for a, b in pairs:
        ev.record(a, sh)
        xt.xtvxy_read_probe(buf.data_ptr(), nbytes, grid, sink.data_ptr(), sh)
        ev.record(b, sh)
    torch.cuda.synchronize()
    ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    del buf
    return {"gbs": round(nbytes / (min(ms) / 1e3) / 1e9, 1), "median_gbs": round(nbytes / (statistics.median(ms) / 1e3) / 1e9, 1),
            "bytes": nbytes, "what": "16-byte non-temporal loads over %d workgroups, best of %d launches" % (grid, reps)}


def scatter_probe(args):
    """Rates of the primitives a scatter to columns outside an LDS window could use, from the
    library's probe kernel: updates per second (best and median of 10 timed launches after 3
    warmup launches, HIP events) and the time the given number of updates takes."""
    import torch

    import dense_linear_algebra_alpha_amd as xt

    xt.load()
    dev = torch.device("cuda", 0)
    n, items = args.probe_columns, args.probe_updates
    grid = 8 * xt.xtvxy_get_device_info().compute_units
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream().cuda_stream or None
    ev = HipEvents()
    kinds = [("fp32 atomics, one copy per XCD, workgroup scope", xt.XTVXY_PROBE_ATOMIC_PER_XCD, 8 * n * 4),
             ("fp32 atomics, one copy, device scope", xt.XTVXY_PROBE_ATOMIC_DEVICE, n * 4),
             ("8-byte item stores, scattered", xt.XTVXY_PROBE_ITEM_STORES, n * 8),
             ("4-byte gathers, scattered", xt.XTVXY_PROBE_GATHERS, n * 4)]
    rows = []
    for skew in (0, 1):
        for what, kind, nbytes in kinds:
            buf = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)
            for _ in range(3):
                xt.xtvxy_scatter_probe(kind, buf.data_ptr(), nbytes, n, items, skew, grid, sink.data_ptr(), sh)
            pairs = [(ev.create(), ev.create()) for _ in range(10)]
            for a, b in pairs:
                ev.record(a, sh)
                xt.xtvxy_scatter_probe(kind, buf.data_ptr(), nbytes, n, items, skew, grid, sink.data_ptr(), sh)
                ev.record(b, sh)
            torch.cuda.synchronize()
            ms = [ev.elapsed_ms(a, b) for a, b in pairs]
            for a, b in pairs:
                ev.destroy(a)
                ev.destroy(b)
            rows.append({"what": what, "skew": skew, "updates": items, "columns": n,
                         "best_ms": round(min(ms), 4), "median_ms": round(statistics.median(ms), 4),
                         "g_updates_per_s": round(items / (min(ms) / 1e3) / 1e9, 2)})
            print(json.dumps(rows[-1]), flush=True)
            del buf
    print(json.dumps({"scatter_probe": rows, "grid": grid, "threads_per_workgroup": 256}))


def tile_stream_probe(args):
    """The wavefront CSR kernel's access pattern alone (xtvxy_tile_stream_probe) on as many
    entries of the logistic workload's size as the launch shape divides: each wavefront its own
    stretch (the kernel's layout) and the workgroup's wavefronts interleaved, at the kernel's
    launch shape (256 threads, 3 workgroups per CU) and around it; GB/s counts 8 bytes per entry
    (best and median of 20 launches after 5 warmup launches, HIP events)."""
    import torch

    import dense_linear_algebra_alpha_amd as xt

    xt.load()
    dev = torch.device("cuda", 0)
    cus = xt.xtvxy_get_device_info().compute_units
    nnz = args.probe_entries
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream().cuda_stream or None
    ev = HipEvents()
    rows = []
    for per_cu in (2, 3, 4):
        grid = per_cu * cus
        entries = nnz // (grid * 2048) * (grid * 2048)
        a = torch.zeros(entries, dtype=torch.int32, device=dev)
        b = torch.zeros(entries, dtype=torch.float32, device=dev)
        for interleave in (0, 1):
            for _ in range(5):
                xt.xtvxy_tile_stream_probe(a.data_ptr(), b.data_ptr(), entries, grid, interleave, sink.data_ptr(), sh)
            pairs = [(ev.create(), ev.create()) for _ in range(20)]
            for p0, p1 in pairs:
                ev.record(p0, sh)
                xt.xtvxy_tile_stream_probe(a.data_ptr(), b.data_ptr(), entries, grid, interleave, sink.data_ptr(), sh)
                ev.record(p1, sh)
            torch.cuda.synchronize()
            ms = [ev.elapsed_ms(p0, p1) for p0, p1 in pairs]
            for p0, p1 in pairs:
                ev.destroy(p0)
                ev.destroy(p1)
            rows.append({"layout": "workgroup's wavefronts interleaved" if interleave else "wavefront's own stretch",
                         "grid": grid, "workgroups_per_cu": per_cu, "entries": entries,
                         "best_us": round(min(ms) * 1e3, 1), "median_us": round(statistics.median(ms) * 1e3, 1),
                         "gbs": round(8 * entries / (min(ms) / 1e3) / 1e9, 1),
                         "median_gbs": round(8 * entries / (statistics.median(ms) / 1e3) / 1e9, 1)})
            print(json.dumps(rows[-1]), flush=True)
        del a, b
    print(json.dumps({"tile_stream_probe": rows, "threads_per_workgroup": 256}))


LOGREG_METRIC = "Newton-CG logistic regression: ms per Newton iteration (fixed schedule), fused vs unfused products"


def logreg_iteration_bytes(m, n, nnz, J, trials, value_bytes=4) -> int:
    """Algorithmic bytes of one Newton step with J CG iterations and `trials` line-search trials:
    the link pass (read t, X s, labels; write t, u, v), the gradient X^T u + lambda w, J
    Hessian-vector products, X s, and the trials (read t, X s, labels). The n-vector algebra
    is left out (n << m). A stored entry is a 4-byte column index and a value of value_bytes."""
    rows = 4 * (m + 1) + (4 + value_bytes) * nnz
    link = 24 * m
    grad = rows + 4 * m + 12 * n
    hvp = rows + 4 * m + 12 * n
    xs = rows + 4 * n + 4 * m
    return link + grad + J * hvp + xs + trials * 12 * m


def bench_logreg(args):
    """The Newton-CG solver on its workload: a fixed schedule (K Newton steps of J CG iterations,
    grad_tol 0) timed for both engines, a run to |g| <= 1e-4 |g_0| for both, the Hessian-vector
    kernel's roofline at the solver's final curvature weights, and the oracle's time for one step
    of the same schedule on the host cores. With bf16 values the fused engine runs on them and the
    comparisons (the fused engine on the values widened to fp32, and the unfused engines, which
    take fp32 only) on the widened values."""
    import numpy as np
    import torch

    import datagen
    import dense_linear_algebra_alpha_amd as xt

    xt.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    P = datagen.LOGISTIC_WORKLOADS[args.workload](seed=args.seed)
    X = P.X
    bf16 = X.values_dtype == "bf16"
    vb = 2 if bf16 else 4
    rp, ci = (torch.from_numpy(a).to(dev) for a in (X.row_ptr, X.col_idx))
    vals = (torch.from_numpy(X.values.view(np.int16)).view(torch.bfloat16) if bf16
            else torch.from_numpy(X.values)).to(dev)
    vals32 = torch.from_numpy(X.values_f32()).to(dev) if bf16 else vals
    lab = torch.from_numpy(P.labels).to(dev)
    plans = {"unfused": xt.CsrUnfusedPlan(rp, ci, vals32, X.n),
             "unfused_explicit_transpose": xt.CsrUnfusedPlan(rp, ci, vals32, X.n, explicit_transpose=True)}
    ws = torch.empty(xt.xtvxy_logreg_newton_cg_f32_workspace_size(X.m, X.n, X.nnz), dtype=torch.uint8, device=dev)
    K, J = args.newton_steps, args.cg_steps

    def solve(engine, **kw):
        w = torch.zeros(X.n, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fused = engine.startswith("fused")
        w, rep, hist = xt.logreg_newton_cg(rp, ci, vals if engine == "fused" else vals32, X.n, lab, P.lam, w,
                                           engine="fused" if fused else "unfused",
                                           unfused_plan=plans.get(engine), workspace=ws, **kw)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, w, rep, hist

    fixed = dict(grad_tol=0.0, max_newton=K, max_cg=J, fixed_cg=True)
    results = {}
    engines = ("fused",) + (("fused_f32_values",) if bf16 else ()) + ("unfused", "unfused_explicit_transpose")
    for engine in engines:
        for _ in range(args.warmup_solves):
            solve(engine, **fixed)
        runs = [solve(engine, **fixed) for _ in range(args.solves)]
        wall = statistics.median(r[0] for r in runs)
        rep = runs[-1][2]
        conv = solve(engine, grad_tol=1e-4, max_newton=50)
        results[engine] = {"ms_per_newton_iteration": round(wall / K * 1e3, 4), "solve_ms": round(wall * 1e3, 3),
                           "line_search_trials": rep["line_search_trials"],
                           "to_1e-4": {"ms": round(conv[0] * 1e3, 3), "newton_iterations": conv[2]["newton_iterations"],
                                       "cg_iterations": conv[2]["cg_iterations"], "status": conv[2]["status"],
                                       "loss": conv[2]["loss"]}}
    fz = results["fused"]
    trials = fz["line_search_trials"] / K
    ibytes = logreg_iteration_bytes(X.m, X.n, X.nnz, J, trials, vb)
    # the Hessian-vector kernel alone, with the generator's curvature weights p(1 - p) of the planted
    # model and the generator's y as the direction
    v = torch.from_numpy(X.v).to(dev)
    d = torch.from_numpy(X.y).to(dev)
    q = torch.empty_like(d)
    # the plan the solver's products take: the model's, refined by the longest row
    hplan = xt.xtvxy_csr_f32_plan_rows(X.m, X.n, X.nnz, int(np.diff(X.row_ptr).max(initial=0)))
    hws_bytes = hplan.workspace_bytes
    hws = torch.empty(max(hws_bytes, 1), dtype=torch.uint8, device=dev)
    sh = torch.cuda.current_stream().cuda_stream or None
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    hvp = xt.xtvxy_csr_bf16_ex if bf16 else xt.xtvxy_csr_f32_ex
    for _ in range(args.warmup):
        hvp(X.m, X.n, X.nnz, 1.0, rp.data_ptr(), ci.data_ptr(), vals.data_ptr(), v.data_ptr(),
            d.data_ptr(), P.lam, d.data_ptr(), q.data_ptr(), hws.data_ptr(), hws_bytes, sh, hplan)
    for i in range(args.steps):
        xt.xtvxy_set_kernel_timing_events(pairs[i][0], pairs[i][1])
        hvp(X.m, X.n, X.nnz, 1.0, rp.data_ptr(), ci.data_ptr(), vals.data_ptr(), v.data_ptr(),
            d.data_ptr(), P.lam, d.data_ptr(), q.data_ptr(), hws.data_ptr(), hws_bytes, sh, hplan)
    torch.cuda.synchronize()
    xt.xtvxy_set_kernel_timing_events(None, None)
    kernel_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    hvp_bytes = (4 + vb) * X.nnz + 4 * (X.m + 1) + 4 * X.m + 12 * X.n
    achieved = hvp_bytes / (statistics.mean(kernel_ms) / 1e3) / 1e9
    iter_s = fz["ms_per_newton_iteration"] / 1e3
    record = {
        "metric": LOGREG_METRIC,
        "value": fz["ms_per_newton_iteration"],
        "unit": "ms",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup_solves,
        "ms_per_step": fz["ms_per_newton_iteration"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generators, seed %d): labels of a planted model" % args.seed,
        "config": {"workload": args.workload, "m": X.m, "n": X.n, "nnz": X.nnz, "lambda": P.lam,
                   "values_storage": "bf16" if bf16 else "f32",
                   "schedule": "%d Newton steps x %d CG iterations, grad_tol 0" % (K, J),
                   "iteration_algorithmic_bytes": int(ibytes)},
        "iteration_effective_gbs": round(ibytes / iter_s / 1e9, 3),
        "fused": fz,
        **({"fused_f32_values": results["fused_f32_values"],
            "speedup_vs_fused_f32_values": round(results["fused_f32_values"]["ms_per_newton_iteration"] /
                                                 fz["ms_per_newton_iteration"], 3)} if bf16 else {}),
        "unfused": results["unfused"],
        "unfused_explicit_transpose": results["unfused_explicit_transpose"],
        "speedup_vs_unfused": round(results["unfused"]["ms_per_newton_iteration"] / fz["ms_per_newton_iteration"], 3),
        "speedup_vs_unfused_explicit_transpose": round(
            results["unfused_explicit_transpose"]["ms_per_newton_iteration"] / fz["ms_per_newton_iteration"], 3),
        "roofline": {"bound": "hbm", "kernel": kernel_name(hplan), "grid": hplan.grid,
                     "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "what": "the Hessian-vector product alone (one fused call, v = p(1 - p), y = z = d, "
                             "beta = lambda)",
                     "kernel_ms_mean": round(statistics.mean(kernel_ms), 5)},
    }
    if not args.no_cpu_baseline:
        import oracle
        import oracle.logreg as lr
        threads = oracle.set_threads(len(os.sched_getaffinity(0)))
        t0 = time.perf_counter()
        lr.newton_cg(X.row_ptr, X.col_idx, X.values_f32(), X.n, P.labels, P.lam, max_newton=1, max_cg=J,
                     fixed_cg=True, grad_tol=0.0)
        cpu_s = time.perf_counter() - t0
        record["cpu_baseline"] = {"value": round(cpu_s * 1e3, 1), "unit": "ms", "cores": 1, "kind": "oracle",
                                  "sample": "one Newton step of the same schedule on the full workload (fp64 "
                                            "scipy.sparse products, single-threaded), setup included; threads "
                                            "available %d" % threads, "cpu_model": cpu_model()}
    print(json.dumps(record), flush=True)


def report_tuning(args, p, kind, abytes, env):
    """--tune: the empirical tuner on this workload; prints the model's plan, the best measured plan,
    their times and the model's regret (model time / best time - 1)."""
    import dense_linear_algebra_alpha_amd as xt
    y, v, z, out, sh = env["y"], env["v"], env["z"], env["out"], env["sh"]
    t0 = time.perf_counter()
    if kind == "dense":
        X = env["X"]
        tune_fn = (xt.xtvxy_dense_f16_tune if env.get("f16") else
                   xt.xtvxy_dense_bf16_tune if env["bf16"] else xt.xtvxy_dense_f32_tune)
        rep = tune_fn(p.m, p.n, p.alpha, X.data_ptr(), p.ldx, xt._ptr(v), y.data_ptr(), p.beta,
                                      xt._ptr(z), out.data_ptr(), args.tune_repeats, sh)
    else:
        rp, ci, vals = env["rp"], env["ci"], env["vals"]
        tune_fn = xt.xtvxy_csr_bf16_tune if env.get("bf16") else xt.xtvxy_csr_f32_tune
        rep = tune_fn(p.m, p.n, p.nnz, p.alpha, rp.data_ptr(), ci.data_ptr(), vals.data_ptr(),
                      xt._ptr(v), y.data_ptr(), p.beta, xt._ptr(z), out.data_ptr(), args.tune_repeats, sh)
    wall = time.perf_counter() - t0
    r = rep.as_dict()
    keep = lambda d: {k: v_ for k, v_ in d.items() if k != "predicted_seconds"}
    record = {"metric": "analytical model regret against the empirical tuner (model time / best time - 1)",
              "value": round(r["model_seconds"] / r["best_seconds"] - 1.0, 4), "unit": "fraction",
              "higher_is_better": False, "config": {"workload": args.workload, "repeats": args.tune_repeats},
              "model_ms": round(r["model_seconds"] * 1e3, 5), "best_ms": round(r["best_seconds"] * 1e3, 5),
              "model_gbs": round(abytes / r["model_seconds"] / 1e9, 1),
              "best_gbs": round(abytes / r["best_seconds"] / 1e9, 1), "candidates": r["candidates"],
              "tuning_seconds": round(wall, 2), "model_plan": keep(r["model"]), "best_plan": keep(r["best"])}
    if args.tune_cache:
        xt.xtvxy_tune_cache_save(args.tune_cache)
    print(json.dumps(record), flush=True)
    return record


def measure_workload(name, args, steps, warmup, unfused_calls, cpu_budget, headline, ctx, csr_path="plain"):
    """Times one workload's fused call (and its comparators); returns the record's fields. CSR
    workloads take the plain entry point (csr_path "plain") or the analysed one ("analysed": the
    structure analysis made once, outside the timed region)."""
    import numpy as np
    import torch

    import datagen
    import dense_linear_algebra_alpha_amd as xt

    dev = torch.device("cuda:0")
    p = datagen.WORKLOADS[name](seed=args.seed)
    kind = "csr" if hasattr(p, "col_idx") else "dense"

    def t(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:  # bf16 bit patterns
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    y, v, z = t(p.y), t(p.v), t(p.z)
    out = torch.empty(p.n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream or None
    # 16-bit storage: of X (dense, bf16 or fp16) or of the values (CSR, bf16); the comparison is then
    # the fp32 fused path on the widened numbers
    f16 = getattr(p, "x_dtype", "f32") == "f16"
    bf16 = getattr(p, "x_dtype", "f32") == "bf16" or f16 or getattr(p, "values_dtype", "f32") == "bf16"
    plan_text = args.plan if headline else None
    with_unfused = unfused_calls > 0 and not args.fused_only
    if kind == "dense":
        X = t(p.X)
        plan_fn, complete_fn, ws_fn, call, call_ex = (
            (xt.xtvxy_dense_bf16_plan, xt.xtvxy_dense_bf16_plan_complete, xt.xtvxy_dense_bf16_workspace_size,
             xt.xtvxy_dense_f16 if f16 else xt.xtvxy_dense_bf16, xt.xtvxy_dense_f16_ex if f16 else xt.xtvxy_dense_bf16_ex)
            if bf16 else
            (xt.xtvxy_dense_f32_plan, xt.xtvxy_dense_f32_plan_complete, xt.xtvxy_dense_f32_workspace_size,
             xt.xtvxy_dense_f32, xt.xtvxy_dense_f32_ex))
        plan = plan_fn(p.m, p.n, p.ldx, 1 if X.data_ptr() % 16 == 0 else 0)
        forced = override(plan, plan_text)
        if forced:
            plan = complete_fn(p.m, p.n, p.ldx, plan)
        ws_bytes = plan.workspace_bytes if forced else ws_fn(p.m, p.n, p.ldx)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        uws_bytes = xt.xtvxy_dense_f32_unfused_reference_workspace_size(p.m, p.n)
        uws = torch.empty(max(uws_bytes, 1), dtype=torch.uint8, device=dev) if with_unfused else None
        # 16-bit X: the comparison is the fp32 fused path on the same matrix widened to fp32
        X32 = t(p.X_f32()) if bf16 and with_unfused else X
        ws32_bytes = xt.xtvxy_dense_f32_workspace_size(p.m, p.n, p.ldx)
        ws32 = torch.empty(max(ws32_bytes, 1), dtype=torch.uint8, device=dev) if bf16 and with_unfused else None

        def fused():
            if forced:
                call_ex(p.m, p.n, p.alpha, X.data_ptr(), p.ldx, xt._ptr(v), y.data_ptr(), p.beta, xt._ptr(z),
                        out.data_ptr(), ws.data_ptr(), ws_bytes, sh, plan)
            else:
                call(p.m, p.n, p.alpha, X.data_ptr(), p.ldx, xt._ptr(v), y.data_ptr(), p.beta, xt._ptr(z),
                     out.data_ptr(), ws.data_ptr(), ws_bytes, sh)

        def unfused():
            if bf16:
                xt.xtvxy_dense_f32(p.m, p.n, p.alpha, X32.data_ptr(), p.ldx, xt._ptr(v), y.data_ptr(), p.beta,
                                   xt._ptr(z), out.data_ptr(), ws32.data_ptr(), ws32_bytes, sh)
            else:
                xt.xtvxy_dense_f32_unfused_reference(p.m, p.n, p.alpha, X.data_ptr(), p.ldx, xt._ptr(v),
                                                     y.data_ptr(), p.beta, xt._ptr(z), out.data_ptr(),
                                                     uws.data_ptr(), uws_bytes, sh)
        unfused_explicit = None
        if with_unfused and not bf16:
            # the stronger comparator: X^T copied once (set-up, outside every timed region) so
            # that both products are transposed sgemvs
            Xt = torch.empty((p.n, p.m), dtype=torch.float32, device=dev)
            xt.xtvxy_dense_f32_transpose(p.m, p.n, X.data_ptr(), p.ldx, Xt.data_ptr(), p.m, sh)
            torch.cuda.synchronize()

            def unfused_explicit():
                xt.xtvxy_dense_f32_unfused_reference_explicit(p.m, p.n, p.alpha, X.data_ptr(), p.ldx, Xt.data_ptr(),
                                                              p.m, xt._ptr(v), y.data_ptr(), p.beta, xt._ptr(z),
                                                              out.data_ptr(), uws.data_ptr(), uws_bytes, sh)
        shape = {"m": p.m, "n": p.n, "ldx": p.ldx, "x_storage": p.x_dtype}
        env = {"X": X, "y": y, "v": v, "z": z, "out": out, "sh": sh, "bf16": bf16, "f16": f16}
    else:
        rp, ci, vals = t(p.row_ptr), t(p.col_idx), t(p.values)
        analysed = csr_path == "analysed"
        analysis = None
        if analysed:
            # the structure analysis (column counts, relabelled columns, row classes): set-up,
            # outside every timed region, like the comparators' plans below
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            analysis = xt.CsrAnalysis(rp, ci, p.n)
            torch.cuda.synchronize()
            analysis_s = time.perf_counter() - t0
            plan = analysis.plan()
            forced = override(plan, plan_text)
            if forced:
                plan = analysis.complete(plan)
            ws_bytes = plan.workspace_bytes
        else:
            plan = xt.xtvxy_csr_f32_plan(p.m, p.n, p.nnz)
            forced = override(plan, plan_text)
            if forced:
                plan = xt.xtvxy_csr_f32_plan_complete(p.m, p.n, p.nnz, plan)
            ws_bytes = plan.workspace_bytes if forced else xt.xtvxy_csr_f32_workspace_size(p.m, p.n, p.nnz)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        uplan = uplan_t = None
        # bf16 values: the comparison is the fp32 fused path (same entry point) on the widened values
        vals32 = t(p.values_f32()) if bf16 and with_unfused else vals

        def fused_call(vt, bf):
            if analysed:
                (xt.xtvxy_csr_bf16_analysed_ex if bf else xt.xtvxy_csr_f32_analysed_ex)(
                    analysis.handle, p.alpha, vt.data_ptr(), xt._ptr(v), y.data_ptr(), p.beta, xt._ptr(z),
                    out.data_ptr(), ws.data_ptr(), ws_bytes, sh, plan if forced else None)
            elif forced:
                (xt.xtvxy_csr_bf16_ex if bf else xt.xtvxy_csr_f32_ex)(
                    p.m, p.n, p.nnz, p.alpha, rp.data_ptr(), ci.data_ptr(), vt.data_ptr(), xt._ptr(v), y.data_ptr(),
                    p.beta, xt._ptr(z), out.data_ptr(), ws.data_ptr(), ws_bytes, sh, plan)
            else:
                (xt.xtvxy_csr_bf16 if bf else xt.xtvxy_csr_f32)(
                    p.m, p.n, p.nnz, p.alpha, rp.data_ptr(), ci.data_ptr(), vt.data_ptr(), xt._ptr(v), y.data_ptr(),
                    p.beta, xt._ptr(z), out.data_ptr(), ws.data_ptr(), ws_bytes, sh)

        def fused():
            fused_call(vals, bf16)

        def unfused():
            if bf16:
                fused_call(vals32, False)
                return
            xt.xtvxy_csr_f32_unfused_reference(uplan.handle, p.alpha, xt._ptr(v), y.data_ptr(), p.beta, xt._ptr(z),
                                               out.data_ptr(), sh)

        def unfused_explicit():
            xt.xtvxy_csr_f32_unfused_reference(uplan_t.handle, p.alpha, xt._ptr(v), y.data_ptr(), p.beta,
                                               xt._ptr(z), out.data_ptr(), sh)
        if with_unfused and not args.tune and not bf16:
            # structure analysis and the transposed copy: outside every timed region
            uplan = xt.CsrUnfusedPlan(rp, ci, vals, p.n)
            uplan_t = xt.CsrUnfusedPlan(rp, ci, vals, p.n, explicit_transpose=True)
        else:
            unfused_explicit = None
        entry = ("xtvxy_csr_bf16" if bf16 else "xtvxy_csr_f32") + ("_analysed" if analysed else "")
        shape = {"m": p.m, "n": p.n, "nnz": p.nnz, "entry_point": entry, "values_storage": "bf16" if bf16 else "f32"}
        if analysed:
            shape["analysis_seconds"] = round(analysis_s, 4)
        env = {"rp": rp, "ci": ci, "vals": vals, "y": y, "v": v, "z": z, "out": out, "sh": sh, "bf16": bf16}

    abytes = algorithmic_bytes(p)
    if args.tune:
        return {"tune": report_tuning(args, p, kind, abytes, env)}
    ev = HipEvents()
    kpairs = [(ev.create(), ev.create()) for _ in range(steps)]
    cpairs = [(ev.create(), ev.create()) for _ in range(steps)]

    def timed(fn, n_calls, n_warm, with_events):
        for _ in range(n_warm):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_calls):
            if with_events:
                xt.xtvxy_set_kernel_timing_events(kpairs[i][0], kpairs[i][1])
                ev.record(cpairs[i][0], sh)
            fn()
            if with_events:
                ev.record(cpairs[i][1], sh)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        xt.xtvxy_set_kernel_timing_events(None, None)
        if not with_events:
            return (t1 - t0) / n_calls, None, None
        return ((t1 - t0) / n_calls, [ev.elapsed_ms(a, b) for a, b in kpairs[:n_calls]],
                [ev.elapsed_ms(a, b) for a, b in cpairs[:n_calls]])

    step_s, kernel_ms, call_ms = timed(fused, steps, warmup, True)
    fused_out = out.cpu().numpy()
    unfused_s = explicit_s = None
    if with_unfused:
        unfused_s, _, _ = timed(unfused, unfused_calls, min(warmup, max(2, unfused_calls // 2)), False)
        unfused_out = out.cpu().numpy()
        if unfused_explicit is not None:
            explicit_s, _, _ = timed(unfused_explicit, unfused_calls, min(warmup, max(2, unfused_calls // 2)), False)
            explicit_out = out.cpu().numpy()
    for a, b in kpairs + cpairs:
        ev.destroy(a)
        ev.destroy(b)

    kernel_s = statistics.mean(kernel_ms) / 1e3
    achieved = abytes / kernel_s / 1e9
    kname = kernel_name(plan)
    rec = {
        "value": round(abytes / step_s / 1e9, 3),
        "ms_per_step": round(step_s * 1e3, 5),
        "steps": steps,
        "warmup": warmup,
        "config": dict({"workload": name, "algorithmic_bytes": abytes, "plan_forced": bool(forced),
                        "plan": {k: v_ for k, v_ in plan.as_dict().items() if k != "predicted_seconds"}}, **shape),
        "hbm_peak_fraction": round(abytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "call_ms": percentiles(call_ms),
        "kernel_ms": percentiles(kernel_ms),
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 3),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(name, kname, kname if kname in ("csr_waves", "csr_rows") else kind),
                     "kernel_ms_mean": round(statistics.mean(kernel_ms), 5),
                     "kernel_ms_min": round(min(kernel_ms), 5)},
        "peaks": {"published_gbs": HBM_PEAK_GBS, "device_properties_gbs": ctx["device_peak_gbs"],
                  "stream_read_ceiling_gbs": ctx["ceiling_gbs"],
                  "kernel_frac_of_device_peak": round(achieved / ctx["device_peak_gbs"], 4),
                  "kernel_frac_of_ceiling": (round(achieved / ctx["ceiling_gbs"], 4)
                                             if ctx["ceiling_gbs"] else None),
                  "call_frac_of_ceiling": (round(abytes / step_s / 1e9 / ctx["ceiling_gbs"], 4)
                                           if ctx["ceiling_gbs"] else None)},
    }
    if unfused_s is not None and bf16:  # the comparison is the fp32 fused path on the widened X or values
        rec["f32_fused_ms_per_step"] = round(unfused_s * 1e3, 5)
        rec["speedup_vs_f32_fused"] = round(unfused_s / step_s, 3)
    elif unfused_s is not None:
        rec["unfused_ms_per_step"] = round(unfused_s * 1e3, 5)
        rec["unfused_calls_timed"] = unfused_calls
        rec["speedup_vs_unfused"] = round(unfused_s / step_s, 3)
    if explicit_s is not None:  # the same chain with X^T kept as a second matrix (CSR, or dense row-major)
        rec["unfused_explicit_transpose_ms_per_step"] = round(explicit_s * 1e3, 5)
        rec["speedup_vs_unfused_explicit_transpose"] = round(explicit_s / step_s, 3)

    # parity of the timed outputs against the oracle (max elementwise error relative to the bound)
    if not args.fused_only:
        import oracle
        if kind == "dense":
            X = p.X.astype(np.float32) if p.x_dtype == "f16" else p.X  # fp16 X widened exactly by numpy
            ref = oracle.dense(X, p.y, p.v, p.z, p.alpha, p.beta, m=p.m, n=p.n, ldx=p.ldx)
            bnd = oracle.dense(X, p.y, p.v, p.z, p.alpha, p.beta, m=p.m, n=p.n, ldx=p.ldx, bound=True)
        else:
            vals64 = p.values_f32()  # bf16 values widened exactly
            ref = oracle.csr(p.row_ptr, p.col_idx, vals64, p.n, p.y, p.v, p.z, p.alpha, p.beta)
            bnd = oracle.csr(p.row_ptr, p.col_idx, vals64, p.n, p.y, p.v, p.z, p.alpha, p.beta, bound=True)
        den = np.where(bnd > 0, bnd, 1.0)
        rec["max_rel_err"] = float(np.max(np.abs(fused_out.astype(np.float64) - ref) / den))
        if unfused_s is not None:
            key = "f32_fused_max_rel_err" if bf16 else "unfused_max_rel_err"
            rec[key] = float(np.max(np.abs(unfused_out.astype(np.float64) - ref) / den))
        if explicit_s is not None:
            rec["unfused_explicit_transpose_max_rel_err"] = float(
                np.max(np.abs(explicit_out.astype(np.float64) - ref) / den))
        if not args.no_cpu_baseline and cpu_budget > 0:
            rec["cpu_baseline"] = cpu_baseline(p, cpu_budget)
            if name in SINGLE_THREAD_CPU:
                rec["cpu_baseline_single_thread"] = cpu_baseline(p, min(cpu_budget, 5.0), threads=1, min_runs=1)
    del p
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU's clocks and translation caches settle over the first ~10-20 ms of work
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default="default",
                    help="comma-separated further workloads measured on the same line ('default': the other "
                         "configurations when the default workload runs; 'none': no others)")
    ap.add_argument("--also-steps", type=int, default=40, help="timed fused calls of each further workload")
    ap.add_argument("--also-warmup", type=int, default=60, help="untimed fused calls of each further workload")
    ap.add_argument("--unfused-steps", type=int, default=20,
                    help="timed calls of the unfused comparators (their transposed products are slow)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle runs for cpu_baseline")
    ap.add_argument("--also-cpu-budget", type=float, default=2.0, help="seconds of oracle runs per further workload")
    ap.add_argument("--fused-only", action="store_true", help="time the fused path only (for profilers)")
    ap.add_argument("--csr-path", choices=("analysed", "plain", "both"), default="both",
                    help="CSR workloads: the analysed entry point, the plain one, or both (the analysed call is "
                         "the record's, the plain one under plain_call)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling measurement")
    ap.add_argument("--plan", default=None,
                    help="JSON object of launch-parameter fields that replace the model's choice, e.g. "
                         "'{\"lds_window\": 16384, \"y_window\": 0, \"bin_columns\": 0}' (the library checks the result)")
    ap.add_argument("--newton-steps", type=int, default=5, help="solver workloads: Newton steps of the timed schedule")
    ap.add_argument("--cg-steps", type=int, default=10, help="solver workloads: CG iterations per Newton step")
    ap.add_argument("--solves", type=int, default=5, help="solver workloads: timed solves per engine")
    ap.add_argument("--warmup-solves", type=int, default=2, help="solver workloads: untimed solves per engine")
    ap.add_argument("--tune", action="store_true",
                    help="run the empirical tuner on the workload and report the analytical model's regret")
    ap.add_argument("--tune-repeats", type=int, default=10, help="timed calls per candidate plan (--tune)")
    ap.add_argument("--tune-cache", default=None, help="save the tuner's cache to this file (--tune)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the reference reading "
                         "for the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--tile-stream-probe", action="store_true",
                    help="the wavefront CSR kernel's access pattern alone (two arrays, 8 entries per lane), "
                         "each wavefront's own stretch against the workgroup's wavefronts interleaved")
    ap.add_argument("--probe-entries", type=int, default=100_006_237,
                    help="entries for --tile-stream-probe (default: the logistic workload's nnz)")
    ap.add_argument("--scatter-probe", action="store_true",
                    help="only measure the rates of the scatter primitives (global fp32 atomics into one copy "
                         "or one copy per XCD, scattered 8-byte item stores, random gathers) and exit")
    ap.add_argument("--probe-columns", type=int, default=1_000_000, help="--scatter-probe: columns n")
    ap.add_argument("--probe-updates", type=int, default=54_782_000,
                    help="--scatter-probe: updates per launch (default: the Zipf matrix's products outside "
                         "an 8986-column window)")
    args = ap.parse_args()
    if args.calibration_copy:
        import torch
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": a.numel() * 4, "repeats": 3}))
        return
    if args.scatter_probe:
        return scatter_probe(args)
    if args.tile_stream_probe:
        return tile_stream_probe(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the fused path is a single-GPU kernel here "
              "(row sharding with one reduce-scatter is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import datagen
    import dense_linear_algebra_alpha_amd as xt

    xt.load()  # fails loudly when the HIP library is not built
    if args.workload in datagen.LOGISTIC_WORKLOADS:
        return bench_logreg(args)
    if args.workload not in datagen.WORKLOADS:
        known = list(datagen.WORKLOADS) + list(datagen.LOGISTIC_WORKLOADS)
        raise SystemExit("unknown workload %s (known: %s)" % (args.workload, ", ".join(known)))
    if args.also == "default":
        also = [w for w in ALSO_DEFAULT if w != args.workload] if (
            args.workload == DEFAULT_WORKLOAD and not args.tune and not args.fused_only and not args.plan) else []
    elif args.also == "none":
        also = []
    else:
        also = [w for w in args.also.split(",") if w]
        for w in also:
            if w not in datagen.WORKLOADS:
                raise SystemExit("unknown workload %s" % w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    info = xt.xtvxy_get_device_info()
    ctx = {"device_peak_gbs": round(info.hbm_bytes_per_s / 1e9, 1), "ceiling_gbs": None}
    ceiling = None
    if not args.no_ceiling and not args.tune:
        ceiling = stream_read_ceiling(xt, torch, dev)
        ctx["ceiling_gbs"] = ceiling["gbs"]
        torch.cuda.empty_cache()
    def measure(w, steps, warmup, cpu_budget, headline):
        """The workload's record; a CSR workload with --csr-path both: the analysed call's record with
        the plain call's under plain_call (same inputs, same comparators)."""
        is_csr = w in datagen.WORKLOADS and w.startswith("csr_")
        unf = 0 if args.no_unfused else args.unfused_steps
        if not is_csr:
            return measure_workload(w, args, steps, warmup, unf, cpu_budget, headline, ctx)
        if args.csr_path != "both":
            return measure_workload(w, args, steps, warmup, unf, cpu_budget, headline, ctx, args.csr_path)
        r = measure_workload(w, args, steps, warmup, unf, cpu_budget, headline, ctx, "analysed")
        torch.cuda.empty_cache()
        plain = measure_workload(w, args, steps, warmup, 0, 0.0, headline, ctx, "plain")
        r["plain_call"] = {k: plain[k] for k in ("value", "ms_per_step", "call_ms", "kernel_ms", "roofline", "config",
                                                 "max_rel_err") if k in plain}
        return r

    print("[bench] %s" % args.workload, file=sys.stderr, flush=True)
    rec = measure(args.workload, args.steps, args.warmup, args.cpu_budget, True)
    if "tune" in rec:
        return
    torch.cuda.empty_cache()
    record = {
        "metric": METRIC,
        "value": rec.pop("value"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": rec.pop("steps"),
        "warmup": rec.pop("warmup"),
        "ms_per_step": rec.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generators, seed %d)" % args.seed,
    }
    record.update(rec)
    if ceiling is not None:
        record["stream_read_ceiling"] = ceiling
    others = {}
    for w in also:
        print("[bench] %s" % w, file=sys.stderr, flush=True)
        o = measure(w, args.also_steps, args.also_warmup, args.also_cpu_budget, False)
        others[w] = o
        torch.cuda.empty_cache()
    if others:
        record["other_configs"] = others
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
