"""Helpers of the GPU parity tests: run the library on seeded inputs and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from parity import max_rel_err

TOL = 1e-4  # max elementwise error relative to the oracle's absolute-value bound


def note(msg: str):
    """Name the case before a GPU step (flushed, so that it survives an abort)."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def _as_tensor(a):
    """numpy -> torch on the host; uint16 arrays are bf16 bit patterns and become torch.bfloat16."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def to_dev(a):
    if a is None:
        return None
    return _as_tensor(a).to(dev())


def dense_oracle(p):
    # fp16 X goes to the oracle widened by numpy (exact); bf16 and fp32 X as stored
    X = p.X.astype(np.float32) if getattr(p, "x_dtype", "f32") == "f16" else p.X
    ref = oracle.dense(X, p.y, p.v, p.z, p.alpha, p.beta, m=p.m, n=p.n, ldx=p.ldx)
    bnd = oracle.dense(X, p.y, p.v, p.z, p.alpha, p.beta, m=p.m, n=p.n, ldx=p.ldx, bound=True)
    return ref, bnd


def csr_oracle(p):
    vals = p.values_f32()  # bf16 values widened exactly: the oracle computes on the numbers they denote
    ref = oracle.csr(p.row_ptr, p.col_idx, vals, p.n, p.y, p.v, p.z, p.alpha, p.beta)
    bnd = oracle.csr(p.row_ptr, p.col_idx, vals, p.n, p.y, p.v, p.z, p.alpha, p.beta, bound=True)
    return ref, bnd


class DenseOnDevice:
    """The arrays of a DenseProblem copied to the GPU."""

    def __init__(self, p, X_offset: int = 0):
        import torch
        self.p = p
        if X_offset:
            src = _as_tensor(p.X)  # float32, or bf16
            buf = torch.empty(p.X.size + X_offset, dtype=src.dtype, device=dev())
            buf[X_offset:].copy_(src)
            self.X = buf[X_offset:]
        else:
            self.X = to_dev(p.X)
        self.y, self.v, self.z = to_dev(p.y), to_dev(p.v), to_dev(p.z)

    def run(self, plan=None, out=None, v="default", alpha=None, beta=None, unfused=False):
        import dense_linear_algebra_alpha_amd as xt
        import torch
        p = self.p
        vv = self.v if isinstance(v, str) else v
        a = p.alpha if alpha is None else alpha
        b = p.beta if beta is None else beta
        if unfused:
            X2 = self.X.view(p.m, p.ldx)[:, : p.n] if p.m > 0 else self.X.view(0, p.n)
            r = xt.dense_unfused(X2, self.y, vv, self.z, a, b, out=out)
        else:
            r = xt.dense(self.X, self.y, vv, self.z, a, b, out=out, m=p.m, n=p.n, ldx=p.ldx, plan=plan)
        torch.cuda.synchronize()
        return r.cpu().numpy()


class CsrOnDevice:
    """The arrays of a CsrProblem copied to the GPU; with entry_offset > 0, col_idx and values
    start that many elements into their buffers (4-byte aligned, not 16-byte aligned for 1-3)."""

    def __init__(self, p, entry_offset: int = 0):
        import torch
        self.p = p
        self.rp = to_dev(p.row_ptr)
        if entry_offset:
            def shifted(a):
                src = _as_tensor(a)
                buf = torch.empty(a.size + entry_offset, dtype=src.dtype, device=dev())
                buf[entry_offset:].copy_(src)
                return buf[entry_offset:]
            self.ci, self.vals = shifted(p.col_idx), shifted(p.values)
        else:
            self.ci, self.vals = to_dev(p.col_idx), to_dev(p.values)
        self.y, self.v, self.z = to_dev(p.y), to_dev(p.v), to_dev(p.z)

    def run(self, plan=None, out=None, alpha=None, beta=None):
        import dense_linear_algebra_alpha_amd as xt
        import torch
        p = self.p
        r = xt.csr(self.rp, self.ci, self.vals, p.n, self.y, self.v, self.z,
                   p.alpha if alpha is None else alpha, p.beta if beta is None else beta, out=out, plan=plan)
        torch.cuda.synchronize()
        return r.cpu().numpy()


def assert_parity(got, ref, bnd, what=""):
    err = max_rel_err(got, ref, bnd)
    assert err <= TOL, "%s: max relative error %.3g > %.1g" % (what, err, TOL)
    return err
