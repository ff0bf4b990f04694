"""Builds libxtvxy.so (the fused kernels and the C ABI) for gfx950 with hipcc.

Objects go to _build/ next to this file and the shared library next to this
file, so it travels with the source tree. Usage: ``python -m
dense_linear_algebra_alpha_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libxtvxy.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "model.cpp", "unfused.cpp", "logreg.cpp", "tune.cpp", "csr_analysis.cpp", "dense.hip", "csr.hip",
           "csr_waves.hip", "csr_rows.hip", "csr_bins.hip",
           "aggregate.hip", "logreg.hip", "probe.hip", "noalloc.hip"]
HEADERS = ["internal.h", "device_util.h", "csr_common.h"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I" + INCLUDE, "-I" + CSRC,
]
# Device code: gfx950 only; hardware float atomics; packed-fp32 instructions off.
DEVICE_FLAGS = [
    "--offload-arch=" + ARCH, "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON_FLAGS + DEVICE_FLAGS + lang + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, msgs))
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libxtvxy.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + [
        "-L" + os.path.join(ROCM, "lib"), "-lrocblas", "-lrocsparse", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


def sources_newer_than_library() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(INCLUDE, "xtvxy.h")]
    return any(os.path.getmtime(f) > t for f in files)


if __name__ == "__main__":
    build(verbose=True)
