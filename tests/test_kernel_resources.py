"""Register budgets of the dense row kernels, read from the compiler's resource report of a
device-only gfx950 compile (no GPU needed). The group-row kernel runs two workgroups per CU, one
wavefront per SIMD each, so every group-row variant must fit two wavefronts per SIMD (at most 256
registers, none spilled); a third of a step's rows more, or a widened copy of the 16-bit rows kept
across the exchange, would drop that to one and halve the kernel's rate without any other sign."""
import os
import re
import shutil
import subprocess

import pytest

from dense_linear_algebra_alpha_amd import build as B


def resource_report(src):
    cmd = [B.HIPCC] + B.COMMON_FLAGS + B.DEVICE_FLAGS + ["-x", "hip", "--cuda-device-only", "-c",
                                                       os.path.join(B.CSRC, src), "-o", os.devnull,
                                                       "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    return kernels


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_every_group_row_kernel_keeps_two_waves_per_simd():
    kernels = resource_report("dense.hip")
    group = {k: v for k, v in kernels.items() if "dense_block_rows" in k and k.endswith("ELb1EEEvNS_9DenseArgsE")}
    # fp32 (f) with 4-element and element loads, 1-8 chunks; bf16 (t: bit patterns) and fp16 (DF16_)
    # with 8-element loads, 1-4 chunks, and element loads, 1-8 chunks
    assert len(group) == 22, sorted(group)
    for name, r in group.items():
        assert r["ScratchSize"] == 0, (name, r)
        assert r["Occupancy"] >= 2, (name, r)
        assert r["VGPRs"] + r.get("AGPRs", 0) <= 256, (name, r)
