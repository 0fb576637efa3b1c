"""The build's guard against kernels that use scratch memory (CPU only: hipcc
cross-compiles for gfx950 without a GPU)."""

import os
import shutil
import subprocess

import pytest

from paged_kv_cache_266_amd import build

SRC = r"""
#include <hip/hip_runtime.h>
// a private array indexed at run time lives in scratch memory
__global__ void spills(int *o, int i)
{
    int a[512];
    for (int j = 0; j < 512; ++j)
        a[j] = o[j + threadIdx.x] * j;
    o[threadIdx.x] = a[(i + threadIdx.x) & 511];
}
__global__ void clean(int *o) { o[threadIdx.x] += 1; }
"""


def test_guard_flags_a_spilling_kernel_and_only_it(tmp_path):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = tmp_path / "t.hip"
    src.write_text(SRC)
    res = subprocess.run([hipcc, f"--offload-arch={build.ARCH}", "-O3", build._REMARKS, "-c", str(src),
                          "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    bad = build.scratch_kernels(res.stderr)
    assert len(bad) == 1 and bad[0].startswith("_Z6spillsPii"), bad


def test_guard_parses_remarks_without_scratch():
    text = ("x.hip:3:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:3:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build.scratch_kernels(text) == []
    assert build.scratch_kernels(text.replace(": 0 [", ": 16 [")) == ["_Z1kv (16 bytes/lane)"]
