"""Build libpagedkv.so in-tree with hipcc for gfx950.

``python -m paged_kv_cache_266_amd.build`` (or ``build()``) always
recompiles.  Each translation unit is compiled to an object in parallel and
linked into ``paged_kv_cache_266_amd/libpagedkv.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import tempfile
from typing import List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
SOURCES = ["decode.hip", "api.cpp", "errors.cpp", "pool.cpp", "sched.cpp", "serve.cpp", "prefill.hip",
           "prefill_api.cpp"]
# the host-only part (page pool, scheduler, status codes): plain C++, no HIP
HOST_SOURCES = ["errors.cpp", "pool.cpp", "sched.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags() -> List[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        # no packed-FP32 instructions anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


# The compiler's per-kernel resource remarks: every kernel the library ships
# must run without scratch (register spills to memory), which would put
# per-lane memory traffic on the streaming loops and whose use has gone with
# wrong results before; the build fails if any kernel needs it.
_REMARKS = "-Rpass-analysis=kernel-resource-usage"
_FN = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def scratch_kernels(remarks: str) -> List[str]:
    """Kernels whose resource remarks report a nonzero ScratchSize."""
    bad, fn = [], None
    for line in remarks.splitlines():
        m = _FN.search(line)
        if m:
            fn = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{fn} ({m.group(1)} bytes/lane)")
    return bad


def _compile(src: str, obj: str, extra: List[str]) -> str:
    cmd = [hipcc(), *common_flags(), *extra, _REMARKS, "-c", "-x", "hip", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    spills = scratch_kernels(res.stderr)
    if spills:
        raise RuntimeError(f"{os.path.basename(src)}: kernels use scratch memory: " + "; ".join(spills))
    return obj


def build(verbose: bool = False, extra_flags: Optional[List[str]] = None) -> str:
    extra = list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        objs = []
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            futs = [ex.submit(_compile, os.path.join(CSRC, s), os.path.join(tmp, s + ".o"), extra)
                    for s in SOURCES]
            for f in futs:
                objs.append(f.result())
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        os.replace(tmp_lib, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_host(out: str, sanitize: bool = True) -> str:
    """The host-only part of the library (page pool, scheduler, status codes)
    as a plain C++ shared library built by g++, with AddressSanitizer and
    UndefinedBehaviorSanitizer by default.  It exports the pool and scheduler
    entry points of include/pagedkv.h and nothing that touches a GPU; load it
    with PKV_HOST_LIBRARY=<out> and the ASan runtime preloaded."""
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", f"-I{os.path.join(ROOT, 'include')}",
           *(SANITIZE_FLAGS if sanitize else []), *srcs, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"host build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return out


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
