"""Build libmoe_mi355x.so (hand-written HIP for gfx950) in the package folder.

    python -m sparse_mixture_experts_rmsnorm_amd.csrc.build

Compiles every source with hipcc in parallel (objects under
sparse_mixture_experts_rmsnorm_amd/_build/), then links the shared library
next to the Python binding.  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

HERE = Path(__file__).resolve().parent
PKG = HERE.parent
ROOT = PKG.parent
BUILD = PKG / "_build"
LIB = PKG / "libmoe_mi355x.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["router.hip", "dispatch.hip", "topology.hip", "gemm.hip", "gemm_mx.hip", "combine.hip",
           "atomic.hip", "backward.hip", "noalloc.hip", "api.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{ROOT / 'include'}", f"-I{HERE}",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
# gfx950 only; packed-fp32 instructions are turned off in the device pass.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> Path:
    obj = BUILD / (src + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-c", str(HERE / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None) -> Path:
    BUILD.mkdir(exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
