"""Build libcoll.so (HIP kernels + C ABI) for gfx950 with hipcc, in tree.

Each source compiles to an object under _build/ in parallel, then one
link step produces libcoll.so next to this file.  Every invocation
recompiles (the build check must exercise the compiler).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcoll.so")

SOURCES = [
    "coll_api.cpp",
    "reduce_kernels.hip",
    "reduce_kernels_p3_7.hip",
    "reduce_kernels_p9_12.hip",
    "reduce_kernels_p13_15.hip",
    "reduce_trees_p3_7.hip",
    "reduce_trees_p9_12.hip",
    "reduce_trees_p13_15.hip",
    "copy_kernels.hip",
    "a2a_lds_kernels.hip",
    "ring_literal.hip",
    "batch_kernels.hip",
    "moe_kernels.hip",
    "fp8_kernels.hip",
    "probe_kernels.hip",
    "batch_noalloc.hip",
    "claim_slots.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcoll.so)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        # keep the compiler from emitting packed fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        "-Wall",
        "-Wno-unused-function",
    ]


# Device code flags.  The kernels read the result of a work-claiming atomic
# well after issuing it; LLVM's atomic optimizer would rewrite the atomic
# into a wave-wide one whose result is read, and waited for, at once.
DEVICE_FLAGS = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = DEVICE_FLAGS if src.endswith(".hip") else []
    cmd = [hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
