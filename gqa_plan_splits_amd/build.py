"""Builds libgqa_splits.so (the C-ABI library) in-tree with hipcc for gfx950.

Run ``python gqa_plan_splits_amd/build.py`` (or ``__graft_entry__.build()``).  The library
holds the host planner, the argument checks and the HIP kernels; nothing is JIT-compiled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqa_splits.so")
SOURCES = ["plan.cpp", "api.cpp", "mla_split.hip", "mla_wide.hip", "gqa_split.hip", "splitk_reduce.hip", "plan_device.hip", "scratch.hip", "ceiling.hip"]
HEADERS = ["kernels.hpp", "device_common.hpp", "mla_common.hpp"]
ARCH = "gfx950"

# -packed-fp32-ops: hipcc must not emit packed fp32 arithmetic (v_pk_*_f32) on its own.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    # code object v5: loadable by the HIP runtime torch ships (ROCm 7.0) as well as ROCm 7.2's
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into one shared library; always recompiles."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB)
    # the host pass does not know the gfx950 target feature; that warning is expected
    noise = "is not a recognized feature for this target"
    for line in (res.stdout + res.stderr).splitlines():
        if noise not in line and "(ignoring feature)" not in line and line.strip() and verbose:
            print(line)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
