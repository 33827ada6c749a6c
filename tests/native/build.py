"""Builds tests/native/decode_abi, a C++ program that calls the C ABI with no Python in the process
(run by tests/test_gpu_native.py).  Needs libgqa_splits.so and oracle/liboracle.so built first;
both are found through the program's rpath, relative to its own location."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "decode_abi")


def build(verbose: bool = False) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "decode_abi.cpp"),
           "-L", os.path.join(ROOT, "gqa_plan_splits_amd"), "-lgqa_splits",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-Wl,-rpath,$ORIGIN/../../gqa_plan_splits_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-o", BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % BIN)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
