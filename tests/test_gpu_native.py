"""The C ABI driven from a C++ program with no Python in its process (tests/native/decode_abi.cpp):
MLA over fp8 and bf16 pools and paged GQA, each through decode() at the planner's np and at np = 3,
against the fp64 oracle linked into the same program.  The program is built with the library
(python tests/native/build.py, also run by __graft_entry__.build())."""
import os
import subprocess

import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "decode_abi")


def test_native_program_through_the_c_abi():
    if not os.path.exists(BIN):
        pytest.skip("tests/native/decode_abi is not built (python tests/native/build.py)")
    # a child process of its own (it initializes the GPU itself)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all cases pass" in res.stdout
