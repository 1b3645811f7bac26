"""The C ABI from plain C (tests/c/abi_check.c: include/kda.h and the HIP
runtime's C API only, no Python or torch): the fp32 forward on a batch, on
packed sequences with an empty and a one-token sequence, and four decode
steps, each against the fp64 C oracle linked into the same program (bar 1e-4).
The program is built with the library (tests/c/build.py); this test runs it
as a child process and checks its report."""
import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_check")


def test_c_program_through_the_abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "tests/c/abi_check is not built (__graft_entry__.build() builds it)"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "all cases ok" in r.stdout
    assert r.stdout.count(" ok") >= 4
