"""The C ABI from a plain host program (tests/c_abi/abi_consumer.cpp): HIP
runtime allocations, no Python or PyTorch in the process.  It quantizes a
small ragged linear layer's X, W and dY, runs FWD and WGRAD with FP32 output
and DGRAD with bf16 output on a stream of its own, and checks codes and
scales bit-exact and the GEMMs within relative Frobenius 1e-3 against the CPU
oracle (the bf16 output against the oracle's result rounded to bf16)."""
from __future__ import annotations

import os
import runpy
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "abi_consumer")


def test_plain_host_program_through_the_c_abi():
    if not os.path.exists(EXE):     # normally built by build(); build it once if absent
        runpy.run_path(os.path.join(HERE, "c_abi", "build.py"))["build"]()
    print("running", EXE, flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_consumer ok" in r.stdout
