"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a
program (tests/pins/oracle_sanitize.c) calls every entry point of
oracle/puro_oracle.c on small and edge-case inputs (ragged rows, zero and
tiny tiles, all three GEMM modes, the neighbour ops); any out-of-bounds
access or undefined behaviour aborts it.  Built with gcc, run on the CPU."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the sanitizer program")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
                    "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "pins", "oracle_sanitize.c"),
                    os.path.join(ROOT, "oracle", "puro_oracle.c"),
                    "-o", exe, "-lm", "-lpthread"], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "oracle sanitize: ok" in r.stdout
