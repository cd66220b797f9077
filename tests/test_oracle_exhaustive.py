"""Exhaustive pin of the oracle's E4M3 encoder over all 2^32 binary32 bit
patterns (NaNs excluded) against an independent brute-force nearest-value
search built from the OCP E4M3 definition (tests/pins/e4m3_exhaustive.c)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_e4m3_encode_exhaustive(tmp_path):
    exe = tmp_path / "e4m3_exhaustive"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "pins", "e4m3_exhaustive.c"),
                    os.path.join(ROOT, "oracle", "puro_oracle.c"), "-lm", "-lpthread"],
                   check=True)
    threads = str(min(os.cpu_count() or 1, 16))
    out = subprocess.run([str(exe), threads], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "mismatches 0" in out.stdout
