"""The quantizers' block walks visit each 128x128 block exactly once, for the
shapes the launchers pick them for (host build of the walk header, no GPU)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_block_walks_are_permutations(tmp_path):
    from fp8_block_scaled_tile_amd import build as hip_build
    exe = str(tmp_path / "walk_check")
    subprocess.run([hip_build.hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "fp8_block_scaled_tile_amd", "csrc"),
                    os.path.join(HERE, "host", "walk_check.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout
