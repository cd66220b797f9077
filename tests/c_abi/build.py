"""Build tests/c_abi/abi_consumer: a plain host program that uses the C ABI of
libpuro_fp8.so (HIP runtime for device memory) and checks it against the CPU
oracle.  Test infrastructure: it links the oracle, so it lives with the tests."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_consumer.cpp")
EXE = os.path.join(HERE, "abi_consumer")


def build() -> str:
    sys.path.insert(0, ROOT)
    from fp8_block_scaled_tile_amd import build as hip_build
    import oracle
    oracle.build(force=False)
    pkg = os.path.join(ROOT, "fp8_block_scaled_tile_amd")
    odir = os.path.join(ROOT, "oracle")
    tmp = EXE + ".tmp"
    cmd = [hip_build.hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", odir, SRC, "-o", tmp,
           "-L", pkg, "-lpuro_fp8", "-L", odir, "-lpuro_oracle",
           "-Wl,-rpath,$ORIGIN/../../fp8_block_scaled_tile_amd:$ORIGIN/../../oracle"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
