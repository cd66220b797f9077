"""The BF16 comparator GEMM (C = A . B^T on bf16 operands with the FP8
path's tiling, no block scales), used only to measure the FP8 / BF16 speedup
kernel for kernel.  Checked against the exact product of the same bf16 values
(float64): relative Frobenius error <= 1e-3 against that product rounded to
bf16, and every element within bf16 rounding plus an accumulation allowance.
Covers ragged M, a half-inactive last tile column, several tiles per
work-group and the split-K path."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from parity import dev, host, random_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


def _bf16_round(x):
    """float64 -> nearest bf16 (ties to even), as float64."""
    f = x.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M,N,K", [
    (300, 384, 512),      # ragged M, one round
    (256, 256, 8192),     # one tile, long K: split-K and the reduce
    (4000, 1152, 1024),   # ragged M, N % 256 == 128, split
    (20000, 1152, 512),   # more tiles than CUs: several units per work-group
])
def test_bf16_comparator_matches_exact_product(pf, M, N, K):
    a = random_bf16((M, K), seed=M + K, stream=f"bf16cmp/a/{M}x{K}")
    b = random_bf16((N, K), seed=N + K, stream=f"bf16cmp/b/{N}x{K}")
    say("bf16 comparator", M, N, K, "workspace", pf.puro_bf16_gemm_nt_workspace_bytes(M, N, K))
    c = host(pf.gemm_bf16_nt(dev(a), dev(b)).float()).astype(np.float64)
    A = a.float().numpy().astype(np.float64)
    B = b.float().numpy().astype(np.float64)
    R = A @ B.T
    ref = _bf16_round(R)
    rel = np.linalg.norm(c - ref) / max(np.linalg.norm(ref), 1e-30)
    mag = np.abs(A) @ np.abs(B).T
    bound = 2.0 ** -8 * np.abs(R) + 2.0 ** -16 * mag + 1e-30
    worst = float(np.max(np.abs(c - R) / bound))
    say(f"   rel_fro {rel:.3e}  worst err/bound {worst:.3f}")
    assert rel <= 1e-3
    assert worst <= 1.0
