"""puro_fp8_gemm_blockscaled_noalloc: the GEMM entry point that allocates
nothing (split-K partials in the library's static device array), called
through the C ABI and checked against puro_fp8_gemm_blockscaled with a
caller workspace on the same inputs: the same kernels run, so the outputs
must agree bit for bit.  Two calls in a row, the second on a smaller
problem, so the second reuses the array the first left behind."""
from __future__ import annotations

import pytest
import torch

from parity import say

pytestmark = pytest.mark.gpu
FWD, DGRAD, WGRAD, DGRAD_W, FWD_T = 0, 1, 2, 3, 4
B_KN = (DGRAD_W, FWD_T)          # b stored [K][N]
NAMES = ["fwd", "dgrad", "wgrad", "dgrad_w", "fwd_t"]
WORKSPACE = 5


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


def _operands(mode, M, N, K, seed):
    g = torch.Generator(device="cuda:0").manual_seed(seed)

    def codes(r, c):
        q = torch.randint(0, 0xFF, (r, c), dtype=torch.uint8, device="cuda:0", generator=g)
        return torch.where((q & 0x7F) == 0x7F, q - 1, q)          # no NaN codes

    sb_shape = {FWD: (N // 128, K // 128), DGRAD: (K // 128, N // 128), WGRAD: (K // 128, N),
                DGRAD_W: (K // 128, N // 128), FWD_T: (N // 128, K // 128)}[mode]
    sa = torch.rand((K // 128, M), device="cuda:0", generator=g) + 0.25
    sb = torch.rand(sb_shape, device="cuda:0", generator=g) + 0.25
    return codes(M, K), sa, (codes(K, N) if mode in B_KN else codes(N, K)), sb


def _noalloc(pf, mode, a, sa, b, sb, out, accumulate):
    M, K = a.shape
    N = b.shape[1] if mode in B_KN else b.shape[0]
    c_dtype = pf.OUT_FP32 if out.dtype == torch.float32 else pf.OUT_BF16
    return pf.puro_fp8_gemm_blockscaled_noalloc(
        mode, M, N, K, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), out.data_ptr(),
        c_dtype, 1 if accumulate else 0, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("cases", [
    # (mode, M, N, K, out dtype, accumulate): a split-K problem that fills the
    # whole array (4 splits x 2048 x 2048 FP32 = 64 MiB), then a smaller one
    [(WGRAD, 2048, 2048, 32768, torch.float32, False), (WGRAD, 1000, 1280, 8192, torch.float32, True)],
    # no split, then a split one with bf16 output, then a smaller split one
    [(FWD, 1000, 768, 512, torch.bfloat16, False), (FWD, 256, 2048, 4096, torch.bfloat16, False),
     (DGRAD, 129, 256, 2048, torch.float32, False)],
    # the modes that read the weight codes as [K][N]: split-K, then smaller
    [(DGRAD_W, 300, 512, 4096, torch.bfloat16, False), (FWD_T, 200, 384, 2048, torch.float32, False)],
])
def test_noalloc_matches_workspace_entry_point(pf, cases):
    for i, (mode, M, N, K, dt, acc) in enumerate(cases):
        ws_need = pf.puro_fp8_gemm_workspace_bytes(mode, M, N, K)
        say("noalloc", NAMES[mode], M, N, K, dt, "acc" if acc else "",
            f"workspace {ws_need} B")
        assert ws_need <= pf.PURO_FP8_NOALLOC_SCRATCH_BYTES
        a, sa, b, sb = _operands(mode, M, N, K, 100 + i)
        c0 = torch.randn((M, N), device="cuda:0").to(dt) if acc else None
        want = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=dt,
                                   out=None if c0 is None else c0.clone(), accumulate=acc)
        got = torch.full((M, N), float("nan"), dtype=dt, device="cuda:0") if c0 is None else c0.clone()
        assert _noalloc(pf, mode, a, sa, b, sb, got, acc) == 0
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), \
            f"case {i}: {int((got != want).sum())} elements differ"


def test_noalloc_rejects_problems_beyond_the_array(pf):
    """A split-K problem whose partials need more than the array is refused
    before anything is enqueued (5 splits x 2560 x 2560 FP32 = 131 MB)."""
    M = N = 2560
    K = 8192
    need = pf.puro_fp8_gemm_workspace_bytes(WGRAD, M, N, K)
    assert need > pf.PURO_FP8_NOALLOC_SCRATCH_BYTES
    a, sa, b, sb = _operands(WGRAD, M, N, K, 7)
    out = torch.zeros((M, N), dtype=torch.float32, device="cuda:0")
    assert _noalloc(pf, WGRAD, a, sa, b, sb, out, False) == WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()
