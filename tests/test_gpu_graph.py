"""One linear layer's launches (quantizers, FWD, DGRAD from the weight's
codes, split-K WGRAD with a caller workspace and with the allocation-free
entry point) captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.
The library allocates, clears and synchronizes nothing, so its calls can be
captured; every replay must reproduce the eager results bit for bit, with
eager work and synchronizations between the replays, and after the inputs
change in place."""
from __future__ import annotations

import pytest
import torch

from parity import say

pytestmark = pytest.mark.gpu
FWD, DGRAD, WGRAD, DGRAD_W = 0, 1, 2, 3
OUT_BF16, OUT_FP32 = 0, 1


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


def _p(t):
    return t.data_ptr()


def test_layer_launches_replay_in_a_graph(pf):
    T, din, dout = 4096, 1024, 512             # WGRAD 512 x 1024 x 4096: split 4 ways
    assert pf.puro_fp8_gemm_workspace_bytes(WGRAD, dout, din, T) > 0
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(11)
    x = torch.randn((T, din), device=dev, generator=g).to(torch.bfloat16)
    dy = (torch.randn((T, dout), device=dev, generator=g) * 1e-3).to(torch.bfloat16)
    w = (torch.randn((dout, din), device=dev, generator=g) * 0.02).to(torch.bfloat16)
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    E = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    qx, sx, qtx, stx = E((T, din), u8), E((din // 128, T), f32), E((din, T), u8), E((T // 128, din), f32)
    qdy, sdy = E((T, dout), u8), E((dout // 128, T), f32)
    qtdy, stdy = E((dout, T), u8), E((T // 128, dout), f32)
    qw, sw = E((dout, din), u8), E((dout // 128, din // 128), f32)
    y, dx = E((T, dout), bf), E((T, din), bf)
    dw, dw_na = E((dout, din), f32), E((dout, din), f32)
    ws_bytes = pf.puro_fp8_gemm_workspace_bytes(WGRAD, dout, din, T)
    ws = E((ws_bytes,), u8)
    outs = (qx, sx, qtx, stx, qdy, sdy, qtdy, stdy, qw, sw, y, dx, dw, dw_na)

    def step():
        st = torch.cuda.current_stream().cuda_stream
        rc = [pf.puro_fp8_quant_act(_p(x), T, din, _p(qx), _p(sx), _p(qtx), _p(stx), st),
              pf.puro_fp8_quant_weight(_p(w), dout, din, _p(qw), None, _p(sw), st),
              pf.puro_fp8_gemm_blockscaled(FWD, T, dout, din, _p(qx), _p(sx), _p(qw), _p(sw),
                                           _p(y), OUT_BF16, 0, None, 0, st),
              pf.puro_fp8_quant_act(_p(dy), T, dout, _p(qdy), _p(sdy), _p(qtdy), _p(stdy), st),
              pf.puro_fp8_gemm_blockscaled(DGRAD_W, T, din, dout, _p(qdy), _p(sdy), _p(qw), _p(sw),
                                           _p(dx), OUT_BF16, 0, None, 0, st),
              pf.puro_fp8_gemm_blockscaled(WGRAD, dout, din, T, _p(qtdy), _p(stdy), _p(qtx), _p(stx),
                                           _p(dw), OUT_FP32, 0, _p(ws), ws_bytes, st),
              pf.puro_fp8_gemm_blockscaled_noalloc(WGRAD, dout, din, T, _p(qtdy), _p(stdy), _p(qtx),
                                                   _p(stx), _p(dw_na), OUT_FP32, 0, st)]
        assert rc == [0] * len(rc), rc

    def eager_reference():
        for o in outs:
            o.zero_()
        step()
        torch.cuda.synchronize()
        return [o.clone() for o in outs]

    say("graph capture: one layer", T, din, dout)
    ref = eager_reference()             # also the first call of the allocation-free entry point
    assert torch.equal(ref[12], ref[13])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    def check_replays(expect, n=3):
        for i in range(n):
            for o in outs:                       # eager fills between the replays
                o.zero_()
            torch.cuda.synchronize()
            _ = (torch.randn(512, 512, device=dev) @ torch.randn(512, 512, device=dev)).sum().item()
            graph.replay()
            torch.cuda.synchronize()
            for k, (got, exp) in enumerate(zip(outs, expect)):
                assert torch.equal(got, exp), f"replay {i}: output {k} differs from the eager result"

    check_replays(ref)
    # new inputs in place: the replays follow them
    x.copy_((torch.randn((T, din), device=dev, generator=g) * 3).to(bf))
    dy.copy_((torch.randn((T, dout), device=dev, generator=g) * 1e-2).to(bf))
    w.copy_((torch.randn((dout, din), device=dev, generator=g) * 0.05).to(bf))
    ref2 = eager_reference()
    assert not torch.equal(ref2[10], ref[10])
    check_replays(ref2)
