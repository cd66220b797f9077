"""Host logic of bench.py: the step enqueues every layer's own launches, in
order, with that layer's shapes (checked with a stand-in binding, no GPU)."""
from __future__ import annotations

import types

import bench


class _Buf:
    def data_ptr(self):
        return 0

    def numel(self):
        return 16


def _layer(name, T, din, dout):
    L = types.SimpleNamespace(spec=types.SimpleNamespace(name=name), T=T, Tp=T, din=din, dout=dout)
    for a in ("x", "qx", "sx", "qtx", "stx", "w", "qw", "qtw", "sw", "y", "dy", "qdy", "sdy",
              "qtdy", "stdy", "dx", "dw", "ws"):
        setattr(L, a, _Buf())
    L.gemms = [("gemm_fwd_bf16", 0, T, dout, din), ("gemm_dgrad_bf16", 1, T, din, dout),
               ("gemm_wgrad_fp32", 2, dout, din, T)]
    return L


def test_step_calls_bind_each_layer():
    seen = []
    pf = types.SimpleNamespace(
        GEMM_FWD=0, GEMM_DGRAD=1, GEMM_WGRAD=2, OUT_BF16=0, OUT_FP32=1,
        puro_fp8_quant_act=lambda x, r, c, *a: seen.append(("act", r, c)) or 0,
        puro_fp8_quant_weight=lambda w, n, k, *a: seen.append(("weight", n, k)) or 0,
        puro_fp8_gemm_blockscaled=lambda m, M, N, K, *a: seen.append(("gemm", m, M, N, K)) or 0)
    layers = [_layer("a", 256, 128, 384), _layer("b", 512, 256, 128)]
    calls = bench.step_calls(pf, layers, None)
    assert [c[0] for c in calls] == ["a"] * 6 + ["b"] * 6
    for _, _, _, fn in calls:
        assert fn() == 0
    expect = []
    for T, din, dout in ((256, 128, 384), (512, 256, 128)):
        expect += [("act", T, din), ("weight", dout, din), ("gemm", 0, T, dout, din),
                   ("act", T, dout), ("gemm", 1, T, din, dout), ("gemm", 2, dout, din, T)]
    assert seen == expect
    works = [c[2] for c in calls]
    assert works[2] == 2.0 * 256 * 384 * 128 and works[8] == 2.0 * 512 * 128 * 256
