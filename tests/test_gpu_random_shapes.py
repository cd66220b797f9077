"""Seeded sweep over random ragged shapes, through the C ABI: quantizer codes
and scales bit-exact against the oracle, GEMM outputs within the gates of
tests/parity.py, in every mode, and the quantize-on-produce kernels (SwiGLU
forward and backward, RMSNorm) against the oracle's band.  Complements the hand-picked shapes of the
other GPU tests with shapes nobody chose (token counts from 1 to a few
thousand, every multiple of 128 for the feature dimensions in range)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from parity import random_bf16, say
from test_gpu_gemm import DGRAD, FWD, WGRAD, run_case
from test_gpu_quant import _check_act

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(2026)
ACT_CASES = [(int(_RNG.integers(1, 3000)), 128 * int(_RNG.integers(1, 25)),
              ("row", "col", "dual")[int(_RNG.integers(0, 3))]) for _ in range(12)]
WEIGHT_CASES = [(128 * int(_RNG.integers(1, 17)), 128 * int(_RNG.integers(1, 17))) for _ in range(6)]
GEMM_CASES = []
for mode in (FWD, DGRAD, WGRAD):
    for _ in range(4):
        T = int(_RNG.integers(1, 700))
        d_in, d_out = 128 * int(_RNG.integers(1, 11)), 128 * int(_RNG.integers(1, 11))
        if mode == WGRAD:
            out, acc = "fp32", bool(_RNG.integers(0, 2))
        else:
            out, acc = ("fp32", "bf16")[int(_RNG.integers(0, 2))], False
        GEMM_CASES.append((mode, T, d_in, d_out, out, acc))


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


@pytest.mark.parametrize("rows,cols,mode", ACT_CASES)
def test_quant_act_random(pf, rows, cols, mode):
    x = random_bf16((rows, cols), seed=rows * 31 + cols, stream=f"rand-act/{rows}x{cols}")
    _check_act(pf, x, row=mode in ("row", "dual"), col=mode in ("col", "dual"), tag="random")


@pytest.mark.parametrize("n,k", WEIGHT_CASES)
def test_quant_weight_random(pf, n, k):
    import oracle
    import synth
    from parity import dev, host
    w = random_bf16((n, k), std=0.02, seed=n * 7 + k, stream=f"rand-w/{n}x{k}")
    say("quant_weight random", n, k)
    out = pf.quant_weight(dev(w), transpose=True)
    q, qt, s = oracle.quant_weight(synth.bits(w))
    assert np.array_equal(host(out["q"]), q)
    assert np.array_equal(host(out["qt"]), qt)
    assert np.array_equal(host(out["s"]).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("mode,T,d_in,d_out,out,acc", GEMM_CASES)
def test_gemm_random(pf, mode, T, d_in, d_out, out, acc):
    run_case(pf, mode, T, d_in, d_out, torch.float32 if out == "fp32" else torch.bfloat16,
             seed=T + d_in + d_out, accumulate=acc)


# ---- quantize-on-produce: random ragged shapes --------------------------------

PRODUCE_CASES = [("swiglu_bwd" if i % 2 else "swiglu", int(_RNG.integers(1, 2500)),
                  128 * int(_RNG.integers(1, 13)), i % 4 < 2) for i in range(6)]
RMSNORM_CASES = [(int(_RNG.integers(1, 2500)), 128 * int(_RNG.integers(1, 65)),
                  (0.0, 1e-6, 1e-5)[int(_RNG.integers(0, 3))]) for _ in range(3)]


@pytest.mark.parametrize("op,rows,f,wide", PRODUCE_CASES)
def test_swiglu_random(pf, op, rows, f, wide):
    """Random ragged SwiGLU shapes, half of them with the gate spread over
    +-80 (the stated range of the error bound), against the oracle's band."""
    import oracle
    import produce_check as pc
    import synth
    from parity import dev
    from test_gpu_produce import TOL, _assert_ok, _host_outputs, _wide_gate
    say(op, "random", rows, f, "wide gate" if wide else "")
    if wide:
        gu, dh = _wide_gate(rows, f, seed=rows + f)
    else:
        d = synth.swiglu_inputs(rows, f, seed=rows + f)
        gu, dh = d["gu"], d["dh"]
    if op == "swiglu_bwd":
        out = pf.swiglu_bwd_quant(dev(dh), dev(gu), row=True, col=True, bf16_out=True)
        y, lo, hi = oracle.swiglu_bwd(synth.bits(dh), synth.bits(gu), TOL)
    else:
        out = pf.swiglu_quant(dev(gu), row=True, col=True, bf16_out=True)
        y, lo, hi = oracle.swiglu_fwd(synth.bits(gu), TOL)
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), f"{op} {rows}x{f}")


@pytest.mark.parametrize("rows,cols,eps", RMSNORM_CASES)
def test_rmsnorm_random(pf, rows, cols, eps):
    import oracle
    import produce_check as pc
    import synth
    from parity import dev, host
    from test_gpu_produce import TOL, _assert_ok, _host_outputs
    say("rmsnorm random", rows, cols, eps)
    d = synth.rmsnorm_inputs(rows, cols, seed=rows + cols)
    out = pf.rmsnorm_quant(dev(d["x"]), dev(d["gamma"]), eps=eps, row=True, col=True,
                           bf16_out=True)
    y, lo, hi, rstd = oracle.rmsnorm_fwd(synth.bits(d["x"]), synth.bits(d["gamma"]),
                                        float(np.float32(eps)), TOL)
    assert np.max(np.abs(host(out["rstd"]).astype(np.float64) - rstd) / rstd) <= TOL
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), f"rmsnorm {rows}x{cols}")
