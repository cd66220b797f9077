"""Seeded sweep over random ragged shapes, through the C ABI: quantizer codes
and scales bit-exact against the oracle, GEMM outputs within the gates of
tests/parity.py, in every mode -- including shapes that take the split-K path
(K >= 2048 with fewer than 256 output tiles) and the persistent multi-unit
walk (more than 256 tiles) -- and the quantize-on-produce kernels (SwiGLU
forward and backward, RMSNorm forward and backward, the residual add) against
the oracle's band.  Complements the
hand-picked shapes of the other GPU tests with shapes nobody chose."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from parity import random_bf16, say
from test_gpu_gemm import (B_KN, DGRAD, DGRAD_W, FWD, FWD_T, MODE_NAMES, ORACLE_MODE, WGRAD,
                           device_operands, device_values, make_inputs, oracle_operands,
                           run_case)
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


# split-K (K >= 16 K-blocks, fewer than 256 output tiles) in every mode, and
# the persistent multi-unit walk (more than 256 output tiles)
SPLITK_CASES = []
for mode in (FWD, DGRAD, WGRAD, DGRAD_W, FWD_T):
    if mode == WGRAD:
        T = int(_RNG.integers(2048, 4200))
        d_in, d_out = 128 * int(_RNG.integers(1, 9)), 128 * int(_RNG.integers(1, 9))
    else:
        T = int(_RNG.integers(1, 1500))
        k_dim, n_dim = 128 * int(_RNG.integers(16, 41)), 128 * int(_RNG.integers(1, 9))
        d_in, d_out = (k_dim, n_dim) if mode in (FWD, FWD_T) else (n_dim, k_dim)
    SPLITK_CASES.append((mode, T, d_in, d_out, ("fp32", "bf16")[int(_RNG.integers(0, 2))]))
MULTI_CASES = []
for mode in (FWD, DGRAD, WGRAD, DGRAD_W, FWD_T):
    if mode == WGRAD:     # M = d_out, N = d_in: > 256 tiles; K = T
        T = int(_RNG.integers(1, 700))
        d_in, d_out = 128 * int(_RNG.integers(34, 48)), 128 * int(_RNG.integers(34, 48))
    else:                 # M = T, N = d_out (FWD) or d_in (DGRAD)
        T = int(_RNG.integers(8300, 12000))
        n_dim, k_dim = 128 * int(_RNG.integers(17, 40)), 128 * int(_RNG.integers(1, 9))
        d_in, d_out = (k_dim, n_dim) if mode in (FWD, FWD_T) else (n_dim, k_dim)
    MULTI_CASES.append((mode, T, d_in, d_out, ("fp32", "bf16")[int(_RNG.integers(0, 2))]))


def _mnk(mode, T, d_in, d_out):
    if mode in (FWD, FWD_T):
        return T, d_out, d_in
    if mode in (DGRAD, DGRAD_W):
        return T, d_in, d_out
    return d_out, d_in, (T + 127) // 128 * 128


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


@pytest.mark.parametrize("rows,cols,mode", ACT_CASES)
def test_quant_act_random(pf, rows, cols, mode):
    x = random_bf16((rows, cols), seed=rows * 31 + cols, stream=f"rand-act/{rows}x{cols}")
    _check_act(pf, x, row=mode in ("row", "dual"), col=mode in ("col", "dual"), tag="random")


# shapes the launcher sends down the XCD-tiled block walk: 4x4-block tiles per
# XCD, stacked 2 high (32-63 block columns, a multiple of 16) or 1 high (64+,
# a multiple of 32), with a whole number of super tiles of block rows and a
# ragged last block row
_XRNG = np.random.default_rng(4096)
XCD_ACT_CASES = []
for _ in range(8):
    ncb = int(_XRNG.choice([32, 48, 64, 96, 128, 160]))
    nrb = (4 if ncb >= 64 else 8) * int(_XRNG.integers(1, 4))
    XCD_ACT_CASES.append((128 * nrb - int(_XRNG.integers(0, 128)), 128 * ncb,
                          ("row", "col", "dual")[int(_XRNG.integers(0, 3))]))


@pytest.mark.parametrize("rows,cols,mode", XCD_ACT_CASES)
def test_quant_act_random_xcd_walk(pf, rows, cols, mode):
    x = random_bf16((rows, cols), seed=rows * 37 + cols, stream=f"rand-xcd/{rows}x{cols}")
    _check_act(pf, x, row=mode in ("row", "dual"), col=mode in ("col", "dual"), tag="random xcd walk")


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


@pytest.mark.parametrize("mode,T,d_in,d_out,out", SPLITK_CASES)
def test_gemm_random_split_k(pf, mode, T, d_in, d_out, out):
    M, N, K = _mnk(mode, T, d_in, d_out)
    assert (M + 255) // 256 * ((N + 255) // 256) < 256 and K >= 2048
    assert pf.puro_fp8_gemm_workspace_bytes(mode, M, N, K) > 0      # the split-K path
    run_case(pf, mode, T, d_in, d_out, torch.float32 if out == "fp32" else torch.bfloat16,
             seed=T + d_in + d_out)


@pytest.mark.parametrize("mode,T,d_in,d_out,out", MULTI_CASES)
def test_gemm_random_multi_unit(pf, mode, T, d_in, d_out, out):
    """More output tiles than compute units, through the linear-layer path:
    device codes bit-exact, outputs on sampled elements plus whole first and
    last rows and the last column."""
    import hw_accum
    import oracle
    from parity import fmt, gemm_gates, host
    M, N, K = _mnk(mode, T, d_in, d_out)
    assert (M + 255) // 256 * ((N + 255) // 256) > 256
    assert pf.puro_fp8_gemm_workspace_bytes(mode, M, N, K) == 0
    x, w, dy = make_inputs(T, d_in, d_out, T + d_in + d_out)
    say("gemm multi-unit", MODE_NAMES[mode], f"T={T} in={d_in} out={d_out}", out)
    a, sa, b, sb = device_operands(pf, mode, x, w, dy)
    out_dtype = torch.float32 if out == "fp32" else torch.bfloat16
    c = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=out_dtype)
    oa, osa, ob, osb = oracle_operands(mode, x, w, dy)
    assert np.array_equal(host(a), oa)
    assert np.array_equal(host(b).T if mode in B_KN else host(b), ob)
    rng = np.random.default_rng(M + N)
    ii = np.concatenate([rng.integers(0, M, 6000), np.zeros(N, np.int64), np.full(N, M - 1),
                         np.arange(M)])
    jj = np.concatenate([rng.integers(0, N, 6000), np.arange(N), np.arange(N),
                         np.full(M, N - 1)])
    omode = ORACLE_MODE[mode]
    ref = oracle.gemm_blockscaled_at(omode, oa, osa, ob, osb, ii, jj)
    bound = hw_accum.bounds(omode, oa, osa, ob, osb, ii, jj, ref)
    g = gemm_gates(device_values(c)[ii, jj], ref, bound, out_dtype == torch.bfloat16,
                   literal=omode != FWD)
    say("   " + fmt(g))
    assert g["ok"], g


# ---- quantize-on-produce: random ragged shapes --------------------------------

PRODUCE_CASES = [("swiglu_bwd" if i % 2 else "swiglu", int(_RNG.integers(1, 2500)),
                  128 * int(_RNG.integers(1, 13)), i % 4 < 2) for i in range(6)]
RMSNORM_CASES = [(int(_RNG.integers(1, 2500)), 128 * int(_RNG.integers(1, 65)),
                  (0.0, 1e-6, 1e-5)[int(_RNG.integers(0, 3))]) for _ in range(3)]


NORM_BWD_CASES = [(int(_RNG.integers(1, 2500)), 128 * int(_RNG.integers(1, 33)),
                   bool(_RNG.integers(0, 2))) for _ in range(4)] + [(1, 128, True)]
RESIDUAL_CASES = [(int(_RNG.integers(1, 2500)), 128 * int(_RNG.integers(1, 33))) for _ in range(3)] + [(1, 256)]


@pytest.mark.parametrize("rows,cols,skip", NORM_BWD_CASES)
def test_rmsnorm_bwd_random(pf, rows, cols, skip):
    """Random ragged RMSNorm-backward shapes (with and without the skip-path
    gradient) against the oracle's band."""
    import oracle
    import produce_check as pc
    import synth
    from parity import dev
    from test_gpu_produce import _assert_ok, _host_outputs, _tol_bwd
    say("rmsnorm_bwd random", rows, cols, skip)
    d = synth.rmsnorm_bwd_inputs(rows, cols, seed=rows + cols)
    rstd = torch.from_numpy(oracle.rmsnorm_fwd(synth.bits(d["x"]), synth.bits(d["gamma"]), 1e-6,
                                               2.0 ** -18)[3].astype(np.float32))
    gin = d["gin"] if skip else None
    out = pf.rmsnorm_bwd_quant(dev(d["dy"]), dev(d["x"]), dev(d["gamma"]), dev(rstd),
                               None if gin is None else dev(gin), row=True, col=True,
                               bf16_out=True)
    y, lo, hi = oracle.rmsnorm_bwd(synth.bits(d["dy"]), synth.bits(d["x"]), synth.bits(d["gamma"]),
                                   rstd.numpy(), None if gin is None else synth.bits(gin),
                                   _tol_bwd(cols))
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), f"rmsnorm_bwd {rows}x{cols}")


@pytest.mark.parametrize("rows,cols", RESIDUAL_CASES)
def test_residual_add_then_norm_random(pf, rows, cols):
    """Random ragged residual add + one-pass norm: h bit-exact, rstd within
    TOL, the norm's outputs within the oracle's band."""
    import oracle
    import produce_check as pc
    import synth
    from parity import bf16_host_bits, dev, host
    from test_gpu_produce import TOL, _assert_ok, _host_outputs
    say("residual + norm random", rows, cols)
    d = synth.residual_inputs(rows, cols, seed=rows + cols)
    r = pf.residual_add_rstd(dev(d["a"]), dev(d["b"]), eps=1e-6)
    h = oracle.residual_add(synth.bits(d["a"]), synth.bits(d["b"]))
    assert np.array_equal(bf16_host_bits(r["h"]), h)
    y, lo, hi, rstd = oracle.rmsnorm_fwd(h, synth.bits(d["gamma"]), float(np.float32(1e-6)), TOL)
    assert np.max(np.abs(host(r["rstd"]).astype(np.float64) - rstd) / rstd) <= TOL
    out = pf.rmsnorm_quant_rstd(r["h"], dev(d["gamma"]), r["rstd"], row=True, col=True,
                                bf16_out=True)
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), f"residual {rows}x{cols}")


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
