"""GPU parity of quantize-on-produce (SwiGLU forward and backward, RMSNorm
forward, each writing FP8 operands straight from the op) against the CPU
oracle.  Calls go through the C ABI.

The oracle evaluates the op in double and rounds once to bf16; the device
evaluates it in FP32 and may return any bf16 value within its error bound,
TOL * M, of the exact one (the bound the C header states).  produce_check
compares every tile bit for bit where it has one correct result, and checks
the others against every correct (scale, codes).

The band holds, besides TOL * M, the FP32 subnormal spacing 2^-149 (a
result below the normal range is rounded to it whatever its relative bound).

Sizes: small cases span several tiles and a ragged last row block; the
block-stack sizes (32768 tokens, FFN 8192, hidden 2048) run in the launch
configuration the benchmark uses and are checked on sampled row blocks
(each row block fixes its 1x128 and 128x1 tiles completely)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import produce_check as pc
import synth
from parity import bf16_host_bits, dev, host, say

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -18


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


def _host_outputs(out, rows=None, row_sel=None, rb_sel=None):
    """Host copies of the device outputs; with row_sel / rb_sel only the
    sampled rows (row codes and scales) and row blocks (transposed codes and
    scales)."""
    h = {}
    if "y" in out:
        y = out["y"] if row_sel is None else out["y"][row_sel]
        h["y"] = bf16_host_bits(y)
    if "q" in out:
        h["q"] = host(out["q"] if row_sel is None else out["q"][row_sel])
        h["s"] = host(out["s"] if row_sel is None else out["s"][:, row_sel])
    if "qt" in out:
        if rb_sel is None:
            h["qt"] = host(out["qt"])
            h["st"] = host(out["st"])
        else:
            cols_idx = torch.cat([torch.arange(128 * rb, 128 * rb + 128) for rb in rb_sel])
            h["qt"] = host(out["qt"][:, cols_idx.to(out["qt"].device)])
            h["st"] = host(out["st"][list(rb_sel)])
    return h


def _same(a, b):
    """Bitwise equality of two device tensors of the same dtype and shape."""
    return a.dtype == b.dtype and a.shape == b.shape and torch.equal(
        a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _assert_ok(res, what):
    assert pc.all_ok(res), f"{what}: {res}"
    say(what, "ok", {k: (v if not isinstance(v, dict) else
                         {kk: (len(vv) if kk == 'bad' else vv) for kk, vv in v.items()})
                     for k, v in res.items()})


# ---- SwiGLU forward ------------------------------------------------------------

@pytest.mark.parametrize("rows,f", [(1, 128), (200, 384), (384, 256), (1100, 640)])
def test_swiglu_fwd_parity(pf, rows, f):
    say("swiglu_quant", rows, f)
    gu = synth.swiglu_inputs(rows, f, seed=rows + f, need=("gu",))["gu"]
    out = pf.swiglu_quant(dev(gu), row=True, col=True, bf16_out=True)
    y, lo, hi = oracle.swiglu_fwd(synth.bits(gu), TOL)
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), f"swiglu {rows}x{f}")


def test_swiglu_fwd_output_subsets(pf):
    """Each subset of outputs equals the same outputs of the all-output call."""
    rows, f = 300, 256
    gu = dev(synth.swiglu_inputs(rows, f, seed=5, need=("gu",))["gu"])
    say("swiglu_quant subsets", rows, f)
    full = pf.swiglu_quant(gu, row=True, col=True, bf16_out=True)
    for row, col, yb in [(True, False, False), (False, True, False), (False, False, True),
                         (True, True, False), (True, False, True), (False, True, True)]:
        part = pf.swiglu_quant(gu, row=row, col=col, bf16_out=yb)
        for k, v in part.items():
            assert _same(v, full[k]), (k, row, col, yb)


def _wide_gate(rows, f, seed):
    """gate | up with the gate spread over [-80, 80] and, in every fifth row,
    over [-104, -64] (where sigmoid(gate) is below 2^-92 and the results head
    for the subnormal range), up ~ N(0, 1)."""
    d = synth.swiglu_inputs(rows, f, seed=seed)
    gu = d["gu"].float()
    gu[:, :f] = (gu[:, :f] * 8.0).clamp(-80.0, 80.0)
    deep = torch.linspace(-104.0, -64.0, f)
    gu[::5, :f] = deep[torch.randperm(f, generator=torch.Generator().manual_seed(seed))]
    return gu.to(torch.bfloat16), d["dh"]


def test_swiglu_fwd_wide_gate(pf):
    rows, f = 300, 256
    gu, _ = _wide_gate(rows, f, seed=12)
    say("swiglu_quant wide gate", rows, f, float(gu[:, :f].float().abs().max()))
    out = pf.swiglu_quant(dev(gu), row=True, col=True, bf16_out=True)
    y, lo, hi = oracle.swiglu_fwd(synth.bits(gu), TOL)
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), "swiglu wide gate")


def test_swiglu_bwd_wide_gate(pf):
    rows, f = 300, 256
    gu, dh = _wide_gate(rows, f, seed=13)
    say("swiglu_bwd_quant wide gate", rows, f)
    out = pf.swiglu_bwd_quant(dev(dh), dev(gu), row=True, col=True, bf16_out=True)
    y, lo, hi = oracle.swiglu_bwd(synth.bits(dh), synth.bits(gu), TOL)
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), "swiglu_bwd wide gate")


# ---- SwiGLU backward -----------------------------------------------------------

# (1000, 4096): the XCD-tiled block walk (32 block columns, 8 block rows)
@pytest.mark.parametrize("rows,f", [(130, 128), (256, 256), (700, 384), (1000, 4096)])
def test_swiglu_bwd_parity(pf, rows, f):
    say("swiglu_bwd_quant", rows, f)
    d = synth.swiglu_inputs(rows, f, seed=3 * rows + f)
    out = pf.swiglu_bwd_quant(dev(d["dh"]), dev(d["gu"]), row=True, col=True, bf16_out=True)
    y, lo, hi = oracle.swiglu_bwd(synth.bits(d["dh"]), synth.bits(d["gu"]), TOL)
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), f"swiglu_bwd {rows}x{f}")


@pytest.mark.parametrize("row,col", [(True, False), (False, True)])
def test_swiglu_bwd_single_orientation(pf, row, col):
    rows, f = 200, 256
    d = synth.swiglu_inputs(rows, f, seed=9)
    say("swiglu_bwd_quant single", row, col)
    out = pf.swiglu_bwd_quant(dev(d["dh"]), dev(d["gu"]), row=row, col=col)
    y, lo, hi = oracle.swiglu_bwd(synth.bits(d["dh"]), synth.bits(d["gu"]), TOL)
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), "swiglu_bwd single")


# ---- RMSNorm forward -------------------------------------------------------------

# (1000, 4096) and (500, 8192) take the XCD-tiled block walk
@pytest.mark.parametrize("rows,cols,eps", [(77, 128, 1e-6), (256, 2048, 1e-5),
                                           (130, 8192, 0.0), (1000, 384, 1e-6),
                                           (1000, 4096, 1e-6), (500, 8192, 1e-5)])
def test_rmsnorm_parity(pf, rows, cols, eps):
    say("rmsnorm_quant", rows, cols, eps)
    d = synth.rmsnorm_inputs(rows, cols, seed=rows + cols)
    out = pf.rmsnorm_quant(dev(d["x"]), dev(d["gamma"]), eps=eps, row=True, col=True,
                           bf16_out=True)
    y, lo, hi, rstd = oracle.rmsnorm_fwd(synth.bits(d["x"]), synth.bits(d["gamma"]),
                                        float(np.float32(eps)), TOL)
    got_rstd = host(out["rstd"]).astype(np.float64)
    assert np.max(np.abs(got_rstd - rstd) / rstd) <= TOL
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows), f"rmsnorm {rows}x{cols}")


# ---- fused equals unfused ----------------------------------------------------------

@pytest.mark.parametrize("op", ["swiglu", "swiglu_bwd", "rmsnorm"])
def test_fused_codes_equal_quant_act_of_the_bf16_output(pf, op):
    """The fused kernel's codes and scales are bit for bit those of the plain
    activation quantizer applied to the same kernel's bf16 output."""
    rows, f = 513, 256
    say("fused vs unfused", op, rows, f)
    if op == "swiglu":
        out = pf.swiglu_quant(dev(synth.swiglu_inputs(rows, f, seed=1, need=("gu",))["gu"]),
                              bf16_out=True)
    elif op == "swiglu_bwd":
        d = synth.swiglu_inputs(rows, f, seed=2)
        out = pf.swiglu_bwd_quant(dev(d["dh"]), dev(d["gu"]), bf16_out=True)
    else:
        d = synth.rmsnorm_inputs(rows, 4 * f, seed=3)
        out = pf.rmsnorm_quant(dev(d["x"]), dev(d["gamma"]), bf16_out=True)
    ref = pf.quant_act(out["y"], row=True, col=True)
    for k in ("q", "s", "qt", "st"):
        assert _same(out[k], ref[k]), k


# ---- block-stack sizes, sampled ------------------------------------------------------

SAMPLE_RBS = (0, 97, 255)          # first, an inner and the last 128-row block of 32768


def _sample_rows():
    return torch.cat([torch.arange(128 * rb, 128 * rb + 128) for rb in SAMPLE_RBS])


def test_swiglu_fwd_block_stack_sampled(pf):
    rows, f = 32768, 8192
    say("swiglu_quant block_stack", rows, f)
    gu = synth.swiglu_inputs(rows, f, seed=0, need=("gu",))["gu"]
    out = pf.swiglu_quant(dev(gu), row=True, col=True)
    sel = _sample_rows()
    h = _host_outputs(out, row_sel=sel.to("cuda:0"), rb_sel=SAMPLE_RBS)
    y, lo, hi = oracle.swiglu_fwd(synth.bits(gu[sel]), TOL)
    _assert_ok(pc.check_outputs(h, y, lo, hi, sel.numel()), "swiglu block_stack")


def test_swiglu_bwd_block_stack_sampled(pf):
    rows, f = 32768, 8192
    say("swiglu_bwd_quant block_stack", rows, f)
    d = synth.swiglu_inputs(rows, f, seed=0)
    out = pf.swiglu_bwd_quant(dev(d["dh"]), dev(d["gu"]), row=True, col=True)
    sel = _sample_rows()
    h = _host_outputs(out, row_sel=sel.to("cuda:0"), rb_sel=SAMPLE_RBS)
    y, lo, hi = oracle.swiglu_bwd(synth.bits(d["dh"][sel]), synth.bits(d["gu"][sel]), TOL)
    _assert_ok(pc.check_outputs(h, y, lo, hi, sel.numel()), "swiglu_bwd block_stack")


def test_rmsnorm_block_stack_sampled(pf):
    rows, cols = 32768, 2048
    say("rmsnorm_quant block_stack", rows, cols)
    d = synth.rmsnorm_inputs(rows, cols, seed=0)
    out = pf.rmsnorm_quant(dev(d["x"]), dev(d["gamma"]), eps=1e-6, row=True, col=True)
    sel = _sample_rows()
    h = _host_outputs(out, row_sel=sel.to("cuda:0"), rb_sel=SAMPLE_RBS)
    y, lo, hi, rstd = oracle.rmsnorm_fwd(synth.bits(d["x"][sel]), synth.bits(d["gamma"]),
                                        float(np.float32(1e-6)), TOL)
    got_rstd = host(out["rstd"][sel.to("cuda:0")]).astype(np.float64)
    assert np.max(np.abs(got_rstd - rstd) / rstd) <= TOL
    _assert_ok(pc.check_outputs(h, y, lo, hi, sel.numel()), "rmsnorm block_stack")


@pytest.mark.parametrize("form", [0, 1, 2])
def test_probe_sigmoid_within_its_bound(pf, form):
    """The FP32 sigmoid the SwiGLU producers evaluate, through
    puro_fp8_probe_sigmoid, against 1 / (1 + e^-g) in double precision on
    64 runs of 2^18 consecutive FP32 inputs per range (16.8 M values each):
    [0, 104], [-64, 0] (both forms), and, for the deep form and the per-wave
    choice, [-104, 0] and [-104, -80].  Relative error at most 5 * 2^-24 (the
    budget the producers' tolerance assumes) wherever the result is normal;
    below that (g < -87.3, a subnormal result) within 5 * 2^-24 of it plus
    half the subnormal spacing 2^-149, and never flushed to zero while the
    exact value is at least 2^-149.  form 0 chooses per wave as the
    producers do, 1 is the plain form (used only when every gate of a wave
    is >= -64), 2 the deep form."""
    import struct
    bits = lambda v: struct.unpack("<I", struct.pack("<f", v))[0]
    run = 1 << 18
    buf = torch.empty(run, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ranges = [(0, 0.0, 104.0), (0x80000000, 0.0, 64.0)]
    if form != 1:
        ranges += [(0x80000000, 0.0, 104.0), (0x80000000, 80.0, 104.0)]
    worst = 0.0
    worst_sub = 0.0
    n_sub = 0
    for sign, lo, hi in ranges:
        say("probe_sigmoid form", form, "-" if sign else "+", lo, hi, "64 runs of", run)
        b0, b1 = bits(lo), bits(hi)
        for k in range(64):
            first = (b0 + (k * (b1 - b0 - run)) // 63) | sign
            assert pf.puro_fp8_probe_sigmoid(first, run, form, buf.data_ptr(), stream) == 0
            got = host(buf).astype(np.float64)
            g = np.arange(first, first + run, dtype=np.uint64).astype(np.uint32).view(np.float32)
            ref = 1.0 / (1.0 + np.exp(-g.astype(np.float64)))
            normal = ref >= 2.0 ** -126
            if normal.any():
                err = np.abs(got[normal] - ref[normal]) / ref[normal]
                worst = max(worst, float(err.max()))
            sub = ~normal & (ref >= 2.0 ** -149)
            if sub.any():
                n_sub += int(sub.sum())
                excess = np.abs(got[sub] - ref[sub]) - 5 * 2.0 ** -24 * ref[sub]
                worst_sub = max(worst_sub, float(excess.max()))
                assert np.all(got[sub] > 0.0)
    say(f"   max relative error {worst / 2.0 ** -24:.3f} x 2^-24; {n_sub} subnormal results, "
        f"worst excess {worst_sub / 2.0 ** -149:.3f} x 2^-149")
    assert worst <= 5 * 2.0 ** -24
    assert worst_sub <= 2.0 ** -150
    assert (n_sub > 0) == (form != 1)


# ---- RMSNorm backward plus the skip path; residual add with rstd -----------------

def _tol_bwd(cols):
    """The FP32 error bound the C header states for the backward, as a
    fraction of its magnitude M: (cols/512 + 18) * 2^-24."""
    return (cols / 512 + 18) * 2.0 ** -24


@pytest.mark.parametrize("rows,cols,skip", [(77, 128, True), (256, 2048, True),
                                            (130, 8192, False), (1000, 384, True),
                                            (1000, 4096, True)])
def test_rmsnorm_bwd_parity(pf, rows, cols, skip):
    say("rmsnorm_bwd_quant", rows, cols, skip)
    d = synth.rmsnorm_bwd_inputs(rows, cols, seed=rows + cols)
    rstd = torch.from_numpy(oracle.rmsnorm_fwd(synth.bits(d["x"]), synth.bits(d["gamma"]),
                                               1e-6, TOL)[3].astype(np.float32))
    gin = d["gin"] if skip else None
    out = pf.rmsnorm_bwd_quant(dev(d["dy"]), dev(d["x"]), dev(d["gamma"]), dev(rstd),
                               None if gin is None else dev(gin), row=True, col=True,
                               bf16_out=True)
    y, lo, hi = oracle.rmsnorm_bwd(synth.bits(d["dy"]), synth.bits(d["x"]),
                                   synth.bits(d["gamma"]), rstd.numpy(),
                                   None if gin is None else synth.bits(gin), _tol_bwd(cols))
    _assert_ok(pc.check_outputs(_host_outputs(out), y, lo, hi, rows),
               f"rmsnorm_bwd {rows}x{cols}")


def test_rmsnorm_bwd_output_subsets(pf):
    """Each subset of outputs equals the same outputs of the all-output call,
    and the codes are those of the plain quantizer on the bf16 result."""
    rows, cols = 300, 512
    d = synth.rmsnorm_bwd_inputs(rows, cols, seed=6)
    rstd = dev(torch.rand(rows, dtype=torch.float32) + 0.5)
    args = [dev(d[k]) for k in ("dy", "x", "gamma")] + [rstd, dev(d["gin"])]
    say("rmsnorm_bwd_quant subsets", rows, cols)
    full = pf.rmsnorm_bwd_quant(*args, row=True, col=True, bf16_out=True)
    for row, col, yb in [(True, False, False), (False, True, False), (False, False, True),
                         (True, True, False), (True, False, True), (False, True, True)]:
        part = pf.rmsnorm_bwd_quant(*args, row=row, col=col, bf16_out=yb)
        for k, v in part.items():
            assert _same(v, full[k]), (k, row, col, yb)
    ref = pf.quant_act(full["y"], row=True, col=True)
    for k in ("q", "s", "qt", "st"):
        assert _same(full[k], ref[k]), k


def test_rmsnorm_bwd_block_stack_sampled(pf):
    rows, cols = 32768, 2048
    say("rmsnorm_bwd_quant block_stack", rows, cols)
    d = synth.rmsnorm_bwd_inputs(rows, cols, seed=0)
    x = dev(d["x"])
    fwd = pf.rmsnorm_quant(x, dev(d["gamma"]), eps=1e-6, row=True, col=False)
    out = pf.rmsnorm_bwd_quant(dev(d["dy"]), x, dev(d["gamma"]), fwd["rstd"], dev(d["gin"]),
                               row=True, col=True)
    sel = _sample_rows()
    h = _host_outputs(out, row_sel=sel.to("cuda:0"), rb_sel=SAMPLE_RBS)
    rstd = host(fwd["rstd"][sel.to("cuda:0")])
    y, lo, hi = oracle.rmsnorm_bwd(synth.bits(d["dy"][sel]), synth.bits(d["x"][sel]),
                                   synth.bits(d["gamma"]), rstd, synth.bits(d["gin"][sel]),
                                   _tol_bwd(cols))
    _assert_ok(pc.check_outputs(h, y, lo, hi, sel.numel()), "rmsnorm_bwd block_stack")


@pytest.mark.parametrize("rows,cols", [(77, 128), (1000, 2048), (130, 8192), (500, 8192)])
def test_residual_add_rstd_then_one_pass_norm(pf, rows, cols):
    """h = a + b bit for bit against the oracle, rstd within TOL of the
    oracle's statistic of h, and the one-pass norm from that rstd equals the
    two-pass puro_fp8_rmsnorm_quant on h wherever the two rstd agree."""
    say("residual_add_rstd", rows, cols)
    d = synth.residual_inputs(rows, cols, seed=rows + cols)
    r = pf.residual_add_rstd(dev(d["a"]), dev(d["b"]), eps=1e-6)
    h_ref = oracle.residual_add(synth.bits(d["a"]), synth.bits(d["b"]))
    assert np.array_equal(bf16_host_bits(r["h"]), h_ref)
    _, _, _, rstd_ref = oracle.rmsnorm_fwd(h_ref, synth.bits(d["gamma"]), float(np.float32(1e-6)),
                                           TOL)
    got_rstd = host(r["rstd"]).astype(np.float64)
    assert np.max(np.abs(got_rstd - rstd_ref) / rstd_ref) <= TOL
    one = pf.rmsnorm_quant_rstd(r["h"], dev(d["gamma"]), r["rstd"], row=True, col=True,
                                bf16_out=True)
    two = pf.rmsnorm_quant(r["h"], dev(d["gamma"]), eps=1e-6, row=True, col=True,
                           bf16_out=True)
    assert torch.equal(two["rstd"], r["rstd"])      # same statistic, same summation order
    for k in ("q", "s", "qt", "st", "y"):
        assert _same(one[k], two[k]), k
    y, lo, hi, _ = oracle.rmsnorm_fwd(h_ref, synth.bits(d["gamma"]), float(np.float32(1e-6)), TOL)
    _assert_ok(pc.check_outputs(_host_outputs(one), y, lo, hi, rows), f"one-pass {rows}x{cols}")
