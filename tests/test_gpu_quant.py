"""GPU parity of the quantizers and the device E4M3 conversion against the
CPU oracle: codes and scales bit-exact.  Calls go through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import bf16_host_bits, dev, host, random_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


def _check_act(pf, x_cpu, row=True, col=True, tag=""):
    rows, cols = x_cpu.shape
    say("quant_act", tag, rows, cols, "row" if row else "", "col" if col else "")
    out = pf.quant_act(dev(x_cpu), row=row, col=col)
    xb = synth.bits(x_cpu)
    if row:
        q, s = oracle.quant_rowwise(xb)
        assert np.array_equal(host(out["q"]), q), "row codes differ"
        assert np.array_equal(host(out["s"]).view(np.uint32), s.view(np.uint32)), "row scales differ"
    if col:
        qt, st = oracle.quant_colwise(xb)
        assert np.array_equal(host(out["qt"]), qt), "column codes differ"
        assert np.array_equal(host(out["st"]).view(np.uint32), st.view(np.uint32)), "column scales differ"


# ---- the device conversion itself ------------------------------------------

def test_probe_encode_exhaustive_below_464(pf):
    """Every binary32 bit pattern with |v| < 464 (both signs): the hardware
    E4M3 conversion equals the oracle's round-to-nearest-even encoder.  These
    cover every scaled value a quantizer can produce (|v| <= 448 * (1+2^-23))."""
    chunk = 1 << 28
    buf = torch.empty(chunk, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for sign in (0, 0x80000000):
        start, end = sign, sign + 0x43E80000          # 464.0f = 0x43E80000
        for first in range(start, end, chunk):
            n = min(chunk, end - first)
            say("probe_encode", hex(first), n)
            assert pf.puro_fp8_probe_encode(first, n, buf.data_ptr(), stream) == 0
            got = host(buf[:n])
            exp = oracle.e4m3_encode_range(first, n)
            bad = np.nonzero(got != exp)[0]
            assert bad.size == 0, (f"first mismatch bits {first + int(bad[0]):#010x}: "
                                   f"device {got[bad[0]]:#04x} oracle {exp[bad[0]]:#04x}")


# ---- activation quantizer ----------------------------------------------------

@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 256), (128, 128), (129, 384),
                                       (300, 512), (1000, 1024), (4096, 2048),
                                       # block rows in groups of 8: 8 + 3, and 8 + 8 + 1
                                       (1300, 640), (2100, 1152),
                                       # the XCD-tiled walk: 4x4 tiles stacked 2 high
                                       # (32-63 block columns) and 1 high (64+), ragged
                                       # last block row; 1100 x 6144 falls back to the
                                       # grouped walk (9 block rows)
                                       (1000, 4096), (1024, 6144), (1000, 8192),
                                       (3000, 12288), (1100, 6144)])
@pytest.mark.parametrize("mode", ["row", "col", "dual"])
def test_quant_act_small(pf, rows, cols, mode):
    x = random_bf16((rows, cols), seed=rows * 7 + cols, stream=f"act/{rows}x{cols}")
    _check_act(pf, x, row=mode in ("row", "dual"), col=mode in ("col", "dual"),
               tag=f"small-{mode}")


@pytest.mark.parametrize("name,which,row,col", [
    ("tiny_fwd", "x", True, False),
    ("qkv_fwd", "x", True, False),
    ("upgate_fwd", "x", True, False),
    ("down_bwd", "dy", True, True),
    ("down_bwd", "x", False, True),
])
def test_quant_act_workloads(pf, name, which, row, col):
    spec = synth.workload(name).linears[0]
    t = synth.linear_inputs(spec, need=(which,))[which]
    _check_act(pf, t, row=row, col=col, tag=f"{name}/{which}")


def test_quant_act_largest_block_stack_gradient(pf):
    """The largest tensor of the transformer-block workload: the up/gate
    output gradient dY [32768 x 16384], dual row + column quantization."""
    spec = synth.workload("block_stack").linears[2]
    t = synth.linear_inputs(spec, need=("dy",))["dy"]
    _check_act(pf, t, row=True, col=True, tag="block_stack/up_gate/dy")


@pytest.mark.parametrize("linear,which", [(0, "x"), (0, "dy"), (1, "x"), (1, "dy"), (2, "x"),
                                          (3, "x"), (3, "dy")])
def test_quant_act_block_stack_launches(pf, linear, which):
    """With the up/gate dY above, every dual quantizer launch of the benchmark
    step at its own shape (32768 tokens; the 2048-, 6144- and 8192-column
    operands), all codes and scales against the oracle."""
    spec = synth.workload("block_stack").linears[linear]
    t = synth.linear_inputs(spec, need=(which,))[which]
    _check_act(pf, t, row=True, col=True, tag=f"block_stack/{spec.name}/{which}")


def test_quant_weight_grouped_block_stack(pf):
    """The benchmark step's grouped weight launch: the block's four weights
    (QKV 6144 x 2048, out-proj 2048 x 2048, up/gate 16384 x 2048, down
    2048 x 8192) in one launch, codes only, against the oracle."""
    ws = [synth.linear_inputs(spec, need=("w",))["w"] for spec in synth.workload("block_stack").linears]
    say("quant_weight_grouped block_stack", [tuple(w.shape) for w in ws])
    got = pf.quant_weight_grouped([dev(w) for w in ws], transpose=False, codes=True)
    for w, g in zip(ws, got):
        q, _, s = oracle.quant_weight(synth.bits(w), transpose=False)
        assert np.array_equal(host(g["q"]), q)
        assert np.array_equal(host(g["s"]).view(np.uint32), s.view(np.uint32))
        assert "qt" not in g


def test_quant_act_special_tiles(pf):
    """Zero tiles, negative zeros, bf16 subnormal amax (the 2^64 rescale),
    huge values, exact power-of-two amax, one outlier per tile."""
    rows, cols = 256, 512
    xb = np.zeros((rows, cols), np.uint16)
    xb[1, :] = 0x8000                                   # all -0.0
    xb[2, :128] = 0x0001                                # smallest subnormal
    xb[2, 128:256] = np.arange(128, dtype=np.uint16) | 0x8000
    xb[3, :] = 0x7F7F                                   # bf16 max
    xb[3, ::3] = 0xFF7F
    xb[4, :] = 0x43E0                                   # 448.0
    xb[5, :] = 0x3F80                                   # 1.0 with one 2.0
    xb[5, 5] = 0x4000
    rng = np.random.default_rng(5)
    xb[6:, :] = (rng.integers(0, 0x7F80, size=(rows - 6, cols)) |
                 (rng.integers(0, 2, size=(rows - 6, cols)) << 15)).astype(np.uint16)
    x = synth.from_bits(xb)
    _check_act(pf, x, row=True, col=True, tag="special")


def test_quant_act_tiny_tiles_mixed_in_waves(pf):
    """Tiles whose amax is below 2^-64 (the 2^64 rescale) beside ordinary
    tiles within one wave, in both directions: every 7th row, one whole
    128-column band, one 128 x 128 block, every third column of another band,
    and zero rows.  Row-wise and column-wise codes and scales are bit-exact."""
    rows, cols = 1024, 1024
    x = random_bf16((rows, cols), seed=77, stream="act/tiny-mixed").float()
    x[::7] *= 2.0 ** -80
    x[:, 256:384] *= 2.0 ** -90
    x[512:640, 640:768] *= 2.0 ** -100
    x[:, 768:896:3] *= 2.0 ** -90
    x[300:310] = 0.0
    _check_act(pf, x.to(torch.bfloat16), row=True, col=True, tag="tiny-mixed")


def test_quant_weight_tiny_and_zero_blocks(pf):
    """Weight blocks with amax below 2^-64 and all-zero blocks beside
    ordinary ones: codes, transposed codes and block scales bit-exact."""
    n, k = 512, 768
    w = random_bf16((n, k), std=0.02, seed=91, stream="w/tiny-blocks").float()
    w[128:256, 256:384] *= 2.0 ** -90
    w[0:128, 640:768] = 0.0
    w[384:512, 0:128] *= 2.0 ** -110
    w = w.to(torch.bfloat16)
    out = pf.quant_weight(dev(w), transpose=True)
    q, qt, s = oracle.quant_weight(synth.bits(w))
    assert (s < 2.0 ** -64).sum() == 3
    assert np.array_equal(host(out["q"]), q)
    assert np.array_equal(host(out["qt"]), qt)
    assert np.array_equal(host(out["s"]).view(np.uint32), s.view(np.uint32))


def test_quant_act_exhaustive_amax_x_pairs(pf):
    """Every non-negative finite bf16 amax (32,640 values) against every bf16
    magnitude x <= amax (about 5.3e8 pairs, alternating signs): one tile per
    row holds amax at position 0 and 127 x values; the row-wise codes and
    scales equal the oracle's bit for bit."""
    amax_bits = np.arange(0, 0x7F80, dtype=np.int64)
    ntile = (amax_bits + 1 + 126) // 127                 # tiles needed per amax
    total = int(ntile.sum())
    say("exhaustive pairs: rows", total)
    tile_amax = np.repeat(amax_bits, ntile).astype(np.int32)
    first = np.concatenate([[0], np.cumsum(ntile)[:-1]])
    tile_idx = (np.arange(total) - np.repeat(first, ntile)).astype(np.int32)  # k-th tile of its amax
    xb = np.empty((total, 128), np.uint16)
    xb[:, 0] = tile_amax.astype(np.uint16)
    lane = np.arange(127, dtype=np.int32)[None, :]
    step = 1 << 18
    for r0 in range(0, total, step):                    # build in chunks (bounded memory)
        ti = tile_idx[r0:r0 + step, None]
        am = tile_amax[r0:r0 + step, None]
        x = np.minimum(ti * 127 + lane, am)              # every magnitude <= amax
        sign = ((lane + ti) & 1) << 15
        xb[r0:r0 + step, 1:] = (x | sign).astype(np.uint16)
    del tile_idx, tile_amax
    xt = synth.from_bits(xb)
    out = pf.quant_act(dev(xt), row=True, col=False)
    q_dev = host(out["q"])
    s_dev = host(out["s"])
    del out
    q, s = oracle.quant_rowwise(xb)
    assert np.array_equal(s_dev.view(np.uint32), s.view(np.uint32))
    bad = np.argwhere(q_dev != q)
    assert bad.size == 0, (bad[:4], xb[tuple(bad[0])])


def test_quant_act_deterministic(pf):
    x = dev(random_bf16((2048, 1024), seed=9, stream="det"))
    say("quant_act determinism")
    a = pf.quant_act(x, row=True, col=True)
    b = pf.quant_act(x, row=True, col=True)
    for k in a:
        assert torch.equal(a[k], b[k])


def test_quant_act_empty(pf):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda:0")
    out = pf.quant_act(x, row=True, col=True)
    assert out["q"].shape == (0, 256) and out["qt"].shape == (256, 0)


# ---- weight quantizer ----------------------------------------------------------

@pytest.mark.parametrize("n,k", [(128, 128), (512, 512), (384, 256), (6144, 2048),
                                 (16384, 2048), (2048, 8192), (2048, 2048), (1280, 384)])
def test_quant_weight(pf, n, k):
    w = random_bf16((n, k), std=0.02, seed=n + k, stream=f"w/{n}x{k}")
    say("quant_weight", n, k)
    out = pf.quant_weight(dev(w), transpose=True)
    q, qt, s = oracle.quant_weight(synth.bits(w))
    assert np.array_equal(host(out["q"]), q)
    assert np.array_equal(host(out["qt"]), qt)
    assert np.array_equal(host(out["s"]).view(np.uint32), s.view(np.uint32))
    out2 = pf.quant_weight(dev(w), transpose=False)
    assert np.array_equal(host(out2["q"]), q) and "qt" not in out2
    out3 = pf.quant_weight(dev(w), transpose=True, codes=False)     # transposed copy only
    assert "q" not in out3
    assert np.array_equal(host(out3["qt"]), qt)
    assert np.array_equal(host(out3["s"]).view(np.uint32), s.view(np.uint32))


def test_quant_weight_grouped_equals_separate_launches(pf):
    """One launch over a block's four weights (with each combination of code
    copies) gives each weight's codes and scales bit for bit as its own
    puro_fp8_quant_weight launch, and as the oracle."""
    import oracle
    shapes = [(768, 256), (256, 256), (2048, 256), (256, 1024)]        # qkv, out, up/gate, down
    ws = [synth.normal(sh, 0.02, 7, f"grouped/{sh[0]}x{sh[1]}").to(torch.bfloat16) for sh in shapes]
    dws = [dev(w) for w in ws]
    for transpose, codes in ((True, True), (False, True), (True, False)):
        say("quant_weight_grouped", len(ws), "transpose" if transpose else "", "codes" if codes else "")
        got = pf.quant_weight_grouped(dws, transpose=transpose, codes=codes)
        for w, dw, g in zip(ws, dws, got):
            one = pf.quant_weight(dw, transpose=transpose, codes=codes)
            for k in one:
                assert torch.equal(g[k], one[k]), k
            q, qt, s = oracle.quant_weight(synth.bits(w), transpose=True)
            assert np.array_equal(host(g["s"]).view(np.uint32), s.view(np.uint32))
            if codes:
                assert np.array_equal(host(g["q"]), q)
            if transpose:
                assert np.array_equal(host(g["qt"]), qt)


def test_quant_weight_grouped_mixed_copies(pf):
    """Descriptors of one launch may ask for different code copies."""
    ws = [dev(synth.normal((384, 512), 0.02, i, f"grouped-mixed/{i}").to(torch.bfloat16))
          for i in range(3)]
    outs = [{"s": torch.empty((3, 4), dtype=torch.float32, device="cuda")} for _ in ws]
    outs[0]["q"] = torch.empty((384, 512), dtype=torch.uint8, device="cuda")
    outs[1]["qt"] = torch.empty((512, 384), dtype=torch.uint8, device="cuda")
    outs[2]["q"] = torch.empty((384, 512), dtype=torch.uint8, device="cuda")
    outs[2]["qt"] = torch.empty((512, 384), dtype=torch.uint8, device="cuda")
    P = lambda t: None if t is None else t.data_ptr()
    descs = (pf.WeightDesc * 3)(*[pf.WeightDesc(P(w), 384, 512, P(o.get("q")), P(o.get("qt")),
                                               P(o["s"])) for w, o in zip(ws, outs)])
    say("quant_weight_grouped mixed copies")
    assert pf.puro_fp8_quant_weight_grouped(descs, 3, torch.cuda.current_stream().cuda_stream) == 0
    for w, o in zip(ws, outs):
        ref = pf.quant_weight(w, transpose=True)
        for k in o:
            assert torch.equal(o[k], ref[k]), k


def test_quant_weight_grouped_sixteen_weights(pf):
    """The largest group (16 descriptors, ragged sizes, each combination of
    code copies): every weight equal to its own launch, so the block search
    over the prefix sums finds every weight's blocks."""
    rng = np.random.default_rng(16)
    shapes = [(128 * int(rng.integers(1, 7)), 128 * int(rng.integers(1, 7))) for _ in range(16)]
    ws = [dev(synth.normal(sh, 0.02, i, f"grouped16/{i}").to(torch.bfloat16))
          for i, sh in enumerate(shapes)]
    P = lambda t: None if t is None else t.data_ptr()
    outs = []
    for i, (n, k) in enumerate(shapes):
        o = {"s": torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda")}
        if i % 3 != 1:
            o["q"] = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        if i % 3 != 0:
            o["qt"] = torch.empty((k, n), dtype=torch.uint8, device="cuda")
        outs.append(o)
    descs = (pf.WeightDesc * 16)(*[pf.WeightDesc(P(w), n, k, P(o.get("q")), P(o.get("qt")), P(o["s"]))
                                   for w, (n, k), o in zip(ws, shapes, outs)])
    say("quant_weight_grouped 16 weights", shapes)
    assert pf.puro_fp8_quant_weight_grouped(descs, 16, torch.cuda.current_stream().cuda_stream) == 0
    for w, o in zip(ws, outs):
        ref = pf.quant_weight(w, transpose=True)
        for key in o:
            assert torch.equal(o[key], ref[key]), key
