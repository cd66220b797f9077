"""The quantize-on-produce checker (tests/produce_check.py) accepts every
correct result and rejects planted mistakes.  A "device" is simulated on the
CPU from the oracle alone: it picks, per element, one of the correct bf16
values (lo, y or hi) and quantizes with the oracle's quantizers."""
from __future__ import annotations

import numpy as np
import pytest

import produce_check as pc


def _simulated_device(orc, y, lo, hi, rng):
    pick = rng.integers(0, 3, y.shape)
    yd = np.where(pick == 0, lo, np.where(pick == 1, y, hi)).astype(np.uint16)
    q, s = orc.quant_rowwise(yd)
    qt, st = orc.quant_colwise(yd)
    return {"y": yd, "q": q, "s": s, "qt": qt, "st": st}


@pytest.fixture(scope="module")
def case(orc):
    rng = np.random.default_rng(21)
    rows, f = 200, 256
    gu = (rng.standard_normal((rows, 2 * f)).astype(np.float32))
    import torch
    gu_bits = torch.from_numpy(gu).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # a band of 2^-14 of |h| (wider than the FP32 error) puts about 2% of the
    # elements near a rounding boundary: most tiles have several correct results
    y, lo, hi = orc.swiglu_fwd(gu_bits, tol=2.0 ** -14)
    return rows, y, lo, hi


def test_checker_accepts_any_correct_choice(orc, case):
    rows, y, lo, hi = case
    assert np.count_nonzero(lo != hi) > 100
    for seed in range(3):
        dev = _simulated_device(orc, y, lo, hi, np.random.default_rng(seed))
        res = pc.check_outputs(dev, y, lo, hi, rows)
        assert pc.all_ok(res), res
        assert res["row"]["ambiguous"] > 0 and res["col"]["ambiguous"] > 0


def test_checker_rejects_planted_mistakes(orc, case):
    rows, y, lo, hi = case
    base = _simulated_device(orc, y, lo, hi, np.random.default_rng(7))
    # one code off by one step
    d = {k: v.copy() for k, v in base.items()}
    d["q"][17, 40] ^= 1
    assert pc.check_outputs(d, y, lo, hi, rows)["row"]["bad"] == [17 * 2 + 0]
    # one row scale changed in its last bit
    d = {k: v.copy() for k, v in base.items()}
    d["s"].view(np.uint32)[1, 5] ^= 1
    assert pc.check_outputs(d, y, lo, hi, rows)["row"]["bad"] == [5 * 2 + 1]
    # one transposed code in a tile with alternatives
    d = {k: v.copy() for k, v in base.items()}
    amb_c = np.nonzero((lo != hi).any(axis=0))[0][0]
    d["qt"][amb_c, 3] ^= 0x80
    assert pc.check_outputs(d, y, lo, hi, rows)["col"]["bad"] == [int(amb_c) * 2]
    # a padding code that is not zero
    d = {k: v.copy() for k, v in base.items()}
    d["qt"][0, rows] = 1
    assert pc.check_outputs(d, y, lo, hi, rows)["pad_nonzero"] == 1
    # a bf16 value that is neither correct result
    d = {k: v.copy() for k, v in base.items()}
    i = np.nonzero(lo == hi)
    d["y"][i[0][0], i[1][0]] += 2
    assert pc.check_outputs(d, y, lo, hi, rows)["bf16_wrong"] == 1


def test_checker_rejects_codes_of_an_unreachable_value(orc, case):
    """A tile quantized from a value two bf16 steps past both correct results
    of its largest element (so its scale moves) is not accepted."""
    rows, y, lo, hi = case
    yd = y.copy()
    r, cb = 3, 1
    seg = slice(128 * cb, 128 * cb + 128)
    c = 128 * cb + int(np.argmax(y[r, seg] & 0x7FFF))
    yd[r, c] = max(lo[r, c] & 0x7FFF, hi[r, c] & 0x7FFF) + 2 | (y[r, c] & 0x8000)
    q, s = orc.quant_rowwise(yd)
    res = pc.check_outputs({"q": q, "s": s}, y, lo, hi, rows)
    assert res["row"]["bad"] == [r * 2 + cb]
