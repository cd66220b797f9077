"""Pins of the oracle's neighbour ops (quantize-on-produce) against facts that
do not come from the oracle: hand-worked bf16 encodings of table values of the
logistic function (tests/golden/neighbour_ops.txt), the Lambert-W closed form
of SiLU's minimum, finite differences of the forward definition, exact scaling
identities of RMSNorm, and PyTorch's float32 -> bfloat16 conversion.

The ops are the BF16 neighbours of the FP8 GEMMs (Puro-2B arXiv report,
section 2.1; training.farm blog, FP8 section: only the linear-layer GEMMs run
in FP8, the rest stays in BF16), so the operand the path quantizes is the
op's bf16 output.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# SiLU's minimum: silu'(x) = 0 <=> 1 + x (1 - sigmoid(x)) = 0, whose root is
# x* = -1 - W(1/e) with W the Lambert W function; silu(x*) = x* + 1 = -W(1/e).
# W(1/e) = 0.27846454276107379510... (published constant).
W_INV_E = 0.2784645427610738


def _golden(op):
    rows = []
    with open(os.path.join(GOLDEN, "neighbour_ops.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line and line[0] == op:
                rows.append([int(v, 16) for v in line[1:]])
    assert rows
    return rows


def _to_bf16_torch(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---- rounding ----------------------------------------------------------------

def test_f64_to_bf16_matches_torch_on_float32_values(orc):
    """For values exactly representable in float32 the rounding equals
    PyTorch's float32 -> bfloat16 conversion (round to nearest even)."""
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 3.0,
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),   # subnormal
                        np.array([0.0, -0.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8], np.float32)])
    want = _to_bf16_torch(x)
    got = np.array([orc.f64_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)


def test_f64_to_bf16_rounds_once():
    """1 + 2^-8 + 2^-30 lies above the midpoint between 1 and 1 + 2^-7, so it
    rounds up (0x3F81); rounding through float32 first lands exactly on the
    midpoint and then goes to even (0x3F80)."""
    import oracle
    assert oracle.f64_to_bf16(1.0 + 2.0**-8 + 2.0**-30) == 0x3F81
    assert oracle.f64_to_bf16(1.0 + 2.0**-8) == 0x3F80          # tie -> even
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0**-8) == 0x3F82      # tie -> even (up)


def test_f64_to_bf16_range_ends(orc):
    """Subnormal steps of 2^-133, overflow past the largest finite bf16."""
    assert orc.f64_to_bf16(2.0**-133) == 0x0001
    assert orc.f64_to_bf16(2.0**-134) == 0x0000                 # tie -> even (0)
    assert orc.f64_to_bf16(1.5 * 2.0**-134) == 0x0001
    assert orc.f64_to_bf16(1.5 * 2.0**-133) == 0x0002           # tie -> even (2)
    assert orc.f64_to_bf16(-(2.0**-126)) == 0x8080              # smallest normal
    top = (2.0 - 2.0**-7) * 2.0**127                            # largest finite bf16
    assert orc.f64_to_bf16(top) == 0x7F7F
    assert orc.f64_to_bf16((2.0 - 2.0**-8) * 2.0**127) == 0x7F80  # tie -> even = inf
    assert orc.f64_to_bf16(-1e300) == 0xFF80
    assert orc.f64_to_bf16(-0.0) == 0x8000


def test_band_ends(orc):
    """(y, lo, hi): the rounding of v and of the two ends of the band."""
    mid = 1.0 + 2.0**-8                                          # between 0x3F80 and 0x3F81
    assert orc.bf16_band(mid, 1e-10) == (0x3F80, 0x3F80, 0x3F81)
    assert orc.bf16_band(mid + 2e-10, 1e-10) == (0x3F81, 0x3F81, 0x3F81)
    assert orc.bf16_band(mid + 2e-10, 3e-10) == (0x3F81, 0x3F80, 0x3F81)
    assert orc.bf16_band(1.0, 1e-6) == (0x3F80, 0x3F80, 0x3F80)
    assert orc.bf16_band(-mid, 1e-10) == (0xBF80, 0xBF81, 0xBF80)  # lo is the more negative
    assert orc.bf16_band(1.0, 2.0**-6) == (0x3F80, 0x3F7C, 0x3F82)  # several steps wide
    assert orc.bf16_band(1e-45, 1e-44) == (0x0000, 0x8000, 0x0000)  # straddles zero
    assert orc.bf16_band(-0.0, 0.0) == (0x8000, 0x8000, 0x8000)    # exact: keeps the sign
    # below the normal range the band also holds the FP32 subnormal spacing:
    # 2^-134 is the midpoint of bf16's 0 and 2^-133 (ties to the even 0), and
    # a device result of 2^-134 +- 2^-150 may round either way
    assert orc.bf16_band(2.0**-134, 2.0**-160) == (0x0000, 0x0000, 0x0001)
    assert orc.bf16_band(2.0**-134, 0.0) == (0x0000, 0x0000, 0x0000)


# ---- SwiGLU ------------------------------------------------------------------

def test_swiglu_fwd_golden(orc):
    rows = _golden("swiglu")
    gu = np.array([[g, u] for g, u, _ in rows], np.uint16)       # f = 1: gate | up
    y, lo, hi = orc.swiglu_fwd(gu, tol=2.0**-18)
    assert [int(v) for v in y[:, 0]] == [want for _, _, want in rows]
    assert np.array_equal(lo, y) and np.array_equal(hi, y)       # none lies near a tie


def test_swiglu_gate_up_layout(orc):
    """With f = 2 the gate of column c is gu[:, c] and its up is gu[:, 2 + c]."""
    gu = np.array([[0x3F80, 0x4000, 0x3F80, 0x3F80],             # gates (1, 2), ups (1, 1)
                   [0x3F80, 0x3F80, 0x4000, 0x3F80]], np.uint16)  # gates (1, 1), ups (2, 1)
    y, _, _ = orc.swiglu_fwd(gu, tol=0.0)
    assert y.tolist() == [[0x3F3B, 0x3FE1], [0x3FBB, 0x3F3B]]


def test_silu_minimum_closed_form(orc):
    """At x* = -1 - W(1/e): silu(x*) = -W(1/e) and silu'(x*) = 0."""
    x = -1.0 - W_INV_E
    h, dgate, dup, _ = orc.swiglu_point(x, 1.0, 1.0)
    assert abs(h - (-W_INV_E)) < 1e-15
    assert abs(dgate) < 1e-15
    assert dup == h                                              # d up = dh * silu(g)


def test_swiglu_grads_at_zero(orc):
    """sigmoid(0) = 1/2 exactly: d gate = dh * up / 2, d up = h = 0."""
    h, dgate, dup, _ = orc.swiglu_point(0.0, 3.0, 2.0)
    assert (h, dgate, dup) == (0.0, 3.0, 0.0)


@pytest.mark.parametrize("g", [-9.0, -3.5, -1.28, -0.7, 0.3, 1.0, 2.5, 6.0])
def test_swiglu_dgate_is_the_derivative(orc, g):
    """d gate = dh * d h / d gate, checked by a central difference of the
    forward definition (step 1e-5, error O(1e-10))."""
    u, dh, step = 0.75, -1.5, 1e-5
    hp = orc.swiglu_point(g + step, u)[0]
    hm = orc.swiglu_point(g - step, u)[0]
    _, dgate, dup, m = orc.swiglu_point(g, u, dh)
    assert abs(dgate - dh * (hp - hm) / (2 * step)) < 1e-8
    assert abs(dup - dh * orc.swiglu_point(g, 1.0)[0]) <= 1e-15 * abs(dup)
    assert m >= abs(dgate)                                        # M bounds the result


def test_swiglu_bwd_layout_and_rounding(orc):
    """d gate lands in columns [0, f), d up in [f, 2f); each is the point
    value rounded once."""
    rng = np.random.default_rng(11)
    f, rows = 3, 5
    gu = _to_bf16_torch(rng.standard_normal((rows, 2 * f)) * 2.0)
    dh = _to_bf16_torch(rng.standard_normal((rows, f)))
    y, lo, hi = orc.swiglu_bwd(dh, gu, tol=0.0)
    assert np.array_equal(y, lo) and np.array_equal(y, hi)
    def wid(b):
        return float(orc.bf16_bits_to_f32(np.array([b], np.uint16))[0])
    for r in range(rows):
        for c in range(f):
            _, dg, du, _ = orc.swiglu_point(wid(gu[r, c]), wid(gu[r, f + c]), wid(dh[r, c]))
            assert y[r, c] == orc.f64_to_bf16(dg)
            assert y[r, f + c] == orc.f64_to_bf16(du)


# ---- RMSNorm -----------------------------------------------------------------

def test_rmsnorm_golden(orc):
    (x0, x1, g0, g1, y0, y1), = _golden("rmsnorm")
    y, _, _, rstd = orc.rmsnorm_fwd(np.array([[x0, x1]], np.uint16),
                                     np.array([g0, g1], np.uint16), eps=0.0, tol=2.0**-18)
    assert y.tolist() == [[y0, y1]]
    assert abs(rstd[0] - math.sqrt(2.0) / 5.0) < 1e-16


def test_rmsnorm_constant_magnitude_rows(orc):
    """|x| = a along a row and eps = 0: rstd = 1/a and y = sign(x) * gamma."""
    rng = np.random.default_rng(3)
    cols = 256
    gamma = _to_bf16_torch(rng.standard_normal(cols))
    signs = np.where(rng.standard_normal((4, cols)) < 0, -1.0, 1.0)
    x = _to_bf16_torch(signs * np.array([[0.375], [3.0], [2.0**-20], [96.0]]))
    y, lo, hi, rstd = orc.rmsnorm_fwd(x, gamma, eps=0.0, tol=2.0**-18)
    want = _to_bf16_torch(signs * (gamma.astype(np.uint32) << 16).view(np.float32))
    assert np.array_equal(y, want)
    assert np.array_equal(y, lo) and np.array_equal(y, hi)
    assert np.allclose(rstd, 1.0 / np.array([0.375, 3.0, 2.0**-20, 96.0]), rtol=1e-15)


def test_rmsnorm_scaling_identities(orc):
    """eps = 0: scaling x by 2^k leaves y unchanged; doubling gamma doubles it."""
    rng = np.random.default_rng(4)
    rows, cols = 6, 384
    xf = rng.standard_normal((rows, cols)).astype(np.float32)
    x = _to_bf16_torch(xf)
    x8 = _to_bf16_torch(xf * 8.0)
    gamma = _to_bf16_torch(rng.standard_normal(cols))
    gamma2 = _to_bf16_torch((gamma.astype(np.uint32) << 16).view(np.float32) * 2.0)
    y, _, _, rs = orc.rmsnorm_fwd(x, gamma, eps=0.0, tol=0.0)
    y8, _, _, rs8 = orc.rmsnorm_fwd(x8, gamma, eps=0.0, tol=0.0)
    y2, _, _, _ = orc.rmsnorm_fwd(x, gamma2, eps=0.0, tol=0.0)
    assert np.array_equal(y, y8)
    assert np.array_equal(rs, rs8 * 8.0)
    nz = (y & 0x7FFF) != 0
    assert np.array_equal(y2[nz], y[nz] + 0x80)                  # exponent + 1


def test_rmsnorm_eps(orc):
    """A zero row with eps = 2^-20 has rstd = 2^10 and signed-zero outputs."""
    x = np.zeros((1, 128), np.uint16)
    x[0, 1] = 0x8000                                             # -0
    gamma = np.full(128, 0x3F80, np.uint16)
    y, _, _, rstd = orc.rmsnorm_fwd(x, gamma, eps=2.0**-20, tol=2.0**-18)
    assert rstd[0] == 1024.0
    assert y[0, 0] == 0x0000 and y[0, 1] == 0x8000


# ---- RMSNorm backward plus the skip path ----------------------------------------

def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rstd32(xb, eps):
    x = _f(xb)
    return (1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)).astype(np.float32)


def test_rmsnorm_bwd_golden(orc):
    rows = _golden("rmsnorm_bwd")
    assert len(rows) == 3
    for x0, x1, g0, g1, d0, d1, i0, i1, o0, o1 in rows:
        x = np.array([[x0, x1]], np.uint16)
        rstd = np.array([math.sqrt(2.0) / 5.0], np.float32)
        gin = np.array([[i0, i1]], np.uint16)
        y, lo, hi = orc.rmsnorm_bwd(np.array([[d0, d1]], np.uint16), x,
                                    np.array([g0, g1], np.uint16), rstd,
                                    gin if (i0 or i1) else None, 2.0**-18)
        assert y.tolist() == [[o0, o1]], [hex(v) for v in y.ravel()]
        assert np.array_equal(lo, y) and np.array_equal(hi, y)


@pytest.mark.parametrize("eps", [0.0, 1e-2])
def test_rmsnorm_bwd_is_the_derivative_of_the_forward(orc, eps):
    """Central differences of the forward y = x gamma / sqrt(mean x^2 + eps),
    written here in double, give gin + J^T dy; the oracle's bf16 result is
    that value rounded (within half a bf16 ulp plus the FP32 rstd's effect)."""
    rng = np.random.default_rng(11)
    rows, cols = 3, 24
    xb = _to_bf16_torch(rng.standard_normal((rows, cols)) * np.array([[1.0], [0.05], [7.0]]))
    gb = _to_bf16_torch(rng.standard_normal(cols))
    dyb = _to_bf16_torch(rng.standard_normal((rows, cols)))
    ginb = _to_bf16_torch(rng.standard_normal((rows, cols)) * 0.1)
    rstd = _rstd32(xb, eps)
    y, lo, hi = orc.rmsnorm_bwd(dyb, xb, gb, rstd, ginb, 2.0**-18)
    x, g, dy, gin = _f(xb), _f(gb), _f(dyb), _f(ginb)

    def loss(xr, dyr):
        return float(np.sum(dyr * xr * g / math.sqrt(np.mean(xr * xr) + eps)))

    got = _f(y)
    for r in range(rows):
        h = 1e-4 * float(np.max(np.abs(x[r])))
        for i in range(cols):
            xp, xm = x[r].copy(), x[r].copy()
            xp[i] += h
            xm[i] -= h
            fd = gin[r, i] + (loss(xp, dy[r]) - loss(xm, dy[r])) / (2.0 * h)
            rs = 1.0 / math.sqrt(np.mean(x[r] ** 2) + eps)
            m = abs(gin[r, i]) + abs(rs * g[i] * dy[r, i]) + \
                abs(x[r, i]) * rs ** 3 * float(np.mean(np.abs(g * dy[r] * x[r])))
            assert abs(got[r, i] - fd) <= 2.0**-8 * abs(fd) + 1e-6 * m, (r, i, got[r, i], fd)
    assert np.all(_f(lo) <= got) and np.all(got <= _f(hi))


def test_rmsnorm_bwd_orthogonal_to_x(orc):
    """eps = 0 makes y invariant under x -> a x, so J x = 0 and sum_i x_i out_i
    = 0 without the skip path (up to the bf16 rounding of out)."""
    rng = np.random.default_rng(12)
    rows, cols = 5, 256
    xb = _to_bf16_torch(rng.standard_normal((rows, cols)))
    gb = _to_bf16_torch(1.0 + 0.3 * rng.standard_normal(cols))
    # dy partly along x, so the two terms are large and must cancel
    dyb = _to_bf16_torch(0.7 * _f(xb) + 0.7 * rng.standard_normal((rows, cols)))
    y, _, _ = orc.rmsnorm_bwd(dyb, xb, gb, _rstd32(xb, 0.0), None, 0.0)
    p = _f(xb) * _f(y)
    assert np.all(np.abs(p.sum(axis=1)) <= 2.0**-8 * np.abs(p).sum(axis=1))
    # the pieces do not cancel on their own: without the second term the sum
    # is O(1) of its magnitude
    direct = _f(xb) * _rstd32(xb, 0.0)[:, None] * _f(gb) * _f(dyb)
    assert np.all(np.abs(direct.sum(axis=1)) > 0.25 * np.abs(direct).sum(axis=1))


def test_rmsnorm_bwd_scaling(orc):
    """eps = 0: x -> 2x (rstd -> rstd/2, exact) halves out; dy -> 2 dy doubles
    it; (gamma, dy) -> (2 gamma, dy/2) leaves it unchanged -- all bit-exact
    exponent shifts of every nonzero bf16 result."""
    rng = np.random.default_rng(13)
    rows, cols = 4, 384
    xf = rng.standard_normal((rows, cols))
    xb, x2b = _to_bf16_torch(xf), _to_bf16_torch(2.0 * xf)
    gf = rng.standard_normal(cols)
    gb, g2b = _to_bf16_torch(gf), _to_bf16_torch(2.0 * gf)
    dyf = rng.standard_normal((rows, cols))
    dyb, dy2b, dyhb = (_to_bf16_torch(dyf), _to_bf16_torch(2.0 * dyf),
                       _to_bf16_torch(0.5 * dyf))
    rs = _rstd32(xb, 0.0)
    y, _, _ = orc.rmsnorm_bwd(dyb, xb, gb, rs, None, 0.0)
    yx2, _, _ = orc.rmsnorm_bwd(dyb, x2b, gb, rs / np.float32(2.0), None, 0.0)
    ydy2, _, _ = orc.rmsnorm_bwd(dy2b, xb, gb, rs, None, 0.0)
    yg2, _, _ = orc.rmsnorm_bwd(dyhb, xb, g2b, rs, None, 0.0)
    nz = (y & 0x7FFF) != 0
    assert nz.mean() > 0.99
    assert np.array_equal(yx2[nz], y[nz] - 0x80)
    assert np.array_equal(ydy2[nz], y[nz] + 0x80)
    assert np.array_equal(yg2, y)


def test_rmsnorm_bwd_skip_path_alone(orc):
    """dy = 0: out is gin, bit for bit, with a one-value band."""
    rng = np.random.default_rng(14)
    rows, cols = 3, 128
    xb = _to_bf16_torch(rng.standard_normal((rows, cols)))
    ginb = _to_bf16_torch(rng.standard_normal((rows, cols)))
    y, lo, hi = orc.rmsnorm_bwd(np.zeros((rows, cols), np.uint16), xb,
                                _to_bf16_torch(rng.standard_normal(cols)), _rstd32(xb, 0.0),
                                ginb, 2.0**-18)
    assert np.array_equal(y, ginb) and np.array_equal(lo, ginb) and np.array_equal(hi, ginb)


def test_residual_add_matches_torch(orc):
    """h = a + b rounded once to bf16, against PyTorch's bf16 addition, over a
    spread of binades (the FP32 sum of two bf16 values rounds to the same
    bf16 as the exact sum), plus signed zeros and cancellation."""
    import torch
    rng = np.random.default_rng(15)
    n = 1 << 16
    a = _to_bf16_torch(rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n)))
    b = _to_bf16_torch(rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n)))
    a[:4] = [0x0000, 0x8000, 0x3F80, 0x4049]
    b[:4] = [0x8000, 0x8000, 0xBF80, 0xC049]
    want = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
            + torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)).view(torch.int16).numpy()
    h = orc.residual_add(a, b)
    assert np.array_equal(h, want.view(np.uint16))
    assert h[:4].tolist() == [0x0000, 0x8000, 0x0000, 0x0000]
