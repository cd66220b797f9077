"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names what fixes the expected value: the OCP E4M3 format
definition, exact rational arithmetic, a brute-force search, a closed form,
or an invariant of tile-wise quantization (Puro-2B arXiv report section 2.1
and the training.farm blog FP8 section: DeepSeek-V3-style fine-grained block
quantization of the linear-layer GEMM operands, FP32 scales).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import reference_defs as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _random_bf16(shape, scale=1.0, seed=0):
    return _bf16_bits_from_f32(_rng(seed).standard_normal(shape).astype(np.float32) * scale)


def _all_finite_nonneg_bf16() -> np.ndarray:
    """Every non-negative finite bf16 bit pattern: 0x0000 .. 0x7F7F."""
    return np.arange(0, 0x7F80, dtype=np.uint16)


# ---------------------------------------------------------------- codec ----

def test_anchor_codes_from_ocp_spec(orc):
    """tests/golden/e4m3_anchors.txt: OCP OFP8 E4M3 anchor encodings."""
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_anchors.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            val, code = line.split()
            v = float(val)
            assert orc.e4m3_encode(v) == int(code, 16), (val, code)
            n += 1
    assert n >= 20


def test_decode_matches_format_definition(orc):
    """Decode of every code equals the value built from the definition
    (sorted table of the 127 finite magnitudes; 0x7F/0xFF are NaN)."""
    dec = orc.e4m3_decode_table()
    exp = ref.decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert math.isnan(dec[c])
        else:
            assert dec[c] == exp[c], hex(c)
    assert dec[0x7E] == 448.0 and dec[0x38] == 1.0 and dec[0x08] == 2.0 ** -6
    assert dec[0x01] == 2.0 ** -9 and dec[0x80] == 0.0 and math.copysign(1, dec[0x80]) < 0


def test_encode_decode_roundtrip_all_codes(orc):
    """E(dec(c)) == c for every finite code (each value is its own nearest)."""
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c


def test_encode_midpoints_tie_to_even(orc):
    """Every midpoint between adjacent finite magnitudes goes to the even code;
    just above / below a midpoint goes to the nearer side."""
    t = ref.e4m3_table()
    for i in range(126):
        mid = (t[i] + t[i + 1]) / 2               # exact in float64 and float32
        even = i if i % 2 == 0 else i + 1
        assert orc.e4m3_encode(np.float32(mid)) == even
        assert orc.e4m3_encode(-np.float32(mid)) == even | 0x80
        up = np.nextafter(np.float32(mid), np.float32(np.inf))
        dn = np.nextafter(np.float32(mid), np.float32(0))
        assert orc.e4m3_encode(up) == i + 1
        assert orc.e4m3_encode(dn) == i


def test_encode_random_vs_nearest_search(orc):
    """Random binary32 values against the table nearest-search."""
    rng = _rng(1)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    got = np.array([orc.e4m3_encode(x) for x in v], dtype=np.uint8)
    assert np.array_equal(got, ref.nearest_code(v))
    # dense sweep of the representable range
    w = np.concatenate([rng.uniform(-470, 470, 20000), rng.uniform(-0.02, 0.02, 20000)]).astype(np.float32)
    got = np.array([orc.e4m3_encode(x) for x in w], dtype=np.uint8)
    assert np.array_equal(got, ref.nearest_code(w))


def test_encode_sign_symmetry_and_monotone(orc):
    rng = _rng(2)
    v = np.sort(rng.uniform(0, 500, 5000).astype(np.float32))
    codes = [orc.e4m3_encode(x) for x in v]
    assert all(orc.e4m3_encode(-x) == c | 0x80 for x, c in zip(v, codes))
    assert all(a <= b for a, b in zip(codes, codes[1:]))


# ---------------------------------------------------------------- scale ----

def test_scale_exhaustive_all_bf16_amax(orc):
    """s = RN32(amax/448) for all 32,640 non-negative finite bf16 amax values,
    against exact rational division rounded to binary32 (gradual underflow)."""
    amax_bits = _all_finite_nonneg_bf16()
    amax = ref.bf16_widen(amax_bits)
    got = np.array([orc.tile_scale(a) for a in amax], dtype=np.float32)
    exp = ref.scale_def(amax)
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))
    # spot-check the float64 route against Fraction arithmetic
    for a in amax[::997]:
        fr = Fraction(float(a)) / 448
        assert float(np.float32(float(fr))) == float(exp[np.where(amax == a)[0][0]]) or a == 0


def test_reciprocal_unbounded_exponent_against_fractions():
    """The reciprocal reading RN24(448/amax), unbounded exponent, computed with
    exact Fractions for a spread of amax (including bf16 subnormals)."""
    amax = ref.bf16_widen(np.arange(1, 0x7F80, 211, dtype=np.uint16)).astype(np.float64)
    r = ref.round24(448.0 / amax)
    for a, rv in zip(amax, r):
        q = Fraction(448) / Fraction(float(a))
        e = q.numerator.bit_length() - q.denominator.bit_length()
        # normalise so that q * 2^(23 - e) lies in [2^23, 2^24)
        scaled = q * Fraction(2) ** (23 - e)
        while scaled >= 2 ** 24:
            scaled /= 2
            e += 1
        while scaled < 2 ** 23:
            scaled *= 2
            e -= 1
        n = scaled.numerator // scaled.denominator
        rem = scaled - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        exact = Fraction(n) * Fraction(2) ** (e - 23)
        assert Fraction(float(rv)) == exact


def test_scaled_value_all_amax_many_x(orc):
    """Element codes for every non-negative finite bf16 amax and 127 x values
    per tile (x = amax, -amax, random |x| <= amax, tiny values), via the
    oracle's row-wise quantizer, against the float64 definition."""
    rng = _rng(3)
    amax_bits = _all_finite_nonneg_bf16()
    R = amax_bits.size
    tiles = np.empty((R, 128), np.uint16)
    tiles[:, 0] = amax_bits
    tiles[:, 1] = amax_bits | 0x8000
    frac = rng.integers(0, 2 ** 16, size=(R, 126), dtype=np.uint32).astype(np.uint16)
    # random magnitudes <= amax: random bf16 below amax's bit pattern
    mag = (frac.astype(np.uint32) * (amax_bits[:, None].astype(np.uint32) + 1) >> 16).astype(np.uint16)
    sign = (rng.integers(0, 2, size=(R, 126)) << 15).astype(np.uint16)
    tiles[:, 2:] = mag | sign
    q, s = orc.quant_rowwise(tiles)
    q_exp, s_exp = ref.rowwise_def(tiles)
    assert np.array_equal(s.view(np.uint32), s_exp.view(np.uint32))
    bad = np.argwhere(q != q_exp)
    assert bad.size == 0, (bad[:5], q[tuple(bad[0])], q_exp[tuple(bad[0])])


def test_zero_and_tiny_tiles(orc):
    """amax = 0 gives s = 0 and signed-zero codes; tiny amax (bf16
    subnormals) stays finite through the 2^64 rescale."""
    x = np.zeros((2, 128), np.uint16)
    x[0, 3] = 0x8000                                   # -0.0
    x[1, :] = 0x0001                                   # smallest bf16 subnormal
    x[1, 7] = 0x8001
    q, s = orc.quant_rowwise(x)
    assert s[0, 0] == 0.0
    assert q[0, 3] == 0x80 and np.all(np.delete(q[0], 3) == 0)
    assert np.all(np.delete(q[1], 7) == 0x7E) and q[1, 7] == 0xFE
    assert s[0, 1] == np.float32(ref.scale_def(ref.bf16_widen(np.array([1], np.uint16))))[0]


# ---------------------------------------------------------- quantizers ----

@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 256), (300, 512)])
def test_rowwise_matches_definition(orc, rows, cols):
    xb = _random_bf16((rows, cols), seed=rows)
    q, s = orc.quant_rowwise(xb)
    qe, se = ref.rowwise_def(xb)
    assert np.array_equal(q, qe) and np.array_equal(s.view(np.uint32), se.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(1, 128), (130, 256), (384, 128)])
def test_colwise_matches_definition(orc, rows, cols):
    xb = _random_bf16((rows, cols), seed=rows + 1)
    qt, st = orc.quant_colwise(xb)
    qe, se = ref.colwise_def(xb)
    assert qt.shape == (cols, (rows + 127) // 128 * 128)
    assert np.array_equal(qt, qe) and np.array_equal(st.view(np.uint32), se.view(np.uint32))


def test_weight_matches_definition(orc):
    wb = _random_bf16((384, 256), scale=0.02, seed=5)
    q, qt, s = orc.quant_weight(wb)
    qe, se = ref.weight_def(wb)
    assert np.array_equal(q, qe) and np.array_equal(s.view(np.uint32), se.view(np.uint32))
    assert np.array_equal(qt, q.T)                     # invariant I4


def test_worked_tile(orc):
    """tests/golden/worked_tile.txt: 127 ones and one 2.0."""
    x = np.full((1, 128), 0x3F80, np.uint16)         # 1.0
    x[0, 5] = 0x4000                                   # 2.0
    q, s = orc.quant_rowwise(x)
    with open(os.path.join(GOLDEN, "worked_tile.txt")) as f:
        rows = [l.split("#")[0].split() for l in f if l.split("#")[0].strip()]
    for r in rows:
        if r[0] == "scale_hex":
            assert s.view(np.uint32)[0, 0] == int(r[1], 16)
        elif r[0] != "amax":
            assert q[0, int(r[0])] == int(r[2], 16)


def test_textbook_case_power_of_two_amax_is_plain_cast(orc):
    """amax = 448 * 2^j gives s = 2^j and r = 2^-j exactly, so the quantizer
    is a plain E4M3 cast of x / 2^j."""
    rng = _rng(7)
    for j in (-20, -5, 0, 3, 10):
        x = rng.uniform(-1, 1, (4, 128)).astype(np.float32) * 448 * 2.0 ** j
        x[:, 0] = 448 * 2.0 ** j
        xb = _bf16_bits_from_f32(x)
        q, s = orc.quant_rowwise(xb)
        assert np.all(s == np.float32(2.0 ** j))
        assert np.array_equal(q, ref.nearest_code(ref.bf16_widen(xb) / np.float32(2.0 ** j)))


def test_dequant_error_within_half_ulp(orc):
    """|dec(q) - v| <= ulp_e4m3(v)/2 in the scaled domain, and the real-domain
    error stays within that bound times s plus three binary32 roundings."""
    xb = _random_bf16((512, 1024), seed=11)
    x = ref.bf16_widen(xb).astype(np.float64)
    q, s = orc.quant_rowwise(xb)
    amax = np.repeat(ref.bf16_widen(xb).reshape(512, 8, 128).__abs__().max(axis=2), 128, axis=1)
    v = ref.scaled_def(ref.bf16_widen(xb), amax).astype(np.float64)
    dq = ref.decode(q)
    assert np.all(np.abs(dq - v) <= ref.ulp_e4m3(v) / 2)
    s_full = np.repeat(s.T, 128, axis=1).astype(np.float64)
    bound = (ref.ulp_e4m3(v) / 2 * (1 + 2.0 ** -21) + 2.0 ** -22 * np.abs(v)) * s_full
    assert np.all(np.abs(dq * s_full - x) <= bound)


def test_invariant_power_of_two_scaling(orc):
    """I1: x -> 2^j x leaves codes unchanged and multiplies s by 2^j."""
    xb = _random_bf16((64, 256), seed=13)
    x = ref.bf16_widen(xb)
    q0, s0 = orc.quant_rowwise(xb)
    for j in (-30, -3, 1, 9, 40):
        xj = _bf16_bits_from_f32(x * np.float32(2.0 ** j))
        qj, sj = orc.quant_rowwise(xj)
        assert np.array_equal(qj, q0)
        assert np.array_equal(sj, (s0.astype(np.float64) * 2.0 ** j).astype(np.float32))


def test_invariant_permutation_within_tile(orc):
    """I2: permuting the elements of a tile permutes its codes."""
    xb = _random_bf16((16, 128), seed=17)
    perm = _rng(17).permutation(128)
    q0, s0 = orc.quant_rowwise(xb)
    q1, s1 = orc.quant_rowwise(xb[:, perm])
    assert np.array_equal(q1, q0[:, perm]) and np.array_equal(s1, s0)


def test_invariant_colwise_is_rowwise_of_transpose(orc):
    """I3: the 128x1 quantization of X equals the 1x128 quantization of X^T."""
    xb = _random_bf16((256, 384), seed=19)
    qt, st = orc.quant_colwise(xb)
    q, s = orc.quant_rowwise(np.ascontiguousarray(xb.T))
    assert np.array_equal(qt, q) and np.array_equal(st, s)


# ---------------------------------------------------------------- GEMM ----

def _random_codes(shape, seed):
    c = _rng(seed).integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)   # no NaN codes


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 128, 256), (128, 256, 256)])
def test_gemm_brute_force_tiny(orc, mode, M, N, K):
    """Brute force: sum over k of dec(a)*sA*dec(b)*sB in float64; the oracle's
    FP32 accumulation stays within 1e-6 relative (Frobenius)."""
    rng = _rng(M + N + K + mode)
    a = _random_codes((M, K), 1)
    b = _random_codes((N, K), 2)
    sa = rng.uniform(0.001, 0.01, (K // 128, M)).astype(np.float32)
    if mode == 0:
        sb = rng.uniform(1e-4, 1e-3, (N // 128, K // 128)).astype(np.float32)
    elif mode == 1:
        sb = rng.uniform(1e-4, 1e-3, (K // 128, N // 128)).astype(np.float32)
    else:
        sb = rng.uniform(1e-4, 1e-3, (K // 128, N)).astype(np.float32)
    c, c64 = orc.gemm_blockscaled(mode, a, sa, b, sb, with_f64=True)
    exp = ref.gemm_brute(mode, a, sa, b, sb)
    assert orc.rel_fro(c, exp) < 1e-6
    assert orc.rel_fro(c64, exp) < 1e-12
    # the element-list entry point computes the same values
    ii = rng.integers(0, M, 50)
    jj = rng.integers(0, N, 50)
    assert np.array_equal(orc.gemm_blockscaled_at(mode, a, sa, b, sb, ii, jj), c[ii, jj])


def test_gemm_closed_form_scaled_identity(orc):
    """W = 3.5 I: diagonal blocks have amax 3.5, s = 2^-7, codes 0x7E;
    off-diagonal blocks are zero.  Y = X W^T = 3.5 * dequant(X) with exactly
    one FP32 rounding."""
    xb = _random_bf16((256, 384), seed=23)
    w = np.zeros((384, 384), np.float32)
    np.fill_diagonal(w, 3.5)
    wb = _bf16_bits_from_f32(w)
    qx, sx = orc.quant_rowwise(xb)
    qw, _, sw = orc.quant_weight(wb)
    assert np.all(sw[np.eye(3, dtype=bool)] == 2.0 ** -7) and np.all(sw[~np.eye(3, dtype=bool)] == 0)
    y = orc.gemm_blockscaled(0, qx, sx, qw, sw)
    s_full = np.repeat(sx.T, 128, axis=1).astype(np.float64)
    exp = (3.5 * ref.decode(qx) * s_full).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_gemm_single_nonzero_kblock_indexes_scales(orc, mode):
    """Only K-block 2 of 4 holds non-zero codes: the result is one term,
    RN32(P) * RN32(sA[2][i] * sB(j, 2)), which exposes a wrong scale index."""
    M, N, K = 128, 256, 512
    rng = _rng(29 + mode)
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[:, 256:384] = _random_codes((M, 128), 3)
    b[:, 256:384] = _random_codes((N, 128), 4)
    sa = rng.uniform(1, 2, (4, M)).astype(np.float32)
    if mode == 0:
        sb = rng.uniform(1, 2, (N // 128, 4)).astype(np.float32)
        sbj = np.repeat(sb[:, 2], 128)
    elif mode == 1:
        sb = rng.uniform(1, 2, (4, N // 128)).astype(np.float32)
        sbj = np.repeat(sb[2], 128)
    else:
        sb = rng.uniform(1, 2, (4, N)).astype(np.float32)
        sbj = sb[2]
    c = orc.gemm_blockscaled(mode, a, sa, b, sb)
    P = ref.decode(a[:, 256:384]) @ ref.decode(b[:, 256:384]).T
    exp = P.astype(np.float32) * (sa[2][:, None] * sbj[None, :]).astype(np.float32)
    assert np.array_equal(c, exp)


def test_gemm_lossless_inputs_match_exact_matmul(orc):
    """Inputs chosen so quantization is lossless (every tile has amax
    448 * 2^j and E4M3-representable entries after dividing by 2^j): the
    quantized GEMM equals the exact bf16 matmul up to FP32 accumulation."""
    rng = _rng(31)
    t = ref.e4m3_table()
    def lossless(shape, j):
        v = rng.choice(t, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v[..., ::128] = 448.0                  # every tile / block reaches amax
        return _bf16_bits_from_f32((v * 2.0 ** j).astype(np.float32))
    xb = lossless((256, 512), -4)
    wb = lossless((256, 512), -9)
    wb_blocks = ref.bf16_widen(wb)
    assert np.abs(wb_blocks).max() == np.float32(448 * 2.0 ** -9)
    qx, sx = orc.quant_rowwise(xb)
    qw, _, sw = orc.quant_weight(wb)
    assert np.array_equal(ref.decode(qx) * np.repeat(sx.T, 128, axis=1), ref.bf16_widen(xb))
    y = orc.gemm_blockscaled(0, qx, sx, qw, sw)
    exact = ref.bf16_widen(xb).astype(np.float64) @ ref.bf16_widen(wb).astype(np.float64).T
    assert orc.rel_fro(y, exact) < 1e-6
    assert np.allclose(orc.matmul_ref(xb, wb), exact, rtol=0, atol=0)


def test_invariant_dgrad_equals_fwd_on_transposed_weight(orc):
    """I5: DGRAD(dY, W^T codes, s_W) == FWD(dY, quant(W^T)) bitwise."""
    dyb = _random_bf16((256, 384), scale=1e-3, seed=37)
    wb = _random_bf16((384, 256), scale=0.02, seed=38)        # W [out=384, in=256]
    qdy, sdy = orc.quant_rowwise(dyb)
    qw, qwt, sw = orc.quant_weight(wb)
    d1 = orc.gemm_blockscaled(1, qdy, sdy, qwt, sw)
    qwT, _, swT = orc.quant_weight(np.ascontiguousarray(wb.T))
    assert np.array_equal(qwT, qwt)
    d2 = orc.gemm_blockscaled(0, qdy, sdy, qwT, swT)
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))


def test_matmul_ref_against_numpy(orc):
    xb = _random_bf16((96, 256), seed=41)
    yb = _random_bf16((64, 256), seed=42)
    x = ref.bf16_widen(xb).astype(np.float64)
    y = ref.bf16_widen(yb).astype(np.float64)
    assert np.allclose(orc.matmul_ref(xb, yb), x @ y.T, rtol=1e-13, atol=1e-12)
    assert np.allclose(orc.matmul_ref(np.ascontiguousarray(xb.T), yb, x_trans=True), x @ y.T,
                       rtol=1e-13, atol=1e-12)
    assert np.allclose(orc.matmul_ref(xb, np.ascontiguousarray(yb.T), y_trans=True), x @ y.T,
                       rtol=1e-13, atol=1e-12)


def test_bf16_rounding_matches_torch(orc):
    """FP32 -> bf16 RNE agrees with torch's conversion (a library routine)
    on random values, exact ties and the extremes."""
    import torch
    rng = _rng(43)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    ties = ((rng.integers(0, 2 ** 16, 1000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[~np.isnan(ties)]
    v = np.concatenate([v, ties, np.array([0.0, -0.0, 3.4028235e38, -3.4028235e38, 1e-45], np.float32)])
    got = orc.f32_to_bf16_bits(v)
    exp = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, exp)
