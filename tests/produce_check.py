"""Checks of quantize-on-produce outputs against the oracle.

The oracle evaluates each neighbour op in double and rounds once to bf16 (y).
A device evaluating the op in FP32 may return any bf16 value between lo and
hi (the roundings of the two ends of its error band; lo == hi == y where one
result is correct).  The operand the path quantizes is the op's bf16 output,
so:

  * a bf16 output element is correct when it lies in [lo, hi];
  * a tile (1x128 along a row, or 128x1 along a column) whose elements all
    have one correct value has exactly one correct (scale, codes): the
    oracle's quantization of y, compared bit for bit;
  * in any other tile the device's scale must be that of an attainable tile
    amax a (an element's band reaches magnitude a, and no element's band
    stays above it), and every code must lie between the codes the oracle
    gives lo and hi of its element at that amax.
"""
from __future__ import annotations

import numpy as np

import oracle


def row_tiles(a: np.ndarray) -> np.ndarray:
    """[rows, cols] -> [rows * cols/128, 128], tile (r, cb) at r * ncb + cb."""
    rows, cols = a.shape
    return np.ascontiguousarray(a.reshape(rows, cols // 128, 128).reshape(-1, 128))


def col_tiles(a: np.ndarray) -> np.ndarray:
    """[rows, cols] (rows zero-padded to a multiple of 128) -> [cols * nrb,
    128], tile (c, rb) at c * nrb + rb, elements in row order."""
    rows, cols = a.shape
    rp = (rows + 127) // 128 * 128
    pad = np.zeros((rp, cols), a.dtype)
    pad[:rows] = a
    return np.ascontiguousarray(pad.T.reshape(cols * (rp // 128), 128))


def _key(bits: np.ndarray, sign: int) -> np.ndarray:
    """Sign-magnitude bit patterns -> integers in value order (both zeros 0)."""
    b = np.asarray(bits).astype(np.int64)
    mag = b & (sign - 1)
    return np.where(b & sign, -mag, mag)


def _between(got, lo, hi, sign: int) -> np.ndarray:
    """got lies in [lo, hi] by value; a zero's sign must be reachable: -0 needs
    lo to carry the sign bit, +0 needs hi without it."""
    got = np.asarray(got).astype(np.int64)
    lo = np.asarray(lo).astype(np.int64)
    hi = np.asarray(hi).astype(np.int64)
    k = _key(got, sign)
    ok = (_key(lo, sign) <= k) & (k <= _key(hi, sign))
    ok &= (got != sign) | ((lo & sign) != 0)
    ok &= (got != 0) | ((hi & sign) == 0)
    return ok


def _widen(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f32(np.asarray(bits, np.uint16))


def check_tiles(ty, tlo, thi, codes, scales) -> dict:
    """ty, tlo, thi: uint16 [T, 128] oracle values; codes: uint8 [T, 128] and
    scales: float32 [T] from the device.  Returns counts and the indices of
    the tiles that match no correct result."""
    ty = np.ascontiguousarray(ty, np.uint16)
    tlo = np.ascontiguousarray(tlo, np.uint16)
    thi = np.ascontiguousarray(thi, np.uint16)
    codes = np.ascontiguousarray(codes, np.uint8)
    sdev = np.ascontiguousarray(scales, np.float32)
    band = tlo != thi
    tile_band = band.any(axis=1)
    bad = []
    uniq = np.nonzero(~tile_band)[0]
    if uniq.size:
        q, s = oracle.quant_rowwise(ty[uniq])
        ok = (q == codes[uniq]).all(axis=1) & (s[0].view(np.uint32) == sdev[uniq].view(np.uint32))
        bad.extend(int(i) for i in uniq[~ok])
    amb = np.nonzero(tile_band)[0]
    if amb.size:
        lo_v = _widen(tlo[amb]).astype(np.float64)
        hi_v = _widen(thi[amb]).astype(np.float64)
        crosses = (lo_v <= 0) & (hi_v >= 0)
        mag_lo = np.where(crosses, 0.0, np.minimum(np.abs(lo_v), np.abs(hi_v)))
        mag_hi = np.maximum(np.abs(lo_v), np.abs(hi_v))
        # the amax the device's scale stands for: the bf16 value a with
        # RN32(a / 448) equal to that scale
        s = sdev[amb]
        a = _widen(np.array([oracle.f64_to_bf16(float(v) * 448.0) & 0x7FFF for v in s],
                            np.uint16))
        a_scale = np.array([oracle.tile_scale(float(v)) for v in a], np.float32)
        a64 = a.astype(np.float64)[:, None]
        ok = a_scale.view(np.uint32) == s.view(np.uint32)
        ok &= (mag_lo.max(axis=1) <= a64[:, 0]) & (a64[:, 0] <= mag_hi.max(axis=1))
        ok &= ((mag_lo <= a64) & (a64 <= mag_hi)).any(axis=1)
        amax = np.repeat(a[:, None], 128, axis=1)
        c_lo = oracle.quant_elems(_widen(tlo[amb]), amax)
        c_hi = oracle.quant_elems(_widen(thi[amb]), amax)
        ok &= _between(codes[amb], c_lo, c_hi, 0x80).all(axis=1)
        bad.extend(int(i) for i in amb[~ok])
    return {"tiles": int(ty.shape[0]), "ambiguous": int(amb.size), "bad": sorted(bad)}


def check_bf16(got: np.ndarray, lo: np.ndarray, hi: np.ndarray) -> int:
    """Number of bf16 output elements outside their correct range."""
    return int(np.count_nonzero(~_between(got, lo, hi, 0x8000)))


def check_outputs(out: dict, y: np.ndarray, lo: np.ndarray, hi: np.ndarray, rows: int) -> dict:
    """out: host copies of the device outputs that were requested ('q', 's',
    'qt', 'st', 'y' as numpy arrays).  y, lo, hi: oracle [rows, cols]."""
    res = {}
    if "y" in out:
        res["bf16_wrong"] = check_bf16(out["y"], lo, hi)
    if "q" in out:
        res["row"] = check_tiles(row_tiles(y), row_tiles(lo), row_tiles(hi), row_tiles(out["q"]),
                                 np.ascontiguousarray(out["s"].T).ravel())
    if "qt" in out:
        cols = y.shape[1]
        qt = out["qt"]                                   # [cols, rows_pad]
        res["col"] = check_tiles(col_tiles(y), col_tiles(lo), col_tiles(hi),
                                 np.ascontiguousarray(qt.reshape(cols * (qt.shape[1] // 128), 128)),
                                 np.ascontiguousarray(out["st"].T).ravel())
        # the padding rows of the transposed copy hold zero codes
        if qt.shape[1] > rows:
            res["pad_nonzero"] = int(np.count_nonzero(qt[:, rows:]))
    return res


def all_ok(res: dict) -> bool:
    ok = res.get("bf16_wrong", 0) == 0 and res.get("pad_nonzero", 0) == 0
    for k in ("row", "col"):
        if k in res:
            ok = ok and not res[k]["bad"]
    return ok
