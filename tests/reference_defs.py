"""Independent restatements used to pin the oracle (test-only, numpy).

These are written from the format and scale definitions with different
machinery than the oracle's C code (sorted-table nearest search instead of
bit construction; float64 division with explicit 24-bit rounding instead of
binary32 operations), so that an error in either shows up as a mismatch.
"""
from __future__ import annotations

import numpy as np


def e4m3_table() -> np.ndarray:
    """The 127 finite non-negative E4M3 values in increasing order; index i is
    the code of the i-th smallest magnitude (OCP OFP8 E4M3 definition)."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for e in range(-6, 9):
        for m in range(8):
            v = (1 + m / 8) * 2.0 ** e
            if v <= 448.0:
                vals.append(v)
    t = np.array(sorted(vals), dtype=np.float64)
    assert t.size == 127
    return t


_TABLE = e4m3_table()


def nearest_code(v) -> np.ndarray:
    """Nearest E4M3 code by table search; ties to the even code; |v| > 448
    saturates; sign bit 0x80 from the sign of v (so -0.0 -> 0x80)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    lo = np.searchsorted(_TABLE, a, side="right") - 1
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    dl = a - _TABLE[lo]
    dh = _TABLE[hi] - a
    pick_hi = (hi != lo) & ((dh < dl) | ((dh == dl) & (hi % 2 == 0)))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a > 448.0, 126, code).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return code | sign


def round24(q: np.ndarray) -> np.ndarray:
    """Round positive float64 values to 24 significant bits (half to even)
    with an unbounded exponent range; returned as float64."""
    m, e = np.frexp(q)
    return np.ldexp(np.round(m * 2.0 ** 24) / 2.0 ** 24, e)


def scale_def(amax) -> np.ndarray:
    """s = RN32(amax / 448): float64 quotient (53 bits >= 2*24+2, so the
    second rounding to binary32 is innocuous), cast to float32."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    return (a / 448.0).astype(np.float32)


def scaled_def(x, amax) -> np.ndarray:
    """v = RN32(x * RN(448/amax)) with an unbounded exponent for the
    reciprocal; amax == 0 gives x * 0."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    safe = np.where(a > 0, a, 1.0)
    r = round24(448.0 / safe)
    v = np.where(a > 0, x * r, x * 0.0)          # exact product in float64
    return v.astype(np.float32)


def quant_def(x, amax) -> np.ndarray:
    return nearest_code(scaled_def(x, amax))


def decode(codes) -> np.ndarray:
    """Exact value of each code from the sorted table (sign from bit 7)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag_idx = (c & 0x7F).astype(np.int64)
    out = np.where(mag_idx <= 126, _TABLE[np.minimum(mag_idx, 126)], np.nan)
    return np.where(c & 0x80, -out, out)


def ulp_e4m3(v) -> np.ndarray:
    """Spacing of E4M3 values around |v| (the binade's step; 2^-9 below the
    smallest normal)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    e = np.minimum(e, 8)
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def bf16_widen(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rowwise_def(xb: np.ndarray):
    """1x128 tiles along columns: (q [R, C], s [C/128, R])."""
    x = bf16_widen(xb)
    R, C = x.shape
    t = x.reshape(R, C // 128, 128)
    amax = np.abs(t).max(axis=2)                         # [R, C/128]
    q = quant_def(t, amax[:, :, None]).reshape(R, C)
    return q, scale_def(amax).T.copy()


def colwise_def(xb: np.ndarray):
    """128x1 tiles along rows, transposed codes: (qt [C, Rp], st [Rp/128, C])."""
    x = bf16_widen(xb)
    R, C = x.shape
    Rp = (R + 127) // 128 * 128
    xp = np.zeros((Rp, C), np.float32)
    xp[:R] = x
    t = xp.reshape(Rp // 128, 128, C)
    amax = np.abs(t).max(axis=1)                         # [Rp/128, C]
    q = quant_def(t, amax[:, None, :]).reshape(Rp, C)
    q[R:] = 0
    return q.T.copy(), scale_def(amax)


def weight_def(wb: np.ndarray):
    """128x128 blocks: (q [N, K], s [N/128, K/128])."""
    w = bf16_widen(wb)
    N, K = w.shape
    t = w.reshape(N // 128, 128, K // 128, 128)
    amax = np.abs(t).max(axis=(1, 3))                    # [N/128, K/128]
    q = quant_def(t, amax[:, None, :, None]).reshape(N, K)
    return q, scale_def(amax)


def gemm_brute(mode: int, a, sa, b, sb) -> np.ndarray:
    """Sum over K-blocks of P_kb * sA * sB in float64 (dequantized per block)."""
    a = decode(a)
    b = decode(b)
    M, K = a.shape
    N = b.shape[0]
    out = np.zeros((M, N), np.float64)
    for kb in range(K // 128):
        P = a[:, kb * 128:(kb + 1) * 128] @ b[:, kb * 128:(kb + 1) * 128].T
        sA = sa[kb].astype(np.float64)[:, None]
        if mode == 0:
            sB = sb[:, kb].astype(np.float64).repeat(128)[None, :N]
        elif mode == 1:
            sB = sb[kb].astype(np.float64).repeat(128)[None, :N]
        else:
            sB = sb[kb].astype(np.float64)[None, :]
        out += P * sA * sB
    return out
