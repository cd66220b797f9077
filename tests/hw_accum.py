"""Element-wise error bound of the GPU's FP8 matrix-core accumulation.

Measured property of the gfx950 FP8 MFMA (see the probe tests and the design
notes): inside one instruction the 128 products of a K-block are summed in
groups of 8 consecutive k; within a group every product is aligned to the
largest one and truncated toward zero below 2^(E_g - 13), where E_g is the
exponent of the group's largest |product|; group sums and the accumulator
input are combined in FP32.  So for one output element

    |P_hw - P_exact| <= sum over groups g of 8 * 2^(E_g - 13)

per K-block, and the kernel's result differs from the oracle's by at most

    sum_kb |sA * sB| * (8 * sum_g 2^(E_g - 13) + 2^-20 * sum_k |p_k|)
      + 2^-20 * (number of K-blocks) * |ref|

(the 2^-20 terms cover every FP32 rounding of the MFMA's group sums, the
scale product and the accumulation, with margin).  An indexing or scaling
mistake in the kernel shows up as an error of the order of the products
themselves, far above this bound.

The worst case adds every truncation with the same sign.  The truncation
errors of different products are bounded (|d| < 2^(E_g - 13)) and their signs
follow the products' signs, so their sum behaves like a random walk:
statistical_bound() returns 8 standard deviations of that sum (variance
q^2/3 per product) plus the same rounding terms.  It decides on which
elements the stated max-element gate is attainable by the hardware at all.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

_DEC32 = None


def _dec32():
    """E4M3 decode table in float32: every E4M3 value, and every product of
    two of them (|p| from 2^-18 to 448^2 < 2^18, at most 8 significant bits),
    is exact in float32."""
    global _DEC32
    if _DEC32 is None:
        _DEC32 = oracle.e4m3_decode_table().astype(np.float32)
    return _DEC32


def element_bound(mode: int, a: np.ndarray, sa: np.ndarray, b: np.ndarray, sb: np.ndarray,
                  ii: np.ndarray, jj: np.ndarray, ref: np.ndarray, chunk: int = 1024) -> np.ndarray:
    """Worst-case bound on |C_gpu - C_oracle| for the elements (ii[t], jj[t])."""
    return _bounds(mode, a, sa, b, sb, ii, jj, ref, chunk)[0]


def statistical_bound(mode: int, a, sa, b, sb, ii, jj, ref, chunk: int = 1024) -> np.ndarray:
    """8-sigma bound of the accumulated truncation error (plus rounding)."""
    return _bounds(mode, a, sa, b, sb, ii, jj, ref, chunk)[1]


def bounds(mode: int, a, sa, b, sb, ii, jj, ref, chunk: int = 1024):
    """(worst-case bound, 8-sigma bound) for the elements (ii[t], jj[t])."""
    return _bounds(mode, a, sa, b, sb, ii, jj, ref, chunk)


def _bounds(mode, a, sa, b, sb, ii, jj, ref, chunk):
    dec = _dec32()
    K = a.shape[1]
    KB = K // 128
    out = np.empty(len(ii), np.float64)
    stat = np.empty(len(ii), np.float64)

    def one_chunk(s0):
        i = np.asarray(ii[s0:s0 + chunk])
        j = np.asarray(jj[s0:s0 + chunk])
        p = np.abs(dec[a[i]] * dec[b[j]])                  # [S, K] exact |products|
        S = p.shape[0]
        gmax = p.reshape(S, K // 8, 8).max(axis=2)
        # gmax = f * 2^e with f in [0.5, 1): the group's largest product has
        # exponent E_g = e - 1, and the truncation quantum is 2^(E_g - 13)
        e = np.frexp(gmax)[1]
        quantum = np.where(gmax > 0, np.ldexp(1.0, e - 14), 0.0)   # [S, K/8], float64
        blk_trunc = 8.0 * quantum.reshape(S, KB, 16).sum(axis=2)   # [S, KB]
        # exact in float64 in any order: multiples of 2^-18 below 2^25
        blk_abs = p.reshape(S, KB, 128).sum(axis=2, dtype=np.float64)
        sA = sa[:, i].T.astype(np.float64)                          # [S, KB]
        if mode == 0:
            sB = sb[j // 128, :].astype(np.float64)
        elif mode == 1:
            sB = sb[:, j // 128].T.astype(np.float64)
        else:
            sB = sb[:, j].T.astype(np.float64)
        sc = np.abs(sA * sB)
        rounding = ((sc * 2.0 ** -20 * blk_abs).sum(axis=1)
                    + 2.0 ** -20 * KB * np.abs(ref[s0:s0 + chunk]))
        out[s0:s0 + chunk] = (sc * blk_trunc).sum(axis=1) + rounding
        var = (sc ** 2 * (8.0 / 3.0) * (quantum ** 2).reshape(S, KB, 16).sum(axis=2)).sum(axis=1)
        stat[s0:s0 + chunk] = 8.0 * np.sqrt(var) + rounding

    # chunks are independent (each writes its own slice); numpy releases the
    # GIL inside these loops, so threads share the work
    starts = range(0, len(ii), chunk)
    workers = min(16, os.cpu_count() or 1, max(1, len(starts)))
    if workers > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one_chunk, starts))
    else:
        for s0 in starts:
            one_chunk(s0)
    return out, stat
