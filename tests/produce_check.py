"""Checks of quantize-on-produce outputs against the oracle.

The oracle evaluates each neighbour op in double and rounds once to bf16 (y);
where a device evaluating the op in FP32 may land on the other side of a bf16
rounding boundary it also gives that other result (y_alt).  The operand the
path quantizes is the op's bf16 output, so:

  * a bf16 output element is correct when it equals y or y_alt;
  * a tile (1x128 along a row, or 128x1 along a column) whose elements all
    have one correct value has exactly one correct (scale, codes): the
    oracle's quantization of y, compared bit for bit;
  * a tile holding k elements with two correct values has up to 2^k correct
    (scale, codes); the device's must equal the oracle's quantization of one
    of those 2^k bf16 tiles (enumerated for k <= MAX_ENUM).  For larger k
    (not expected at the tolerances used) the tile is reported, not passed.
"""
from __future__ import annotations

import numpy as np

import oracle

MAX_ENUM = 10


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


def check_tiles(ty: np.ndarray, talt: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> dict:
    """ty, talt: uint16 [T, 128] oracle values; codes: uint8 [T, 128] and
    scales: float32 [T] from the device.  Returns counts and the indices of
    tiles that match no correct result."""
    ty = np.ascontiguousarray(ty, np.uint16)
    talt = np.ascontiguousarray(talt, np.uint16)
    codes = np.ascontiguousarray(codes, np.uint8)
    sbits = np.ascontiguousarray(scales, np.float32).view(np.uint32)
    amb = ty != talt
    tile_amb = amb.any(axis=1)
    bad = []
    uniq = np.nonzero(~tile_amb)[0]
    if uniq.size:
        q, s = oracle.quant_rowwise(ty[uniq])
        ok = (q == codes[uniq]).all(axis=1) & (s[0].view(np.uint32) == sbits[uniq])
        bad.extend(int(i) for i in uniq[~ok])
    too_many = 0
    for t in np.nonzero(tile_amb)[0]:
        idx = np.nonzero(amb[t])[0]
        k = idx.size
        if k > MAX_ENUM:
            too_many += 1
            bad.append(int(t))
            continue
        pick = ((np.arange(1 << k)[:, None] >> np.arange(k)) & 1).astype(bool)
        cand = np.repeat(ty[t][None, :], 1 << k, axis=0)
        cand[:, idx] = np.where(pick, talt[t, idx][None, :], ty[t, idx][None, :])
        q, s = oracle.quant_rowwise(cand)
        ok = (q == codes[t][None, :]).all(axis=1) & (s[0].view(np.uint32) == sbits[t])
        if not ok.any():
            bad.append(int(t))
    return {"tiles": int(ty.shape[0]), "ambiguous": int(tile_amb.sum()),
            "too_many": too_many, "bad": bad}


def check_bf16(got: np.ndarray, y: np.ndarray, y_alt: np.ndarray) -> int:
    """Number of bf16 output elements equal to neither correct value."""
    got = np.asarray(got, np.uint16)
    return int(np.count_nonzero((got != y) & (got != y_alt)))


def check_outputs(out: dict, y: np.ndarray, y_alt: np.ndarray, rows: int) -> dict:
    """out: host copies of the device outputs that were requested ('q', 's',
    'qt', 'st', 'y' as numpy arrays).  y, y_alt: oracle [rows, cols]."""
    res = {}
    if "y" in out:
        res["bf16_wrong"] = check_bf16(out["y"], y, y_alt)
    if "q" in out:
        res["row"] = check_tiles(row_tiles(y), row_tiles(y_alt), row_tiles(out["q"]),
                                 np.ascontiguousarray(out["s"].T).ravel())
    if "qt" in out:
        cols = y.shape[1]
        qt = out["qt"]                                   # [cols, rows_pad]
        res["col"] = check_tiles(col_tiles(y), col_tiles(y_alt),
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
