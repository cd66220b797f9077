"""CPU oracle for the fine-grained block-quantized FP8 linear layer.

TEST INFRASTRUCTURE ONLY.  This package is the ground truth that the HIP
library is checked against.  Only ``tests/``, the smoke check and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product package
never does, and this package never imports the product package.

The arithmetic lives in ``puro_oracle.c`` (plain C, built here with gcc);
this module only compiles it and marshals numpy arrays through ctypes.  What
each function computes, and which passage of the pages it follows, is stated
in ``puro_oracle.h``:

* "Puro-2B" arXiv report, section 2.1 (Pipeline at a Glance), and the
  training.farm blog, FP8 section: main linear-layer GEMMs in blockwise FP8,
  DeepSeek-V3-style fine-grained block quantization; sensitive ops and state
  stay in BF16/FP32.
* the bit.fan article, section "FP8 training and its trade-off": the same
  statement (quantization tiles for the major linear layers).

Parity status of each function (what pins it) is listed in the tests:
``tests/test_oracle_pins.py`` and ``tests/test_oracle_exhaustive.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "puro_oracle.c")
_LIB = os.path.join(_HERE, "libpuro_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra",
           "-Wno-unused-parameter"]

_lock = threading.Lock()
_lib = None

MODE_FWD, MODE_DGRAD, MODE_WGRAD = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (always recompiles when ``force``)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_decode.restype = ctypes.c_double
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_encode_range.restype = None
        lib.orc_e4m3_encode_range.argtypes = [ctypes.c_uint32, I64, P]
        lib.orc_tile_scale.restype = ctypes.c_float
        lib.orc_tile_scale.argtypes = [ctypes.c_float]
        lib.orc_scaled_value.restype = ctypes.c_float
        lib.orc_scaled_value.argtypes = [ctypes.c_float, ctypes.c_float]
        lib.orc_quant_elem.restype = ctypes.c_uint8
        lib.orc_quant_elem.argtypes = [ctypes.c_float, ctypes.c_float]
        lib.orc_quant_elems.restype = None
        lib.orc_quant_elems.argtypes = [P, P, I64, P]
        for name in ("orc_quant_rowwise", "orc_quant_colwise"):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = [P, I64, I64, P, P]
        lib.orc_quant_weight.restype = ctypes.c_int
        lib.orc_quant_weight.argtypes = [P, I64, I64, P, P, P]
        lib.orc_gemm_blockscaled.restype = ctypes.c_int
        lib.orc_gemm_blockscaled.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, P,
                                             P, P, I64, I64]
        lib.orc_gemm_blockscaled_at.restype = ctypes.c_int
        lib.orc_gemm_blockscaled_at.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, P,
                                                P, P, I64, P]
        lib.orc_matmul_ref.restype = ctypes.c_int
        lib.orc_matmul_ref.argtypes = [I64, I64, I64, P, I64, I64, P, I64, I64, P, I64, I64]
        lib.orc_f32_to_bf16.restype = ctypes.c_uint16
        lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_bf16_array.restype = None
        lib.orc_f32_to_bf16_array.argtypes = [P, I64, P]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_swiglu_fwd.restype = ctypes.c_int
        lib.orc_swiglu_fwd.argtypes = [P, I64, I64, ctypes.c_double, P, P, P]
        lib.orc_swiglu_bwd.restype = ctypes.c_int
        lib.orc_swiglu_bwd.argtypes = [P, P, I64, I64, ctypes.c_double, P, P, P]
        lib.orc_rmsnorm_bwd.restype = ctypes.c_int
        lib.orc_rmsnorm_bwd.argtypes = [P, P, P, P, P, I64, I64, ctypes.c_double, P, P, P]
        lib.orc_residual_add.restype = ctypes.c_int
        lib.orc_residual_add.argtypes = [P, P, I64, P]
        lib.orc_rmsnorm_fwd.restype = ctypes.c_int
        lib.orc_rmsnorm_fwd.argtypes = [P, P, I64, I64, ctypes.c_double, ctypes.c_double, P, P, P,
                                        P]
        lib.orc_swiglu_point.restype = None
        lib.orc_swiglu_point.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, P]
        lib.orc_bf16_band.restype = None
        lib.orc_bf16_band.argtypes = [ctypes.c_double, ctypes.c_double, P]
        lib.orc_set_threads.restype = None
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_get_threads.restype = ctypes.c_int
        lib.orc_get_threads.argtypes = []
        _lib = lib
        return lib


def lib():
    """The loaded ctypes handle (for tests that call C entry points directly)."""
    return _load()


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments")


# ---- scalar codec ----------------------------------------------------------

def e4m3_encode(v: float) -> int:
    return int(_load().orc_e4m3_encode(float(v)))


def e4m3_decode(code: int) -> float:
    return float(_load().orc_e4m3_decode(int(code)))


def e4m3_decode_table() -> np.ndarray:
    """float64[256]: the exact value of every code (NaN for 0x7F/0xFF)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode_range(first_bits: int, n: int) -> np.ndarray:
    """Codes of the binary32 values with bit patterns first_bits .. +n-1."""
    out = np.empty(int(n), np.uint8)
    _load().orc_e4m3_encode_range(int(first_bits) & 0xFFFFFFFF, int(n), _ptr(out))
    return out


def tile_scale(amax: float) -> float:
    return float(_load().orc_tile_scale(float(amax)))


def scaled_value(x: float, amax: float) -> float:
    return float(_load().orc_scaled_value(float(x), float(amax)))


def quant_elem(x: float, amax: float) -> int:
    return int(_load().orc_quant_elem(float(x), float(amax)))


def quant_elems(x: np.ndarray, amax: np.ndarray) -> np.ndarray:
    """Elementwise quant_elem over float32 arrays of one shape."""
    x = _c(np.asarray(x, np.float32), np.float32)
    amax = _c(np.broadcast_to(np.asarray(amax, np.float32), x.shape), np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_quant_elems(_ptr(x), _ptr(amax), x.size, _ptr(out))
    return out


# ---- quantizers ------------------------------------------------------------

def quant_rowwise(x_bits: np.ndarray):
    """x_bits: uint16 [rows, cols] bf16 bit patterns -> (q u8 [rows, cols],
    s f32 [cols/128, rows])."""
    x = _c(x_bits, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((cols // 128, rows), np.float32)
    _check(_load().orc_quant_rowwise(_ptr(x), rows, cols, _ptr(q), _ptr(s)), "quant_rowwise")
    return q, s


def quant_colwise(x_bits: np.ndarray):
    """x_bits: uint16 [rows, cols] -> (qt u8 [cols, rows_pad],
    st f32 [rows_pad/128, cols]); rows_pad = ceil(rows/128)*128."""
    x = _c(x_bits, np.uint16)
    rows, cols = x.shape
    rp = (rows + 127) // 128 * 128
    qt = np.empty((cols, rp), np.uint8)
    st = np.empty((rp // 128, cols), np.float32)
    _check(_load().orc_quant_colwise(_ptr(x), rows, cols, _ptr(qt), _ptr(st)), "quant_colwise")
    return qt, st


def quant_weight(w_bits: np.ndarray, transpose: bool = True):
    """w_bits: uint16 [n, k] -> (q u8 [n, k], qt u8 [k, n] or None,
    s f32 [n/128, k/128])."""
    w = _c(w_bits, np.uint16)
    n, k = w.shape
    q = np.empty((n, k), np.uint8)
    qt = np.empty((k, n), np.uint8) if transpose else None
    s = np.empty((n // 128, k // 128), np.float32)
    _check(_load().orc_quant_weight(_ptr(w), n, k, _ptr(q), _ptr(qt), _ptr(s)), "quant_weight")
    return q, qt, s


# ---- GEMM ------------------------------------------------------------------

def gemm_blockscaled(mode: int, a: np.ndarray, sa: np.ndarray, b: np.ndarray,
                     sb: np.ndarray, rows=None, with_f64: bool = False):
    """C = sum_kb RN32(P_kb) * RN32(sA*sB), FP32 accumulation (see header).

    a: u8 [M, K]; b: u8 [N, K]; sa: f32 [K/128, M]; sb per mode.  ``rows`` =
    (begin, end) restricts the output to those rows of C.  Returns float32
    [rows, N] (and the float64-accumulated variant if ``with_f64``)."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("K mismatch")
    r0, r1 = (0, M) if rows is None else rows
    c = np.empty((r1 - r0, N), np.float32)
    c64 = np.empty((r1 - r0, N), np.float64) if with_f64 else None
    _check(_load().orc_gemm_blockscaled(mode, M, N, K, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                                        _ptr(c), _ptr(c64), r0, r1), "gemm_blockscaled")
    return (c, c64) if with_f64 else c


def gemm_blockscaled_at(mode: int, a, sa, b, sb, ii, jj) -> np.ndarray:
    """The same sum for the output elements (ii[t], jj[t])."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    ii = _c(np.asarray(ii, dtype=np.int64), np.int64)
    jj = _c(np.asarray(jj, dtype=np.int64), np.int64)
    M, K = a.shape
    N = b.shape[0]
    out = np.empty(ii.shape[0], np.float32)
    _check(_load().orc_gemm_blockscaled_at(mode, M, N, K, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                                           _ptr(ii), _ptr(jj), ii.shape[0], _ptr(out)),
           "gemm_blockscaled_at")
    return out


def matmul_ref(x_bits: np.ndarray, y_bits: np.ndarray, x_trans: bool = False,
               y_trans: bool = False, rows=None) -> np.ndarray:
    """Unquantized reference in float64 over bf16 inputs:
    R = op(X) @ op(Y)^T with op(X) [M, K] and op(Y) [N, K]; ``x_trans`` means
    X is stored [K, M], ``y_trans`` means Y is stored [K, N]."""
    x = _c(x_bits, np.uint16)
    y = _c(y_bits, np.uint16)
    if x_trans:
        K, M = x.shape
        xs_i, xs_k = 1, M
    else:
        M, K = x.shape
        xs_i, xs_k = K, 1
    if y_trans:
        Ky, N = y.shape
        ys_j, ys_k = 1, N
    else:
        N, Ky = y.shape
        ys_j, ys_k = Ky, 1
    if Ky != K:
        raise ValueError("K mismatch")
    r0, r1 = (0, M) if rows is None else rows
    r = np.empty((r1 - r0, N), np.float64)
    _check(_load().orc_matmul_ref(M, N, K, _ptr(x), xs_i, xs_k, _ptr(y), ys_j, ys_k,
                                  _ptr(r), r0, r1), "matmul_ref")
    return r


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().orc_f32_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: the top half of the word)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16(v: float) -> int:
    """bf16 bit pattern of a double, rounded once to nearest even."""
    return int(_load().orc_f64_to_bf16(float(v)))


def bf16_band(v: float, band: float):
    """(y, lo, hi) for one value: y its bf16 rounding, lo and hi the roundings
    of v - band and v + band."""
    out = np.empty(3, np.uint16)
    _load().orc_bf16_band(float(v), float(band), _ptr(out))
    return int(out[0]), int(out[1]), int(out[2])


# ---- neighbour ops (quantize-on-produce) -------------------------------------
# The op runs in double and is rounded once to bf16 (y); a device evaluating
# it in FP32 within tol * M may return any bf16 value between lo and hi (both
# included; lo == hi == y where only one result is correct).  What the path
# then quantizes is the bf16 tensor, exactly as quant_rowwise / quant_colwise
# do.

def swiglu_point(g: float, u: float, dh: float = 0.0):
    """Unrounded (h, d_gate, d_up, M_gate) at one point, in double."""
    out = np.empty(4, np.float64)
    _load().orc_swiglu_point(float(g), float(u), float(dh), _ptr(out))
    return tuple(float(v) for v in out)


def _three(shape):
    return tuple(np.empty(shape, np.uint16) for _ in range(3))


def swiglu_fwd(gu_bits: np.ndarray, tol: float):
    """gu: uint16 [rows, 2f] (gate | up) -> (y, lo, hi) uint16 [rows, f]."""
    gu = _c(gu_bits, np.uint16)
    rows, f2 = gu.shape
    f = f2 // 2
    y, lo, hi = _three((rows, f))
    _check(_load().orc_swiglu_fwd(_ptr(gu), rows, f, float(tol), _ptr(y), _ptr(lo), _ptr(hi)),
           "swiglu_fwd")
    return y, lo, hi


def swiglu_bwd(dh_bits: np.ndarray, gu_bits: np.ndarray, tol: float):
    """dh: uint16 [rows, f], gu: uint16 [rows, 2f] -> (y, lo, hi) uint16
    [rows, 2f] holding (d gate | d up)."""
    dh = _c(dh_bits, np.uint16)
    gu = _c(gu_bits, np.uint16)
    rows, f = dh.shape
    if gu.shape != (rows, 2 * f):
        raise ValueError("gu must be [rows, 2f]")
    y, lo, hi = _three((rows, 2 * f))
    _check(_load().orc_swiglu_bwd(_ptr(dh), _ptr(gu), rows, f, float(tol), _ptr(y), _ptr(lo),
                                  _ptr(hi)), "swiglu_bwd")
    return y, lo, hi


def rmsnorm_fwd(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float, tol: float):
    """x: uint16 [rows, cols], gamma: uint16 [cols] -> (y, lo, hi, rstd) with
    rstd float64 [rows]."""
    x = _c(x_bits, np.uint16)
    gamma = _c(gamma_bits, np.uint16)
    rows, cols = x.shape
    if gamma.shape != (cols,):
        raise ValueError("gamma must be [cols]")
    y, lo, hi = _three((rows, cols))
    rstd = np.empty(rows, np.float64)
    _check(_load().orc_rmsnorm_fwd(_ptr(x), _ptr(gamma), rows, cols, float(eps), float(tol),
                                   _ptr(y), _ptr(lo), _ptr(hi), _ptr(rstd)), "rmsnorm_fwd")
    return y, lo, hi, rstd


def rmsnorm_bwd(dy_bits: np.ndarray, x_bits: np.ndarray, gamma_bits: np.ndarray,
                rstd: np.ndarray, gin_bits, tol: float):
    """RMSNorm backward + residual add: dy, x, gin (or None) uint16 [rows,
    cols], gamma uint16 [cols], rstd float32 [rows] (the forward's) ->
    (y, lo, hi) uint16 [rows, cols]."""
    dy = _c(dy_bits, np.uint16)
    x = _c(x_bits, np.uint16)
    gamma = _c(gamma_bits, np.uint16)
    rs = _c(rstd, np.float32)
    rows, cols = x.shape
    if dy.shape != (rows, cols) or gamma.shape != (cols,) or rs.shape != (rows,):
        raise ValueError("rmsnorm_bwd: shapes")
    gin = None if gin_bits is None else _c(gin_bits, np.uint16)
    if gin is not None and gin.shape != (rows, cols):
        raise ValueError("rmsnorm_bwd: gin shape")
    y, lo, hi = _three((rows, cols))
    _check(_load().orc_rmsnorm_bwd(_ptr(dy), _ptr(x), _ptr(gamma), _ptr(rs),
                                   None if gin is None else _ptr(gin), rows, cols, float(tol),
                                   _ptr(y), _ptr(lo), _ptr(hi)), "rmsnorm_bwd")
    return y, lo, hi


def residual_add(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """h = a + b of two bf16 arrays (uint16 bits), rounded once to bf16."""
    a = _c(a_bits, np.uint16)
    b = _c(b_bits, np.uint16)
    if a.shape != b.shape:
        raise ValueError("residual_add: shapes")
    h = np.empty(a.shape, np.uint16)
    _check(_load().orc_residual_add(_ptr(a), _ptr(b), a.size, _ptr(h)), "residual_add")
    return h


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# ---- metrics ---------------------------------------------------------------

def rel_fro(c: np.ndarray, ref: np.ndarray) -> float:
    """||C - R||_F / ||R||_F in float64."""
    c = np.asarray(c, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((c - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def max_rel(c: np.ndarray, ref: np.ndarray, floor: float = 1e-2) -> float:
    """max |C - R| / max(|R|, floor)."""
    c = np.asarray(c, np.float64)
    ref = np.asarray(ref, np.float64)
    if c.size == 0:
        return 0.0
    return float(np.max(np.abs(c - ref) / np.maximum(np.abs(ref), floor)))
