"""Fine-grained block-quantized FP8 linear layer for AMD MI355X (gfx950).

Python binding of ``libpuro_fp8.so`` (C ABI in ``include/puro_fp8.h``).  This
module only marshals arguments: every step of the quantizers and GEMM runs in
the library's hand-written HIP kernels.  PyTorch supplies device memory and
the current stream; codes travel as ``torch.uint8``.

Two layers:

* ``puro_fp8_*`` -- the C entry points under their own names, taking raw
  device pointers (ints) and returning the status code.
* ``quant_act`` / ``quant_weight`` / ``gemm_blockscaled`` -- allocate the
  outputs with torch, call the entry points on the current stream, and raise
  ``PuroError`` with the library's status string on failure.

Importing this package does not touch the GPU or load the library.  The
first call into the library loads it; if the shared library has not been
built, that call raises ImportError.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

from . import _lib

__all__ = [
    "PuroError", "GEMM_FWD", "GEMM_DGRAD", "GEMM_WGRAD", "GEMM_DGRAD_W", "GEMM_FWD_T", "OUT_BF16", "OUT_FP32",
    "puro_fp8_quant_act", "puro_fp8_quant_weight", "puro_fp8_gemm_blockscaled",
    "puro_fp8_gemm_workspace_bytes", "puro_fp8_status_string", "puro_fp8_abi_version",
    "puro_fp8_gemm_blockscaled_noalloc", "PURO_FP8_NOALLOC_SCRATCH_BYTES",
    "puro_fp8_probe_encode", "puro_fp8_probe_sigmoid", "puro_fp8_probe_mfma", "quant_act", "quant_weight",
    "gemm_blockscaled",
    "puro_bf16_gemm_nt", "puro_bf16_gemm_nt_workspace_bytes", "gemm_bf16_nt",
    "puro_fp8_swiglu_quant", "puro_fp8_swiglu_bwd_quant", "puro_fp8_rmsnorm_quant",
    "swiglu_quant", "swiglu_bwd_quant", "rmsnorm_quant", "library_path",
    "puro_fp8_rmsnorm_quant_rstd", "puro_fp8_rmsnorm_bwd_quant", "puro_bf16_residual_add_rstd",
    "rmsnorm_quant_rstd", "rmsnorm_bwd_quant", "residual_add_rstd",
    "puro_fp8_quant_weight_grouped", "quant_weight_grouped", "WeightDesc",
    "PURO_FP8_MAX_GROUPED_WEIGHTS",
]

GEMM_FWD, GEMM_DGRAD, GEMM_WGRAD, GEMM_DGRAD_W, GEMM_FWD_T = 0, 1, 2, 3, 4
OUT_BF16, OUT_FP32 = 0, 1
PURO_FP8_NOALLOC_SCRATCH_BYTES = 64 << 20
PURO_FP8_MAX_GROUPED_WEIGHTS = 16
WeightDesc = _lib.WeightDesc
PURO_OK = 0


class PuroError(RuntimeError):
    def __init__(self, status: int):
        self.status = int(status)
        super().__init__(puro_fp8_status_string(status))


def library_path() -> str:
    return _lib.path()


# ---- the C entry points ------------------------------------------------------

def puro_fp8_quant_act(x, rows, cols, q, s, qt, st, stream) -> int:
    return _lib.get().puro_fp8_quant_act(x, rows, cols, q, s, qt, st, stream)


def puro_fp8_quant_weight(w, n, k, q, qt, s, stream) -> int:
    return _lib.get().puro_fp8_quant_weight(w, n, k, q, qt, s, stream)


def puro_fp8_quant_weight_grouped(descs, count, stream) -> int:
    """descs: a ctypes array of WeightDesc (or a pointer to its first element)."""
    return _lib.get().puro_fp8_quant_weight_grouped(descs, count, stream)


def puro_fp8_gemm_blockscaled(mode, M, N, K, a, sa, b, sb, c, c_dtype, accumulate, workspace,
                              workspace_bytes, stream) -> int:
    return _lib.get().puro_fp8_gemm_blockscaled(mode, M, N, K, a, sa, b, sb, c, c_dtype,
                                                accumulate, workspace, workspace_bytes, stream)


def puro_fp8_gemm_blockscaled_noalloc(mode, M, N, K, a, sa, b, sb, c, c_dtype, accumulate,
                                      stream) -> int:
    return _lib.get().puro_fp8_gemm_blockscaled_noalloc(mode, M, N, K, a, sa, b, sb, c, c_dtype,
                                                        accumulate, stream)


def puro_fp8_gemm_workspace_bytes(mode, M, N, K) -> int:
    return int(_lib.get().puro_fp8_gemm_workspace_bytes(mode, M, N, K))


def puro_fp8_status_string(status) -> str:
    return _lib.get().puro_fp8_status_string(int(status)).decode()


def puro_fp8_abi_version() -> int:
    return int(_lib.get().puro_fp8_abi_version())


def puro_fp8_probe_encode(first_bits, n, out, stream) -> int:
    return _lib.get().puro_fp8_probe_encode(first_bits, n, out, stream)


def puro_fp8_probe_sigmoid(first_bits, n, form, out, stream) -> int:
    return _lib.get().puro_fp8_probe_sigmoid(first_bits, n, form, out, stream)


def puro_fp8_probe_mfma(form, a, b, scale_a, scale_b, d, stream) -> int:
    return _lib.get().puro_fp8_probe_mfma(form, a, b, scale_a, scale_b, d, stream)


def puro_bf16_gemm_nt(M, N, K, a, b, c, workspace, workspace_bytes, stream) -> int:
    return _lib.get().puro_bf16_gemm_nt(M, N, K, a, b, c, workspace, workspace_bytes, stream)


def puro_bf16_gemm_nt_workspace_bytes(M, N, K) -> int:
    return int(_lib.get().puro_bf16_gemm_nt_workspace_bytes(M, N, K))


def puro_fp8_swiglu_quant(gu, rows, f, q, s, qt, st, y, stream) -> int:
    return _lib.get().puro_fp8_swiglu_quant(gu, rows, f, q, s, qt, st, y, stream)


def puro_fp8_swiglu_bwd_quant(dh, gu, rows, f, q, s, qt, st, y, stream) -> int:
    return _lib.get().puro_fp8_swiglu_bwd_quant(dh, gu, rows, f, q, s, qt, st, y, stream)


def puro_fp8_rmsnorm_quant(x, gamma, rows, cols, eps, rstd, q, s, qt, st, y, stream) -> int:
    return _lib.get().puro_fp8_rmsnorm_quant(x, gamma, rows, cols, eps, rstd, q, s, qt, st, y,
                                             stream)


def puro_fp8_rmsnorm_quant_rstd(x, gamma, rstd, rows, cols, q, s, qt, st, y, stream) -> int:
    return _lib.get().puro_fp8_rmsnorm_quant_rstd(x, gamma, rstd, rows, cols, q, s, qt, st, y,
                                                  stream)


def puro_fp8_rmsnorm_bwd_quant(dy, x, gamma, rstd, gin, rows, cols, coef, q, s, qt, st, y,
                               stream) -> int:
    return _lib.get().puro_fp8_rmsnorm_bwd_quant(dy, x, gamma, rstd, gin, rows, cols, coef, q, s,
                                                 qt, st, y, stream)


def puro_bf16_residual_add_rstd(a, b, rows, cols, eps, h, rstd, stream) -> int:
    return _lib.get().puro_bf16_residual_add_rstd(a, b, rows, cols, eps, h, rstd, stream)


# ---- torch-facing wrappers --------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc):
    if rc != PURO_OK:
        raise PuroError(rc)


def _need(t, dtype, shape, name):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{name}: expected a contiguous CUDA tensor")
    return t


def _bf16_2d(t, name):
    """A 2-D bfloat16 CUDA tensor, made contiguous.  The device check keeps a
    host tensor's pointer from ever reaching a kernel."""
    torch = _torch()
    if t.dtype != torch.bfloat16 or t.dim() != 2:
        raise TypeError(f"{name}: expected a 2-D bfloat16 tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a CUDA tensor, got one on {t.device}")
    return t.contiguous()


def _same_device(first, *others):
    for t in others:
        if t.device != first.device:
            raise ValueError(f"tensors on different devices: {first.device} and {t.device}")


def quant_act(x, row: bool = True, col: bool = False, stream=None):
    """1x128 (row) and/or 128x1 (col, transposed) quantization of a bf16
    [rows, cols] CUDA tensor.  Returns a dict with ``q`` u8 [rows, cols] and
    ``s`` f32 [cols/128, rows] (row), ``qt`` u8 [cols, rows_pad] and ``st``
    f32 [rows_pad/128, cols] (col)."""
    torch = _torch()
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    rp = (rows + 127) // 128 * 128
    out = {}
    dev = x.device
    if row:
        out["q"] = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        out["s"] = torch.empty((cols // 128, rows), dtype=torch.float32, device=dev)
    if col:
        out["qt"] = torch.empty((cols, rp), dtype=torch.uint8, device=dev)
        out["st"] = torch.empty((rp // 128, cols), dtype=torch.float32, device=dev)
    _check(puro_fp8_quant_act(_ptr(x), rows, cols, _ptr(out.get("q")), _ptr(out.get("s")),
                              _ptr(out.get("qt")), _ptr(out.get("st")), _stream(stream)))
    return out


def _produce_outputs(rows, cols, dev, row, col, bf16_out):
    torch = _torch()
    rp = (rows + 127) // 128 * 128
    out = {}
    if row:
        out["q"] = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        out["s"] = torch.empty((cols // 128, rows), dtype=torch.float32, device=dev)
    if col:
        out["qt"] = torch.empty((cols, rp), dtype=torch.uint8, device=dev)
        out["st"] = torch.empty((rp // 128, cols), dtype=torch.float32, device=dev)
    if bf16_out:
        out["y"] = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    return out


def swiglu_quant(gu, row: bool = True, col: bool = True, bf16_out: bool = False, stream=None):
    """SwiGLU of gu = (gate | up) [rows, 2f] written as FP8 operands: ``q``/``s``
    (1x128), ``qt``/``st`` (128x1, transposed) and optionally ``y`` (bf16 h),
    layouts as in quant_act with cols = f."""
    gu = _bf16_2d(gu, "gu")
    rows, f2 = gu.shape
    out = _produce_outputs(rows, f2 // 2, gu.device, row, col, bf16_out)
    _check(puro_fp8_swiglu_quant(_ptr(gu), rows, f2 // 2, _ptr(out.get("q")), _ptr(out.get("s")),
                                 _ptr(out.get("qt")), _ptr(out.get("st")), _ptr(out.get("y")),
                                 _stream(stream)))
    return out


def swiglu_bwd_quant(dh, gu, row: bool = True, col: bool = True, bf16_out: bool = False,
                     stream=None):
    """SwiGLU backward: (d gate | d up) [rows, 2f] from dh [rows, f] and gu,
    written as FP8 operands (and optionally bf16 ``y``)."""
    dh = _bf16_2d(dh, "dh")
    gu = _bf16_2d(gu, "gu")
    _same_device(dh, gu)
    rows, f = dh.shape
    if tuple(gu.shape) != (rows, 2 * f):
        raise ValueError("gu must be [rows, 2f] for dh [rows, f]")
    out = _produce_outputs(rows, 2 * f, dh.device, row, col, bf16_out)
    _check(puro_fp8_swiglu_bwd_quant(_ptr(dh), _ptr(gu), rows, f, _ptr(out.get("q")),
                                     _ptr(out.get("s")), _ptr(out.get("qt")), _ptr(out.get("st")),
                                     _ptr(out.get("y")), _stream(stream)))
    return out


def rmsnorm_quant(x, gamma, eps: float = 1e-6, row: bool = True, col: bool = True,
                  bf16_out: bool = False, stream=None):
    """RMSNorm of x [rows, cols] with gain gamma [cols] written as FP8 operands
    (and optionally bf16 ``y``); ``rstd`` f32 [rows] is always returned."""
    torch = _torch()
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    if gamma.dtype != torch.bfloat16 or tuple(gamma.shape) != (cols,):
        raise TypeError("gamma: expected a bfloat16 tensor of shape [cols]")
    _same_device(x, gamma)
    gamma = gamma.contiguous()
    out = _produce_outputs(rows, cols, x.device, row, col, bf16_out)
    out["rstd"] = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(puro_fp8_rmsnorm_quant(_ptr(x), _ptr(gamma), rows, cols, float(eps), _ptr(out["rstd"]),
                                  _ptr(out.get("q")), _ptr(out.get("s")), _ptr(out.get("qt")),
                                  _ptr(out.get("st")), _ptr(out.get("y")), _stream(stream)))
    return out


def _gamma(gamma, cols, *others):
    torch = _torch()
    if gamma.dtype != torch.bfloat16 or tuple(gamma.shape) != (cols,):
        raise TypeError("gamma: expected a bfloat16 tensor of shape [cols]")
    _same_device(gamma, *others)
    return gamma.contiguous()


def _rstd(rstd, rows, dev):
    torch = _torch()
    if rstd.dtype != torch.float32 or tuple(rstd.shape) != (rows,):
        raise TypeError("rstd: expected a float32 tensor of shape [rows]")
    if rstd.device != dev:
        raise ValueError("rstd: on a different device")
    return rstd.contiguous()


def rmsnorm_quant_rstd(x, gamma, rstd, row: bool = True, col: bool = True,
                       bf16_out: bool = False, stream=None):
    """As rmsnorm_quant with the row statistic rstd f32 [rows] given (as
    residual_add_rstd returns it): one pass over x."""
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    gamma = _gamma(gamma, cols, x)
    rstd = _rstd(rstd, rows, x.device)
    out = _produce_outputs(rows, cols, x.device, row, col, bf16_out)
    _check(puro_fp8_rmsnorm_quant_rstd(_ptr(x), _ptr(gamma), _ptr(rstd), rows, cols,
                                       _ptr(out.get("q")), _ptr(out.get("s")), _ptr(out.get("qt")),
                                       _ptr(out.get("st")), _ptr(out.get("y")), _stream(stream)))
    return out


def rmsnorm_bwd_quant(dy, x, gamma, rstd, gin=None, row: bool = True, col: bool = True,
                      bf16_out: bool = False, stream=None):
    """RMSNorm backward plus the skip-path gradient gin (None = 0) as FP8
    operands: gin + rstd*gamma*dy - x*rstd^3*mean(gamma*dy*x).  Also returns
    ``coef`` f32 [rows] (the per-row second term's factor)."""
    torch = _torch()
    dy = _bf16_2d(dy, "dy")
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    if tuple(dy.shape) != (rows, cols):
        raise TypeError("dy: expected the shape of x")
    gamma = _gamma(gamma, cols, x, dy)
    rstd = _rstd(rstd, rows, x.device)
    if gin is not None:
        gin = _bf16_2d(gin, "gin")
        if tuple(gin.shape) != (rows, cols):
            raise TypeError("gin: expected the shape of x")
        _same_device(x, gin)
    out = _produce_outputs(rows, cols, x.device, row, col, bf16_out)
    out["coef"] = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(puro_fp8_rmsnorm_bwd_quant(_ptr(dy), _ptr(x), _ptr(gamma), _ptr(rstd), _ptr(gin), rows,
                                      cols, _ptr(out["coef"]), _ptr(out.get("q")),
                                      _ptr(out.get("s")), _ptr(out.get("qt")), _ptr(out.get("st")),
                                      _ptr(out.get("y")), _stream(stream)))
    return out


def residual_add_rstd(a, b, eps: float = 1e-6, stream=None):
    """h = a + b (bf16) and the RMSNorm statistic of h, rstd f32 [rows]."""
    torch = _torch()
    a = _bf16_2d(a, "a")
    b = _bf16_2d(b, "b")
    if a.shape != b.shape:
        raise TypeError("residual_add_rstd: a and b differ in shape")
    _same_device(a, b)
    rows, cols = a.shape
    h = torch.empty_like(a)
    rstd = torch.empty(rows, dtype=torch.float32, device=a.device)
    _check(puro_bf16_residual_add_rstd(_ptr(a), _ptr(b), rows, cols, float(eps), _ptr(h), _ptr(rstd),
                                  _stream(stream)))
    return {"h": h, "rstd": rstd}


def quant_weight(w, transpose: bool = True, codes: bool = True, stream=None):
    """128x128 block quantization of a bf16 [n, k] CUDA tensor.  Returns a dict
    with ``s`` f32 [n/128, k/128], ``q`` u8 [n, k] (unless codes=False) and
    ``qt`` u8 [k, n] (if transpose)."""
    torch = _torch()
    w = _bf16_2d(w, "w")
    n, k = w.shape
    dev = w.device
    if not codes and not transpose:
        raise ValueError("quant_weight: nothing to write (codes=False, transpose=False)")
    out = {"s": torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev)}
    if codes:
        out["q"] = torch.empty((n, k), dtype=torch.uint8, device=dev)
    if transpose:
        out["qt"] = torch.empty((k, n), dtype=torch.uint8, device=dev)
    _check(puro_fp8_quant_weight(_ptr(w), n, k, _ptr(out.get("q")), _ptr(out.get("qt")),
                                 _ptr(out["s"]), _stream(stream)))
    return out


def quant_weight_grouped(ws, transpose: bool = True, codes: bool = True, stream=None):
    """Several bf16 [n, k] CUDA weights quantized 128x128 in one launch: a list
    of dicts as quant_weight returns them, bit for bit."""
    torch = _torch()
    ws = [_bf16_2d(w, f"w[{i}]") for i, w in enumerate(ws)]
    if len(ws) > PURO_FP8_MAX_GROUPED_WEIGHTS:
        raise ValueError(f"quant_weight_grouped: at most {PURO_FP8_MAX_GROUPED_WEIGHTS} weights")
    if not codes and not transpose:
        raise ValueError("quant_weight_grouped: nothing to write (codes=False, transpose=False)")
    if ws:
        _same_device(ws[0], *ws[1:])
    outs = []
    descs = (WeightDesc * max(1, len(ws)))()
    for i, w in enumerate(ws):
        n, k = w.shape
        o = {"s": torch.empty((n // 128, k // 128), dtype=torch.float32, device=w.device)}
        if codes:
            o["q"] = torch.empty((n, k), dtype=torch.uint8, device=w.device)
        if transpose:
            o["qt"] = torch.empty((k, n), dtype=torch.uint8, device=w.device)
        descs[i] = WeightDesc(_ptr(w), n, k, _ptr(o.get("q")), _ptr(o.get("qt")), _ptr(o["s"]))
        outs.append(o)
    _check(puro_fp8_quant_weight_grouped(descs, len(ws), _stream(stream)))
    return outs


def gemm_blockscaled(mode: int, a, sa, b, sb, out_dtype=None, out=None, accumulate=False,
                     workspace=None, stream=None):
    """Block-scaled FP8 GEMM: C[M, N] (+)= blocks of a[M, K] . b[N, K]^T with
    scales sa [K/128, M] and sb (see the C header for each mode's layout)."""
    torch = _torch()
    if mode not in (GEMM_FWD, GEMM_DGRAD, GEMM_WGRAD, GEMM_DGRAD_W, GEMM_FWD_T):
        raise ValueError(f"unknown GEMM mode {mode}")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = a.shape
    b_kn = mode in (GEMM_DGRAD_W, GEMM_FWD_T)       # b stored [K][N]
    N = b.shape[1] if b_kn else b.shape[0]
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    c_dtype = OUT_FP32 if out_dtype == torch.float32 else OUT_BF16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be bfloat16 or float32")
    _need(a, torch.uint8, (M, K), "a")
    _need(b, torch.uint8, (K, N) if b_kn else (N, K), "b")
    _need(sa, torch.float32, (K // 128, M), "sa")
    sb_shape = {GEMM_FWD: (N // 128, K // 128), GEMM_FWD_T: (N // 128, K // 128),
                GEMM_DGRAD: (K // 128, N // 128), GEMM_DGRAD_W: (K // 128, N // 128),
                GEMM_WGRAD: (K // 128, N)}[mode]
    _need(sb, torch.float32, sb_shape, "sb")
    _same_device(a, sa, b, sb)
    if out is None:
        out = (torch.zeros if accumulate else torch.empty)((M, N), dtype=out_dtype, device=a.device)
    else:
        _need(out, out_dtype, (M, N), "out")
        _same_device(a, out)
    need = puro_fp8_gemm_workspace_bytes(mode, M, N, K)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
        _same_device(a, workspace)
        if not workspace.is_contiguous():
            raise ValueError("workspace: expected a contiguous tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(puro_fp8_gemm_blockscaled(mode, M, N, K, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                                     _ptr(out), c_dtype, 1 if accumulate else 0, ws_ptr, ws_bytes,
                                     _stream(stream)))
    return out


def gemm_bf16_nt(a, b, out=None, workspace=None, stream=None):
    """The BF16 comparator: bf16 C [M, N] = a [M, K] . b [N, K]^T with FP32
    accumulation, on this library's own tiling (measurement only; not part of
    the FP8 path).  Both operands K-contiguous bf16 CUDA tensors."""
    torch = _torch()
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("gemm_bf16_nt expects a [M, K] and b [N, K]")
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.bfloat16, (M, K), "a")
    _need(b, torch.bfloat16, (N, K), "b")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    else:
        _need(out, torch.bfloat16, (M, N), "out")
    need = puro_bf16_gemm_nt_workspace_bytes(M, N, K)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
        _same_device(a, workspace)
        if not workspace.is_contiguous():
            raise ValueError("workspace: expected a contiguous tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(puro_bf16_gemm_nt(M, N, K, _ptr(a), _ptr(b), _ptr(out), ws_ptr, ws_bytes,
                             _stream(stream)))
    return out
