"""Loader of the in-tree libpuro_fp8.so with the C signatures of
include/puro_fp8.h.  Fails loudly when the library has not been built."""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_PATH = os.path.join(_HERE, "libpuro_fp8.so")
_lock = threading.Lock()
_handle = None

EXPORTS = (
    "puro_fp8_quant_act", "puro_fp8_quant_weight", "puro_fp8_gemm_blockscaled",
    "puro_fp8_gemm_workspace_bytes", "puro_fp8_status_string", "puro_fp8_abi_version",
    "puro_fp8_probe_encode", "puro_bf16_gemm_nt", "puro_bf16_gemm_nt_workspace_bytes",
    "puro_fp8_swiglu_quant", "puro_fp8_swiglu_bwd_quant", "puro_fp8_rmsnorm_quant",
    "puro_fp8_probe_sigmoid", "puro_fp8_probe_mfma", "puro_fp8_gemm_blockscaled_noalloc",
    "puro_fp8_rmsnorm_quant_rstd", "puro_fp8_rmsnorm_bwd_quant", "puro_bf16_residual_add_rstd",
    "puro_fp8_quant_weight_grouped",
)


class WeightDesc(ctypes.Structure):
    """puro_fp8_weight_desc: the arguments of one puro_fp8_quant_weight call."""
    _fields_ = [("w", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("qt", ctypes.c_void_p), ("s", ctypes.c_void_p)]


def path() -> str:
    return _PATH


def get():
    global _handle
    with _lock:
        if _handle is not None:
            return _handle
        if not os.path.exists(_PATH):
            raise ImportError(f"{_PATH} is missing: build it with "
                              "`python -m fp8_block_scaled_tile_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.puro_fp8_quant_act.restype = I
        lib.puro_fp8_quant_act.argtypes = [P, I64, I64, P, P, P, P, P]
        lib.puro_fp8_quant_weight.restype = I
        lib.puro_fp8_quant_weight.argtypes = [P, I64, I64, P, P, P, P]
        lib.puro_fp8_gemm_blockscaled.restype = I
        lib.puro_fp8_gemm_blockscaled.argtypes = [I, I64, I64, I64, P, P, P, P, P, I, I, P,
                                                  ctypes.c_size_t, P]
        lib.puro_fp8_gemm_blockscaled_noalloc.restype = I
        lib.puro_fp8_gemm_blockscaled_noalloc.argtypes = [I, I64, I64, I64, P, P, P, P, P, I, I, P]
        lib.puro_fp8_gemm_workspace_bytes.restype = ctypes.c_size_t
        lib.puro_fp8_gemm_workspace_bytes.argtypes = [I, I64, I64, I64]
        lib.puro_fp8_status_string.restype = ctypes.c_char_p
        lib.puro_fp8_status_string.argtypes = [I]
        lib.puro_fp8_abi_version.restype = I
        lib.puro_fp8_abi_version.argtypes = []
        lib.puro_fp8_probe_encode.restype = I
        lib.puro_fp8_probe_encode.argtypes = [ctypes.c_uint32, I64, P, P]
        lib.puro_fp8_probe_sigmoid.restype = I
        lib.puro_fp8_probe_sigmoid.argtypes = [ctypes.c_uint32, I64, I, P, P]
        lib.puro_fp8_probe_mfma.restype = I
        lib.puro_fp8_probe_mfma.argtypes = [I, P, P, I, I, P, P]
        lib.puro_bf16_gemm_nt.restype = I
        lib.puro_bf16_gemm_nt.argtypes = [I64, I64, I64, P, P, P, P, ctypes.c_size_t, P]
        lib.puro_bf16_gemm_nt_workspace_bytes.restype = ctypes.c_size_t
        lib.puro_bf16_gemm_nt_workspace_bytes.argtypes = [I64, I64, I64]
        lib.puro_fp8_swiglu_quant.restype = I
        lib.puro_fp8_swiglu_quant.argtypes = [P, I64, I64, P, P, P, P, P, P]
        lib.puro_fp8_swiglu_bwd_quant.restype = I
        lib.puro_fp8_swiglu_bwd_quant.argtypes = [P, P, I64, I64, P, P, P, P, P, P]
        lib.puro_fp8_rmsnorm_quant.restype = I
        lib.puro_fp8_rmsnorm_quant.argtypes = [P, P, I64, I64, ctypes.c_float, P, P, P, P, P, P,
                                               P]
        lib.puro_fp8_rmsnorm_quant_rstd.restype = I
        lib.puro_fp8_rmsnorm_quant_rstd.argtypes = [P, P, P, I64, I64, P, P, P, P, P, P]
        lib.puro_fp8_rmsnorm_bwd_quant.restype = I
        lib.puro_fp8_rmsnorm_bwd_quant.argtypes = [P, P, P, P, P, I64, I64, P, P, P, P, P, P, P]
        lib.puro_bf16_residual_add_rstd.restype = I
        lib.puro_bf16_residual_add_rstd.argtypes = [P, P, I64, I64, ctypes.c_float, P, P, P]
        lib.puro_fp8_quant_weight_grouped.restype = I
        lib.puro_fp8_quant_weight_grouped.argtypes = [ctypes.POINTER(WeightDesc), I, P]
        _handle = lib
        return lib
