"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/puro_fp8.h declares, and rejects bad arguments synchronously with the
documented status codes (these calls return before any HIP call, so no
kernel is launched and no GPU is needed)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "puro_fp8.h")

OK, NULLP, SHAPE, ALIGN, ENUM, WS, VALUE = 0, 1, 2, 3, 4, 5, 9

# fake device addresses: never dereferenced, since validation fails first
P16 = 0x7F0000000000          # 16-byte aligned
P_ODD = 0x7F0000000008        # 8-byte aligned only


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(puro_(?:fp8|bf16)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import fp8_block_scaled_tile_amd as pf
    if not os.path.exists(pf.library_path()):
        from fp8_block_scaled_tile_amd import build
        build.build()
    return pf


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("puro_fp8_quant_act", "puro_fp8_quant_weight", "puro_fp8_gemm_blockscaled",
              "puro_fp8_gemm_workspace_bytes", "puro_fp8_status_string",
              "puro_fp8_abi_version", "puro_fp8_probe_encode", "puro_fp8_swiglu_quant",
              "puro_fp8_swiglu_bwd_quant", "puro_fp8_rmsnorm_quant", "puro_bf16_gemm_nt",
              "puro_fp8_probe_sigmoid", "puro_fp8_probe_mfma",
              "puro_fp8_gemm_blockscaled_noalloc", "puro_fp8_rmsnorm_quant_rstd",
              "puro_fp8_rmsnorm_bwd_quant", "puro_bf16_residual_add_rstd",
              "puro_fp8_quant_weight_grouped"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    handle = ctypes.CDLL(lib.library_path())
    for name in _declared_functions():
        assert hasattr(handle, name), f"{name} not exported"


def test_abi_version_and_status_strings(lib):
    assert lib.puro_fp8_abi_version() == 1
    for code in range(10):
        s = lib.puro_fp8_status_string(code)
        assert s.startswith("PURO_")
    assert "unknown" in lib.puro_fp8_status_string(77)


def test_quant_act_validation(lib):
    f = lib.puro_fp8_quant_act
    assert f(P16, 16, 100, P16, P16, None, None, None) == SHAPE       # cols % 128
    assert f(P16, -1, 128, P16, P16, None, None, None) == SHAPE
    assert f(P16, 16, 0, P16, P16, None, None, None) == SHAPE
    assert f(None, 16, 128, P16, P16, None, None, None) == NULLP
    assert f(P16, 16, 128, None, None, None, None, None) == NULLP     # no output
    assert f(P16, 16, 128, P16, None, None, None, None) == NULLP      # half a pair
    assert f(P16, 16, 128, None, None, P16, None, None) == NULLP
    assert f(P_ODD, 16, 128, P16, P16, None, None, None) == ALIGN
    assert f(P16, 16, 128, P16, P_ODD, None, None, None) == ALIGN
    assert f(P16, 16, 128, None, None, P16, P_ODD, None) == ALIGN
    assert f(P16, 0, 128, P16, P16, P16, P16, None) == OK             # empty: no-op


def test_quant_weight_validation(lib):
    f = lib.puro_fp8_quant_weight
    assert f(P16, 100, 128, P16, None, P16, None) == SHAPE
    assert f(P16, 128, 0, P16, None, P16, None) == SHAPE
    assert f(None, 128, 128, P16, None, P16, None) == NULLP
    assert f(P16, 128, 128, None, None, P16, None) == NULLP      # neither q nor qt
    assert f(P16, 128, 128, P16, None, None, None) == NULLP
    assert f(P16, 128, 128, P16, P_ODD, P16, None) == ALIGN
    assert f(P16, 128, 128, P_ODD, P16, P16, None) == ALIGN


def test_gemm_validation(lib):
    f = lib.puro_fp8_gemm_blockscaled
    args = lambda **kw: dict(dict(mode=0, M=256, N=256, K=256, a=P16, sa=P16, b=P16, sb=P16,
                                  c=P16, c_dtype=0, acc=0, ws=None, wsb=0), **kw)

    def call(**kw):
        d = args(**kw)
        return f(d["mode"], d["M"], d["N"], d["K"], d["a"], d["sa"], d["b"], d["sb"], d["c"],
                 d["c_dtype"], d["acc"], d["ws"], d["wsb"], None)

    assert call(mode=5) == ENUM
    assert call(mode=4, N=(1 << 29) + 128) == SHAPE          # FWD_T: N <= 2^29
    assert call(mode=-1) == ENUM
    assert call(mode=3, N=(1 << 29) + 128) == SHAPE          # DGRAD_W: N <= 2^29
    assert call(mode=3, a=None) == NULLP
    assert call(c_dtype=2) == ENUM
    assert call(acc=1, c_dtype=0) == ENUM                  # accumulate needs FP32
    assert call(N=200) == SHAPE
    assert call(K=100) == SHAPE
    assert call(M=-5) == SHAPE
    assert call(K=0) == SHAPE
    assert call(K=(1 << 24) + 128) == SHAPE                 # contraction limit
    assert call(a=None) == NULLP
    assert call(sb=None) == NULLP
    assert call(c=None) == NULLP
    assert call(b=P_ODD) == ALIGN
    assert call(M=0) == OK                                  # empty: no-op
    # a problem that splits K needs a workspace
    need = lib.puro_fp8_gemm_workspace_bytes(2, 2048, 2048, 32768)
    assert need > 0
    assert call(mode=2, M=2048, N=2048, K=32768, c_dtype=1) == WS
    assert call(mode=2, M=2048, N=2048, K=32768, c_dtype=1, ws=P16, wsb=need - 16) == WS
    assert call(mode=2, M=2048, N=2048, K=32768, c_dtype=1, ws=P_ODD, wsb=need) == ALIGN


def test_workspace_query(lib):
    q = lib.puro_fp8_gemm_workspace_bytes
    assert q(0, 16384, 6144, 2048) == 0                    # enough tiles: no split
    assert q(2, 2048, 2048, 32768) % (2048 * 2048 * 4) == 0
    assert q(0, 256, 100, 256) == 0                        # invalid shape -> 0
    assert q(5, 256, 256, 256) == 0
    assert q(3, 256, 256, 4096) == q(1, 256, 256, 4096) > 0     # DGRAD_W splits as DGRAD


def test_noalloc_gemm_validation(lib):
    """The allocation-free GEMM refuses bad arguments, and problems whose
    split-K partials exceed its static array, before touching a device."""
    f = lib.puro_fp8_gemm_blockscaled_noalloc
    assert f(5, 256, 256, 256, P16, P16, P16, P16, P16, 0, 0, None) == ENUM
    assert f(0, 256, 256, 256, P16, P16, P16, P16, P16, 0, 1, None) == ENUM      # += needs FP32
    assert f(0, 256, 200, 256, P16, P16, P16, P16, P16, 0, 0, None) == SHAPE
    assert f(0, 0, 256, 256, None, None, None, None, None, 0, 0, None) == OK
    assert f(0, 256, 256, 256, None, P16, P16, P16, P16, 0, 0, None) == NULLP
    assert f(0, 256, 256, 256, P16 + 8, P16, P16, P16, P16, 0, 0, None) == ALIGN
    big = lib.puro_fp8_gemm_workspace_bytes(2, 2560, 2560, 8192)
    assert big > lib.PURO_FP8_NOALLOC_SCRATCH_BYTES
    assert f(2, 2560, 2560, 8192, P16, P16, P16, P16, P16, 1, 0, None) == WS
    header = open(HEADER).read()
    assert "#define PURO_FP8_NOALLOC_SCRATCH_BYTES (64u << 20)" in header
    assert lib.PURO_FP8_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_probe_validation(lib):
    assert lib.puro_fp8_probe_encode(0, -1, P16, None) == SHAPE
    assert lib.puro_fp8_probe_encode(0, 10, None, None) == NULLP
    assert lib.puro_fp8_probe_encode(0, 0, None, None) == OK
    assert lib.puro_fp8_probe_sigmoid(0, -1, 0, P16, None) == SHAPE
    assert lib.puro_fp8_probe_sigmoid(0, 10, 0, None, None) == NULLP
    assert lib.puro_fp8_probe_sigmoid(0, 10, 1, P16 + 2, None) == ALIGN
    assert lib.puro_fp8_probe_sigmoid(0, 10, 3, P16, None) == ENUM
    assert lib.puro_fp8_probe_sigmoid(0, 10, -1, P16, None) == ENUM
    assert lib.puro_fp8_probe_sigmoid(0, 0, 2, None, None) == OK
    assert lib.puro_fp8_probe_mfma(6, P16, P16, 0, 0, P16, None) == ENUM
    assert lib.puro_fp8_probe_mfma(-1, P16, P16, 0, 0, P16, None) == ENUM
    assert lib.puro_fp8_probe_mfma(0, None, P16, 0, 0, P16, None) == NULLP
    assert lib.puro_fp8_probe_mfma(0, P16, P16, 0, 0, P16 + 4, None) == ALIGN
    assert lib.puro_fp8_probe_mfma(5, P16, P16, 256, 0, P16, None) == VALUE
    assert lib.puro_fp8_probe_mfma(5, P16, P16, 0, -1, P16, None) == VALUE


def test_plain_host_consumer_compiles_and_links(tmp_path):
    """The C header is usable from a plain C++ host program: the ABI consumer
    compiles against include/puro_fp8.h and links against the library (it is
    run by the GPU tests)."""
    import subprocess
    from fp8_block_scaled_tile_amd import build as hip_build
    import oracle
    oracle.build(force=False)
    src = os.path.join(ROOT, "tests", "c_abi", "abi_consumer.cpp")
    out = str(tmp_path / "abi_consumer")
    subprocess.run([hip_build.hipcc(), "--offload-arch=gfx950", "-O0", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"), src,
                    "-o", out, "-L", os.path.join(ROOT, "fp8_block_scaled_tile_amd"), "-lpuro_fp8",
                    "-L", os.path.join(ROOT, "oracle"), "-lpuro_oracle"],
                   check=True, capture_output=True, text=True)
    assert os.path.exists(out)


def test_bf16_comparator_validation(lib):
    f = lib.puro_bf16_gemm_nt
    q = lib.puro_bf16_gemm_nt_workspace_bytes
    assert f(256, 256, 100, P16, P16, P16, None, 0, None) == SHAPE     # K % 64
    assert f(256, 200, 128, P16, P16, P16, None, 0, None) == SHAPE     # N % 128
    assert f(-1, 256, 128, P16, P16, P16, None, 0, None) == SHAPE
    assert f(256, 256, (1 << 23) + 64, P16, P16, P16, None, 0, None) == SHAPE   # 2K > 2^24 bytes
    assert f(256, 256, 128, None, P16, P16, None, 0, None) == NULLP
    assert f(256, 256, 128, P16, P16, None, None, 0, None) == NULLP
    assert f(256, 256, 128, P16, P_ODD, P16, None, 0, None) == ALIGN
    assert f(0, 256, 128, P16, P16, P16, None, 0, None) == OK          # empty: no-op
    need = q(256, 256, 8192)                                            # one tile, long K: split
    assert need > 0 and need % (256 * 256 * 4) == 0
    assert f(256, 256, 8192, P16, P16, P16, None, 0, None) == WS
    assert f(256, 256, 8192, P16, P16, P16, P16, need - 16, None) == WS
    assert q(32768, 6144, 2048) == 0 and q(256, 100, 128) == 0


def test_swiglu_quant_validation(lib):
    f = lib.puro_fp8_swiglu_quant
    assert f(P16, 16, 100, P16, P16, None, None, None, None) == SHAPE     # f % 128
    assert f(P16, 16, 0, P16, P16, None, None, None, None) == SHAPE
    assert f(P16, -1, 128, P16, P16, None, None, None, None) == SHAPE
    assert f(None, 16, 128, P16, P16, None, None, None, None) == NULLP
    assert f(P16, 16, 128, None, None, None, None, None, None) == NULLP   # no output at all
    assert f(P16, 16, 128, P16, None, None, None, None, None) == NULLP    # half a pair
    assert f(P16, 16, 128, None, None, None, P16, None, None) == NULLP
    assert f(P_ODD, 16, 128, P16, P16, None, None, None, None) == ALIGN
    assert f(P16, 16, 128, None, None, None, None, P_ODD, None) == ALIGN  # bf16 output
    assert f(P16, 0, 128, P16, P16, P16, P16, P16, None) == OK            # empty: no-op


def test_swiglu_bwd_quant_validation(lib):
    f = lib.puro_fp8_swiglu_bwd_quant
    assert f(P16, P16, 16, 64, P16, P16, None, None, None, None) == SHAPE
    assert f(P16, P16, 16, -128, P16, P16, None, None, None, None) == SHAPE
    assert f(None, P16, 16, 128, P16, P16, None, None, None, None) == NULLP
    assert f(P16, None, 16, 128, P16, P16, None, None, None, None) == NULLP
    assert f(P16, P16, 16, 128, None, None, None, None, None, None) == NULLP
    assert f(P16, P_ODD, 16, 128, P16, P16, None, None, None, None) == ALIGN
    assert f(P16, P16, 16, 128, None, None, P16, P_ODD, None, None) == ALIGN
    assert f(P16, P16, 0, 128, P16, P16, None, None, None, None) == OK


def test_quant_weight_grouped_validation(lib):
    f = lib.puro_fp8_quant_weight_grouped
    D = lib.WeightDesc
    good = lambda: D(P16, 256, 384, P16, None, P16)
    arr = lambda *ds: (D * len(ds))(*ds)
    assert f(None, 0, None) == OK                                          # nothing to do
    assert f(None, 1, None) == NULLP
    assert f(arr(good()), -1, None) == SHAPE
    assert f(arr(*[good() for _ in range(17)]), 17, None) == SHAPE         # more than 16
    assert f(arr(good(), D(P16, 200, 384, P16, None, P16)), 2, None) == SHAPE
    assert f(arr(good(), D(P16, 256, 384, None, None, P16)), 2, None) == NULLP   # no codes at all
    assert f(arr(good(), D(P16, 256, 384, P16, P16, None)), 2, None) == NULLP    # no scales
    assert f(arr(D(P_ODD, 256, 384, P16, None, P16)), 1, None) == ALIGN
    assert f(arr(good(), D(P16, 256, 384, P16, P_ODD, P16)), 2, None) == ALIGN


def test_rmsnorm_quant_validation(lib):
    f = lib.puro_fp8_rmsnorm_quant
    ok = (P16, P16, 16, 256, 1e-6, P16, P16, P16, P16, P16, None, None)
    call = lambda i, v: f(*(ok[:i] + (v,) + ok[i + 1:]))
    assert call(3, 200) == SHAPE                                           # cols % 128
    assert call(2, -3) == SHAPE
    assert call(0, None) == NULLP
    assert call(1, None) == NULLP                                          # gamma
    assert call(5, None) == NULLP                                          # rstd is required
    assert f(P16, P16, 16, 256, 1e-6, P16, None, None, None, None, None, None) == NULLP
    assert call(1, P_ODD) == ALIGN
    assert call(5, P_ODD) == ALIGN
    assert call(4, -1e-6) == VALUE                                         # eps < 0
    assert call(4, float("nan")) == VALUE
    assert call(4, float("inf")) == VALUE
    assert f(P16, P16, 0, 256, 1e-6, P16, P16, P16, None, None, None, None) == OK


def test_rmsnorm_quant_rstd_validation(lib):
    f = lib.puro_fp8_rmsnorm_quant_rstd
    ok = (P16, P16, P16, 16, 256, P16, P16, None, None, None, None)
    call = lambda i, v: f(*(ok[:i] + (v,) + ok[i + 1:]))
    assert call(4, 200) == SHAPE
    assert call(3, -1) == SHAPE
    assert call(2, None) == NULLP                                          # rstd is an input
    assert call(0, None) == NULLP
    assert call(2, P_ODD) == ALIGN
    assert call(5, None) == NULLP                                          # no output at all
    assert call(3, 0) == OK


def test_rmsnorm_bwd_quant_validation(lib):
    f = lib.puro_fp8_rmsnorm_bwd_quant
    # dy, x, gamma, rstd, gin, rows, cols, coef, q, s, qt, st, y, stream
    ok = (P16, P16, P16, P16, None, 16, 256, P16, P16, P16, None, None, None, None)
    call = lambda i, v: f(*(ok[:i] + (v,) + ok[i + 1:]))
    assert call(6, 100) == SHAPE
    assert call(5, -2) == SHAPE
    for i in (0, 1, 2, 3, 7):                                              # gin alone may be NULL
        assert call(i, None) == NULLP, i
    for i in (0, 1, 2, 3, 4, 7):
        assert call(i, P_ODD) == ALIGN, i
    assert call(8, None) == NULLP                                          # q without s / no output
    assert call(5, 0) == OK


def test_residual_add_rstd_validation(lib):
    f = lib.puro_bf16_residual_add_rstd
    ok = (P16, P16, 16, 256, 1e-6, P16, P16, None)
    call = lambda i, v: f(*(ok[:i] + (v,) + ok[i + 1:]))
    assert call(3, 200) == SHAPE
    assert call(3, 0) == SHAPE
    assert call(2, -1) == SHAPE
    for i in (0, 1, 5, 6):
        assert call(i, None) == NULLP, i
        assert call(i, P_ODD) == ALIGN, i
    assert call(4, -1.0) == VALUE
    assert call(4, float("nan")) == VALUE
    assert call(2, 0) == OK
