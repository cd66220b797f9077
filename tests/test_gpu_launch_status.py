"""An entry point's status is its own launch's: a failed HIP runtime call of
the caller's, left unread on the thread, is not reported as this library's
launch failure.  The earlier failure is planted from the host (an invalid
device ordinal to hipSetDevice, which touches no GPU), the entry point is
called on preallocated buffers right after it, and its output is compared
with the same call made without the planted error."""
from __future__ import annotations

import ctypes

import pytest

pytestmark = pytest.mark.gpu


def _hip_runtime():
    # the HIP runtime already loaded in this process (torch and the library
    # share it; dlopen of the soname returns that instance)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipGetLastError.argtypes = []
    hip.hipGetLastError.restype = ctypes.c_int
    return hip


def test_status_ignores_an_earlier_unread_runtime_error():
    import torch

    import fp8_block_scaled_tile_amd as pf

    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    rows, cols = 300, 256
    x = torch.randn(rows, cols, device=dev, generator=g).to(torch.bfloat16)
    q = torch.empty(rows, cols, dtype=torch.uint8, device=dev)
    s = torch.empty(cols // 128, rows, dtype=torch.float32, device=dev)
    ref = pf.quant_act(x, row=True)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    hip = _hip_runtime()
    print("planting an invalid-ordinal hipSetDevice error", flush=True)
    try:
        assert hip.hipSetDevice(1 << 20) != 0
        rc = pf.puro_fp8_quant_act(x.data_ptr(), rows, cols, q.data_ptr(), s.data_ptr(), None,
                                   None, stream)
    finally:
        hip.hipGetLastError()          # consume whatever is left, for later launch checks
    assert rc == 0, pf.puro_fp8_status_string(rc)
    torch.cuda.synchronize()
    assert torch.equal(q, ref["q"])
    assert torch.equal(s, ref["s"])
