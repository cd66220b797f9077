"""The torch-facing wrappers reject what the C ABI cannot check: host
(CPU) tensors, tensors on different devices, non-contiguous workspaces and
unknown modes raise in Python before any pointer reaches the library (a host
pointer handed to a kernel would fault the GPU instead of failing cleanly).
Runs without a GPU."""
from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")

import fp8_block_scaled_tile_amd as pf  # noqa: E402

BF16 = torch.bfloat16


def _cpu(*shape, dtype=BF16):
    return torch.zeros(*shape, dtype=dtype)


@pytest.mark.parametrize("call", [
    lambda: pf.quant_act(_cpu(128, 256), row=True, col=True),
    lambda: pf.quant_weight(_cpu(256, 256)),
    lambda: pf.swiglu_quant(_cpu(128, 512)),
    lambda: pf.swiglu_bwd_quant(_cpu(128, 256), _cpu(128, 512)),
    lambda: pf.rmsnorm_quant(_cpu(128, 256), _cpu(256)),
    lambda: pf.gemm_blockscaled(pf.GEMM_FWD, _cpu(256, 256, dtype=torch.uint8),
                                _cpu(2, 256, dtype=torch.float32),
                                _cpu(256, 256, dtype=torch.uint8),
                                _cpu(2, 2, dtype=torch.float32)),
    lambda: pf.gemm_bf16_nt(_cpu(256, 128), _cpu(256, 128)),
], ids=["quant_act", "quant_weight", "swiglu", "swiglu_bwd", "rmsnorm", "gemm", "gemm_bf16"])
def test_host_tensors_are_rejected(call):
    with pytest.raises(ValueError):
        call()


def test_unknown_gemm_mode_is_rejected():
    with pytest.raises(ValueError):
        pf.gemm_blockscaled(7, _cpu(256, 256, dtype=torch.uint8), _cpu(2, 256, dtype=torch.float32),
                            _cpu(256, 256, dtype=torch.uint8), _cpu(2, 2, dtype=torch.float32))


def test_wrong_dtype_is_a_type_error():
    with pytest.raises(TypeError):
        pf.quant_act(_cpu(128, 256, dtype=torch.float32))
