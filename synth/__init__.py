"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the quantization method: it only draws
random bf16 tensors with the shapes and value distributions of the
transformer-shaped workloads (normal activations with outlier channels,
heavy-tailed Student-t(3) activations, N(0, 0.02) weights, N(0, 1e-3) output
gradients), and converts bf16 tensors to raw bit patterns for the oracle.

Every tensor is drawn from torch's CPU generator seeded by (seed, stream id),
so the bytes are the same on every machine and independent of thread count;
the same bytes go to the oracle (as numpy uint16 bit patterns) and, after a
plain copy, to the device.

Readings of the workload descriptions (all fixed here, in one place):
  * "N(0, s)" names the standard deviation s.
  * outlier channels are a seeded random choice of columns (a permutation of
    the column indices, first n taken), multiplied by the factor before the
    bf16 rounding; "1% of channels" means round(0.01 * C) channels.
  * Student-t(3) is the standard t with 3 degrees of freedom,
    z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) with z_i standard normal.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["normal", "student_t3", "with_outliers", "bits", "from_bits",
           "LinearSpec", "WORKLOADS", "workload", "linear_inputs", "swiglu_inputs",
           "rmsnorm_inputs", "rmsnorm_bwd_inputs", "residual_inputs"]


def _gen(seed: int, stream: str) -> torch.Generator:
    sid = zlib.crc32(stream.encode()) & 0xFFFFFFFF
    g = torch.Generator(device="cpu")
    g.manual_seed(((int(seed) & 0xFFFFFFFF) << 32) | sid)
    return g


def normal(shape, std: float, seed: int, stream: str) -> torch.Tensor:
    """float32 tensor ~ N(0, std) on the CPU."""
    g = _gen(seed, stream)
    return torch.randn(*shape, generator=g, dtype=torch.float32) * float(std)


def student_t3(shape, seed: int, stream: str) -> torch.Tensor:
    """float32 tensor of i.i.d. standard Student-t(3) draws on the CPU."""
    g = _gen(seed, stream)
    z0 = torch.randn(*shape, generator=g, dtype=torch.float32)
    chi = torch.zeros(*shape, dtype=torch.float32)
    for _ in range(3):
        z = torch.randn(*shape, generator=g, dtype=torch.float32)
        chi.addcmul_(z, z)
        del z
    chi.div_(3.0).sqrt_()
    return z0.div_(chi)


def with_outliers(x: torch.Tensor, count: int, factor: float, seed: int,
                  stream: str) -> torch.Tensor:
    """Multiply ``count`` seeded columns of a [rows, cols] float tensor by
    ``factor`` (in place) and return it."""
    if count <= 0:
        return x
    g = _gen(seed, stream + "/outlier-cols")
    cols = torch.randperm(x.shape[1], generator=g)[:count]
    x[:, cols] *= float(factor)
    return x


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


# ---- the transformer-shaped workloads --------------------------------------

@dataclass(frozen=True)
class LinearSpec:
    """One linear layer W[out, in] applied to T tokens."""
    name: str
    tokens: int
    d_in: int
    d_out: int
    x_kind: str = "normal"         # "normal" | "t3"
    x_outliers: int = 0            # number of outlier channels in X
    x_outlier_factor: float = 1.0
    x_std: float = 1.0
    w_std: float = 0.02
    dy_std: float = 1e-3
    fwd: bool = True
    dgrad: bool = True
    wgrad: bool = True
    fwd_out: str = "bf16"          # "bf16" | "fp32"


def _pct_channels(c: int) -> int:
    return int(np.floor(0.01 * c + 0.5))


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    linears: tuple = field(default_factory=tuple)


def _block_stack(tokens: int = 32768, hidden: int = 2048, ffn: int = 8192) -> tuple:
    def L(name, d_in, d_out):
        return LinearSpec(name, tokens, d_in, d_out, x_outliers=_pct_channels(d_in),
                          x_outlier_factor=20.0)
    return (L("qkv", hidden, 3 * hidden), L("out_proj", hidden, hidden),
            L("up_gate", hidden, 2 * ffn), L("down", ffn, hidden))


WORKLOADS = {
    "tiny_fwd": Workload(
        "tiny_fwd", "X[256x512] N(0,1) with 4 outlier channels x50, W[512x512] N(0,0.02); "
        "forward, FP32 output, seed 0",
        (LinearSpec("tiny", 256, 512, 512, x_outliers=4, x_outlier_factor=50.0,
                    dgrad=False, wgrad=False, fwd_out="fp32"),)),
    "qkv_fwd": Workload(
        "qkv_fwd", "attention QKV projection forward, X[16384x2048] N(0,1) with 1% of "
        "channels x20, W[6144x2048] N(0,0.02), bf16 output",
        (LinearSpec("qkv", 16384, 2048, 6144, x_outliers=_pct_channels(2048),
                    x_outlier_factor=20.0, dgrad=False, wgrad=False),)),
    "upgate_fwd": Workload(
        "upgate_fwd", "SwiGLU up+gate forward, X[16384x2048] Student-t(3), "
        "W[16384x2048] N(0,0.02), bf16 output",
        (LinearSpec("up_gate", 16384, 2048, 16384, x_kind="t3", dgrad=False,
                    wgrad=False),)),
    "down_bwd": Workload(
        "down_bwd", "MLP down-projection backward, dY[16384x2048] N(0,1e-3), "
        "W[2048x8192] N(0,0.02), X[16384x8192] N(0,1); dgrad bf16, wgrad FP32",
        (LinearSpec("down", 16384, 8192, 2048, fwd=False),)),
    "block_stack": Workload(
        "block_stack", "linear stack of one 2048-hidden, 16-head, 8192-FFN block on "
        "8x4096 tokens: fwd+dgrad+wgrad of QKV, out-proj, up/gate, down",
        _block_stack()),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def linear_inputs(spec: LinearSpec, seed: int = 0, need=("x", "w", "dy")) -> dict:
    """bf16 CPU tensors X [T, in], W [out, in], dY [T, out] for one linear."""
    out = {}
    base = f"{spec.name}/{spec.tokens}x{spec.d_in}x{spec.d_out}"
    if "x" in need:
        if spec.x_kind == "t3":
            x = student_t3((spec.tokens, spec.d_in), seed, base + "/x")
        else:
            x = normal((spec.tokens, spec.d_in), spec.x_std, seed, base + "/x")
        with_outliers(x, spec.x_outliers, spec.x_outlier_factor, seed, base + "/x")
        out["x"] = x.to(torch.bfloat16)
        del x
    if "w" in need:
        out["w"] = normal((spec.d_out, spec.d_in), spec.w_std, seed, base + "/w").to(torch.bfloat16)
    if "dy" in need:
        out["dy"] = normal((spec.tokens, spec.d_out), spec.dy_std, seed, base + "/dy").to(torch.bfloat16)
    return out


# ---- inputs of the BF16 neighbour ops (quantize-on-produce) ------------------
# Readings: the up+gate projection's bf16 output (gate | up) is drawn as
# N(0, 1) with 1% of its columns x4 (|gate| stays below ~20); the gradient of
# the SwiGLU output as N(0, 1e-3) like the other output gradients; the
# residual stream entering RMSNorm as N(0, 1) with 1% of channels x20 like the
# linear inputs; the learned RMSNorm gain as 1 + N(0, 0.1); the gradients
# reaching the norm's backward (from the next projection's DGRAD, and along
# the skip path) as N(0, 1e-3) like the other output gradients; the
# projection output added to the residual stream as N(0, 1).

def swiglu_inputs(rows: int, f: int, seed: int = 0, need=("gu", "dh")) -> dict:
    """bf16 CPU tensors gu [rows, 2f] (gate | up) and dh [rows, f]."""
    out = {}
    base = f"swiglu/{rows}x{f}"
    if "gu" in need:
        gu = normal((rows, 2 * f), 1.0, seed, base + "/gu")
        with_outliers(gu, _pct_channels(2 * f), 4.0, seed, base + "/gu")
        out["gu"] = gu.to(torch.bfloat16)
        del gu
    if "dh" in need:
        out["dh"] = normal((rows, f), 1e-3, seed, base + "/dh").to(torch.bfloat16)
    return out


def rmsnorm_inputs(rows: int, cols: int, seed: int = 0) -> dict:
    """bf16 CPU tensors x [rows, cols] and gamma [cols]."""
    base = f"rmsnorm/{rows}x{cols}"
    x = normal((rows, cols), 1.0, seed, base + "/x")
    with_outliers(x, _pct_channels(cols), 20.0, seed, base + "/x")
    gamma = 1.0 + normal((cols,), 0.1, seed, base + "/gamma")
    return {"x": x.to(torch.bfloat16), "gamma": gamma.to(torch.bfloat16)}


def rmsnorm_bwd_inputs(rows: int, cols: int, seed: int = 0) -> dict:
    """bf16 CPU tensors x [rows, cols], gamma [cols] (as rmsnorm_inputs), the
    gradient dy of the norm's output and gin of the skip path [rows, cols]."""
    out = rmsnorm_inputs(rows, cols, seed)
    base = f"rmsnorm_bwd/{rows}x{cols}"
    out["dy"] = normal((rows, cols), 1e-3, seed, base + "/dy").to(torch.bfloat16)
    out["gin"] = normal((rows, cols), 1e-3, seed, base + "/gin").to(torch.bfloat16)
    return out


def residual_inputs(rows: int, cols: int, seed: int = 0) -> dict:
    """bf16 CPU tensors a (the residual stream, as rmsnorm_inputs' x) and b
    (a projection's output) [rows, cols], and gamma [cols]."""
    d = rmsnorm_inputs(rows, cols, seed)
    b = normal((rows, cols), 1.0, seed, f"residual/{rows}x{cols}/b").to(torch.bfloat16)
    return {"a": d["x"], "b": b, "gamma": d["gamma"]}
