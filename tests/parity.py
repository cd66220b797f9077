"""Helpers for the GPU parity tests: run the same seeded bf16 inputs through
the HIP library (via its C ABI) and through the CPU oracle, and compare.

Tolerance gates (reading of the stated bounds, applied per comparison):
  * codes and scales: bit-exact;
  * GEMM, FP32 output: relative Frobenius error <= 1e-3 and
    max |C - R| / max(|R|, 1e-2) <= 5e-3 against the oracle's FP32 result;
  * GEMM, bf16 output: the relative Frobenius gate is taken against the
    oracle's result rounded to bf16 (rounding alone is ~1.5e-3 relative
    against an unrounded reference), the max-element gate against the
    oracle's FP32 result (bf16 rounding is at most 2^-8 < 5e-3 relative).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

REL_FRO_GATE = 1e-3
MAX_REL_GATE = 5e-3


def say(*a):
    """Name the case on stderr (uncaptured, flushed) before a GPU step."""
    print("[case]", *a, file=sys.__stderr__, flush=True)


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda:0").contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def gate_fp32(c: np.ndarray, ref32: np.ndarray):
    rf = oracle.rel_fro(c, ref32)
    mr = oracle.max_rel(c, ref32)
    return rf, mr, (rf <= REL_FRO_GATE and mr <= MAX_REL_GATE)


def gate_bf16(c_bits: np.ndarray, ref32: np.ndarray):
    c = oracle.bf16_bits_to_f32(c_bits)
    ref_b = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(np.ascontiguousarray(ref32, np.float32)))
    rf = oracle.rel_fro(c, ref_b)
    mr = oracle.max_rel(c, ref32)
    return rf, mr, (rf <= REL_FRO_GATE and mr <= MAX_REL_GATE)


def random_bf16(shape, std=1.0, seed=0, stream="t"):
    return synth.normal(shape, std, seed, stream).to(torch.bfloat16)
