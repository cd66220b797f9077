#!/usr/bin/env python3
"""Throughput of the block-scaled FP8 linear-layer hot path on one MI355X.

One step = the full FP8 path of every linear layer of one transformer block
(2048 hidden, 16 heads, 8192 FFN; QKV 2048->6144, out-proj 2048->2048,
up/gate 2048->16384, down 8192->2048) on a micro-batch of 8 x 4096 = 32768
tokens, inputs already resident in HBM:

  per linear:  quant_act(X, 1x128 + 128x1^T)   quant_weight(W, 128x128 + W^T)
               FWD    Y  = X . W^T      (bf16 out)
               quant_act(dY, 1x128 + 128x1^T)
               DGRAD  dX = dY . W       (bf16 out)
               WGRAD  dW = dY^T . X     (FP32 out)

The metric is the GEMM work of the step (2*M*N*K summed over the 12 GEMMs,
13.19 TFLOP) divided by the whole step's time (quantizers included), in
TFLOP/s.  Inside the timed region HIP events bracket the launches of the
FWD and DGRAD GEMMs (on the stream the kernels run on): the dominant
kernel's achieved rate, reported against the MI355X dense FP8 MFMA peak
(5.0 PFLOP/s), comes from them.  The per-kernel table ("kernels", the
quantizers' rates against HBM at 8 TB/s) comes from the same K steps run
again with events around every launch.

For context, the same 12 products are also timed as plain BF16 GEMMs, after
the FP8 timed region: with the vendor library (torch.matmul,
"bf16_reference") and with this library's own tiling on the bf16 matrix
cores ("bf16_tiled"), each with the FP8/BF16 step and GEMM speedups.  The
vendor's FP8 GEMM with one scale per tensor (torch._scaled_mm,
"fp8_tensorwise_reference") runs the same products on the step's FP8 codes:
a tuned FP8 GEMM without block scales, as a yardstick for the block-scaled
GEMMs (not the same method).

Quantize-on-produce ("produce"): the BF16 neighbour ops of one block at the
same token count (RMSNorm x2 before QKV and up/gate, SwiGLU forward before
down, SwiGLU backward after down's DGRAD), each writing FP8 operands straight
from the op, timed against the unfused pair (the op writing bf16, then
quant_act on it).  Not part of the step above, whose inputs are bf16 tensors.

After the timed region every launch of one step is also run on its own, 50
times, each right after a 512 MiB write that evicts the L2s and the MALL
("kernels_cold": median, p10, p90 per launch), and a plain 1 GiB elementwise
kernel gives the device's achievable HBM rate ("hbm_copy_reference").

The CPU baseline times the plain CPU oracle (quantize + block-scaled GEMM in
all three modes) on a bounded slice of the same workload: the first
`--cpu-tokens` tokens of every linear layer, all host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s (fwd+dgrad+wgrad) and % of MI355X FP8 peak"
FP8_PEAK_TFLOPS = 5000.0          # MI355X dense FP8 MFMA, published
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_block_stack.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_block_stack.json")
_CSRC = os.path.join(ROOT, "fp8_block_scaled_tile_amd", "csrc")
# the sources each profiled kernel is compiled from (its file and the headers it includes)
GEMM_SOURCES = [os.path.join(_CSRC, n) for n in ("gemm.hip", "device_common.hpp")]
QUANT_SOURCES = [os.path.join(_CSRC, n) for n in ("quant.hip", "quant_block.hpp", "device_common.hpp")]

# the GEMM classes whose launches carry events inside the timed region: the
# dominant kernel is the one of these with the most time per step (FWD and
# DGRAD are within a few percent of each other; the WGRAD classes run fewer
# FLOP per step)
ROOFLINE_CLASSES = ("gemm_fwd_bf16", "gemm_dgrad_bf16")

# kernel symbol of each launch class (for matching rocprofv3 summaries)
KERNEL_SYMBOLS = {
    "gemm_fwd_bf16": "void puro::gemm_bs_kernel<0, 0>",
    "gemm_dgrad_bf16": "void puro::gemm_bs_kernel<1, 0>",
    "gemm_wgrad_fp32": "void puro::gemm_bs_kernel<2, 1>",
    "gemm_wgrad_splitk": "void puro::gemm_bs_kernel<2, 3> + splitk_reduce_kernel<1>",
    "quant_act_dual": "void puro::quant_block_kernel<true, true, false, false>",
    "quant_weight_t": "void puro::quant_block_kernel<false, false, true, true>",
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="block_stack")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-tokens", type=int, default=3072,
                   help="token slice for the CPU-oracle baseline (0 = skip)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16-reference", action="store_true",
                   help="skip the GEMM comparisons: BF16 vendor and own tiling, and the vendor "
                        "FP8 GEMM with per-tensor scales (context only)")
    p.add_argument("--no-cold-stats", action="store_true",
                   help="skip the per-launch cold-cache distribution (median / p10 / p90)")
    p.add_argument("--cold-iters", type=int, default=50,
                   help="cold-cache runs per launch of the step")
    p.add_argument("--no-produce", action="store_true",
                   help="skip the quantize-on-produce comparison (fused vs op + quant_act)")
    p.add_argument("--produce-iters", type=int, default=20,
                   help="timed calls per variant in the quantize-on-produce comparison")
    p.add_argument("--ingest-pmc", nargs=4,
                   metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="turn rocprofv3 --pmc counter CSVs (bench run, then the copy "
                        "calibration run) into the traffic file and exit")
    p.add_argument("--ingest-mfma", metavar="MFMA_CSV",
                   help="turn a rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE "
                        "CSV of a bench run into the matrix-core file and exit")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (counter calibration) and exit")
    return p.parse_args()


def sha(paths) -> str:
    """Hash of a kernel's source code (its files in order): comments and blank
    lines are dropped, so editing a comment does not invalidate counters taken
    on the same code."""
    import re
    text = ""
    for path in paths:
        with open(path) as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


# ---- per-launch algorithmic work -------------------------------------------

def act_dual_bytes(rows, cols):
    # read bf16, write 1x128 codes + 128x1 transposed codes, two scale sets
    return rows * cols * (2 + 1 + 1) + 2 * (rows * cols // 128) * 4


def weight_t_bytes(n, k):
    return n * k * (2 + 1 + 1) + (n * k // (128 * 128)) * 4


class Linear:
    """Device buffers of one linear layer's FP8 path (allocated once)."""

    def __init__(self, torch, pf, spec, tensors):
        T, din, dout = spec.tokens, spec.d_in, spec.d_out
        Tp = (T + 127) // 128 * 128
        d = "cuda:0"
        u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16
        self.spec = spec
        self.T, self.Tp, self.din, self.dout = T, Tp, din, dout
        self.x = tensors["x"].to(d)
        self.w = tensors["w"].to(d)
        self.dy = tensors["dy"].to(d)
        self.qx = torch.empty((T, din), dtype=u8, device=d)
        self.sx = torch.empty((din // 128, T), dtype=f32, device=d)
        self.qtx = torch.empty((din, Tp), dtype=u8, device=d)
        self.stx = torch.empty((Tp // 128, din), dtype=f32, device=d)
        self.qw = torch.empty((dout, din), dtype=u8, device=d)
        self.qtw = torch.empty((din, dout), dtype=u8, device=d)
        self.sw = torch.empty((dout // 128, din // 128), dtype=f32, device=d)
        self.y = torch.empty((T, dout), dtype=bf16, device=d)
        self.qdy = torch.empty((T, dout), dtype=u8, device=d)
        self.sdy = torch.empty((dout // 128, T), dtype=f32, device=d)
        self.qtdy = torch.empty((dout, Tp), dtype=u8, device=d)
        self.stdy = torch.empty((Tp // 128, dout), dtype=f32, device=d)
        self.dx = torch.empty((T, din), dtype=bf16, device=d)
        self.dw = torch.empty((dout, din), dtype=f32, device=d)
        self.gemms = [  # (class, mode, M, N, K)
            ("gemm_fwd_bf16", pf.GEMM_FWD, T, dout, din),
            ("gemm_dgrad_bf16", pf.GEMM_DGRAD, T, din, dout),
            (None, pf.GEMM_WGRAD, dout, din, Tp),
        ]
        ws_need = max(pf.puro_fp8_gemm_workspace_bytes(m, M, N, K) for _, m, M, N, K in self.gemms)
        self.ws = torch.empty(max(ws_need, 16), dtype=u8, device=d)
        self.wgrad_split = pf.puro_fp8_gemm_workspace_bytes(pf.GEMM_WGRAD, dout, din, Tp) > 0
        self.gemms[2] = ("gemm_wgrad_splitk" if self.wgrad_split else "gemm_wgrad_fp32",
                         pf.GEMM_WGRAD, dout, din, Tp)

    def flops(self):
        return sum(2.0 * M * N * K for _, _, M, N, K in self.gemms)


def spec0_tokens(specs):
    return specs[0].tokens


def check(pf, rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: {pf.puro_fp8_status_string(rc)}")


def step_calls(pf, layers, stream):
    """The launches of one step in order: (layer, class, work, fn), where work
    is the launch's algorithmic bytes (quantizers) or FLOP (GEMMs)."""
    P = lambda t: t.data_ptr()

    def layer_calls(L):     # a scope per layer: each lambda binds its own L
        return [
            ("quant_act_dual", act_dual_bytes(L.T, L.din), lambda: pf.puro_fp8_quant_act(
                P(L.x), L.T, L.din, P(L.qx), P(L.sx), P(L.qtx), P(L.stx), stream)),
            ("quant_weight_t", weight_t_bytes(L.dout, L.din), lambda: pf.puro_fp8_quant_weight(
                P(L.w), L.dout, L.din, P(L.qw), P(L.qtw), P(L.sw), stream)),
            (L.gemms[0][0], 2.0 * L.T * L.dout * L.din, lambda: pf.puro_fp8_gemm_blockscaled(
                pf.GEMM_FWD, L.T, L.dout, L.din, P(L.qx), P(L.sx), P(L.qw), P(L.sw), P(L.y),
                pf.OUT_BF16, 0, P(L.ws), L.ws.numel(), stream)),
            ("quant_act_dual", act_dual_bytes(L.T, L.dout), lambda: pf.puro_fp8_quant_act(
                P(L.dy), L.T, L.dout, P(L.qdy), P(L.sdy), P(L.qtdy), P(L.stdy), stream)),
            (L.gemms[1][0], 2.0 * L.T * L.din * L.dout, lambda: pf.puro_fp8_gemm_blockscaled(
                pf.GEMM_DGRAD, L.T, L.din, L.dout, P(L.qdy), P(L.sdy), P(L.qtw), P(L.sw), P(L.dx),
                pf.OUT_BF16, 0, P(L.ws), L.ws.numel(), stream)),
            (L.gemms[2][0], 2.0 * L.dout * L.din * L.Tp, lambda: pf.puro_fp8_gemm_blockscaled(
                pf.GEMM_WGRAD, L.dout, L.din, L.Tp, P(L.qtdy), P(L.stdy), P(L.qtx), P(L.stx),
                P(L.dw), pf.OUT_FP32, 0, P(L.ws), L.ws.numel(), stream)),
        ]

    return [(L.spec.name, name, work, fn) for L in layers for name, work, fn in layer_calls(L)]


def run_step(pf, layers, stream, rec=None):
    """Enqueue one step.  rec(name, work) returns (start_event, end_event) to
    bracket a launch, or None to launch unbracketed."""
    for _, name, work, fn in step_calls(pf, layers, stream):
        ev = rec(name, work) if rec else None
        if ev:
            ev[0].record()
        check(pf, fn(), name)
        if ev:
            ev[1].record()


def cold_kernel_stats(torch, pf, layers, stream, iters):
    """Every launch of one step on its own, `iters` times, each right after a
    512 MiB write that evicts the L2s and the MALL: median, p10 and p90 of the
    event-timed duration per launch, and the rate at the median."""
    import numpy as np
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = []
    for layer, name, work, fn in step_calls(pf, layers, stream):
        evs = []
        for _ in range(iters):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            check(pf, fn(), name)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs])
        p10, p50, p90 = (float(v) for v in np.percentile(t, [10, 50, 90]))
        e = {"layer": layer, "kernel": name, "median_ms": round(p50, 4), "p10_ms": round(p10, 4),
             "p90_ms": round(p90, 4)}
        if name.startswith("gemm"):
            e["tflops"] = round(work / (p50 * 1e-3) / 1e12, 1)
        else:
            e["gbps"] = round(work / (p50 * 1e-3) / 1e9, 1)
        out.append(e)
    del flush
    return out


def _median_ms(torch, fn, iters):
    """Median event-timed duration of fn() over `iters` back-to-back calls
    (after two untimed ones)."""
    import numpy as np
    for _ in range(2):
        fn()
    evs = []
    for _ in range(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def produce_bench(torch, pf, tokens, hidden, ffn, stream, iters, seed):
    """Fused (op -> FP8 codes, 1x128 + 128x1^T) against unfused (op -> bf16,
    then quant_act) for the neighbour ops of one block.  Algorithmic bytes:
    inputs read once, outputs written once (codes 1 B + 1 B, scales 8 B per
    128 elements; bf16 2 B)."""
    import synth
    dual = 2.0 + 8.0 / 128.0                       # q + qt + s + st per element
    ops = []

    def bufs(rows, cols):
        rp = (rows + 127) // 128 * 128
        u8, f32 = torch.uint8, torch.float32
        return {"q": torch.empty((rows, cols), dtype=u8, device="cuda"),
                "s": torch.empty((cols // 128, rows), dtype=f32, device="cuda"),
                "qt": torch.empty((cols, rp), dtype=u8, device="cuda"),
                "st": torch.empty((rp // 128, cols), dtype=f32, device="cuda"),
                "y": torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")}

    def qa(b, rows, cols):
        return lambda: check(pf, pf.puro_fp8_quant_act(b["y"].data_ptr(), rows, cols, b["q"].data_ptr(),
                                                       b["s"].data_ptr(), b["qt"].data_ptr(),
                                                       b["st"].data_ptr(), stream), "quant_act")

    def measure(name, rows, cols, fused, op_only, quant, bytes_fused, bytes_unfused, count):
        f_ms = _median_ms(torch, fused, iters)
        o_ms = _median_ms(torch, op_only, iters)
        q_ms = _median_ms(torch, quant, iters)
        rate = bytes_fused / (f_ms * 1e-3) / 1e9
        ops.append({"op": name, "out_shape": [rows, cols], "per_block": count,
                    "fused_ms": round(f_ms, 4), "unfused_ms": round(o_ms + q_ms, 4),
                    "unfused_op_ms": round(o_ms, 4), "unfused_quant_ms": round(q_ms, 4),
                    "speedup": round((o_ms + q_ms) / f_ms, 3),
                    "fused_mb": round(bytes_fused / 1e6, 1), "unfused_mb": round(bytes_unfused / 1e6, 1),
                    "fused_gbps": round(rate, 1), "frac_hbm_peak": round(rate / HBM_PEAK_GBPS, 4)})

    # SwiGLU forward: gu [T, 2F] -> h [T, F]
    d = synth.swiglu_inputs(tokens, ffn, seed=seed)
    gu, dh = d["gu"].to("cuda"), d["dh"].to("cuda")
    del d
    b = bufs(tokens, ffn)
    P = lambda t: t.data_ptr()
    measure("swiglu_fwd", tokens, ffn,
            lambda: check(pf, pf.puro_fp8_swiglu_quant(P(gu), tokens, ffn, P(b["q"]), P(b["s"]), P(b["qt"]),
                                                       P(b["st"]), None, stream), "swiglu_quant"),
            lambda: check(pf, pf.puro_fp8_swiglu_quant(P(gu), tokens, ffn, None, None, None, None,
                                                       P(b["y"]), stream), "swiglu"),
            qa(b, tokens, ffn),
            tokens * ffn * (4.0 + dual), tokens * ffn * (4.0 + 2.0 + 2.0 + dual), 1)
    del b
    # SwiGLU backward: dh [T, F], gu -> (d gate | d up) [T, 2F]
    b = bufs(tokens, 2 * ffn)
    measure("swiglu_bwd", tokens, 2 * ffn,
            lambda: check(pf, pf.puro_fp8_swiglu_bwd_quant(P(dh), P(gu), tokens, ffn, P(b["q"]), P(b["s"]),
                                                           P(b["qt"]), P(b["st"]), None, stream),
                          "swiglu_bwd_quant"),
            lambda: check(pf, pf.puro_fp8_swiglu_bwd_quant(P(dh), P(gu), tokens, ffn, None, None, None,
                                                           None, P(b["y"]), stream), "swiglu_bwd"),
            qa(b, tokens, 2 * ffn),
            tokens * ffn * (6.0 + 2 * dual), tokens * ffn * (6.0 + 4.0 + 2 * (2.0 + dual)), 1)
    del b, gu, dh
    # RMSNorm: x [T, H], gamma [H] -> y [T, H] (twice per block)
    d = synth.rmsnorm_inputs(tokens, hidden, seed=seed)
    x, gamma = d["x"].to("cuda"), d["gamma"].to("cuda")
    rstd = torch.empty(tokens, dtype=torch.float32, device="cuda")
    b = bufs(tokens, hidden)
    measure("rmsnorm", tokens, hidden,
            lambda: check(pf, pf.puro_fp8_rmsnorm_quant(P(x), P(gamma), tokens, hidden, 1e-6, P(rstd),
                                                        P(b["q"]), P(b["s"]), P(b["qt"]), P(b["st"]),
                                                        None, stream), "rmsnorm_quant"),
            lambda: check(pf, pf.puro_fp8_rmsnorm_quant(P(x), P(gamma), tokens, hidden, 1e-6, P(rstd),
                                                        None, None, None, None, P(b["y"]), stream),
                          "rmsnorm"),
            qa(b, tokens, hidden),
            tokens * hidden * (2.0 + dual) + 4.0 * tokens,
            tokens * hidden * (2.0 + 2.0 + 2.0 + dual) + 4.0 * tokens, 2)
    del b, x, gamma, rstd
    fused = sum(o["fused_ms"] * o["per_block"] for o in ops)
    unfused = sum(o["unfused_ms"] * o["per_block"] for o in ops)
    return {"ops": ops, "fused_ms_per_block": round(fused, 4),
            "unfused_ms_per_block": round(unfused, 4),
            "saved_ms_per_block": round(unfused - fused, 4),
            "kind": "neighbour ops of one block writing FP8 operands directly vs op (bf16 out) + "
                    "quant_act; median of event-timed calls; not part of the step"}


def hbm_copy_reference(torch):
    """A plain elementwise kernel of known size on the same device: torch.neg
    over 2^28 float32 (1 GiB read, 1 GiB written), best of 10."""
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    best = 1e9
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.neg(x, out=y)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del x, y
    return {"kernel": "torch.neg over 2^28 float32 (1 GiB in, 1 GiB out)", "gbps": round(2 * (1 << 30) / (best * 1e-3) / 1e9, 1)}


# ---- counters (rocprofv3 --pmc) ----------------------------------------------

def _read_pmc_csv(path):
    """{kernel_name: [values per dispatch]} from a rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
            val = row.get("Counter_Value") or row.get("Counter-Value")
            if val is None:
                continue
            out.setdefault(name, []).append(float(val))
    return out


def ingest_pmc(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Write the traffic file: per kernel, FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) scaled by the factor a plain copy of known size reads on the
    same counters (bytes expected / bytes counted)."""
    fetch = _read_pmc_csv(fetch_csv)
    write = _read_pmc_csv(write_csv)
    cf = _read_pmc_csv(copy_fetch_csv)
    cw = _read_pmc_csv(copy_write_csv)
    copy_bytes = float(1 << 30)
    def copy_factor(tbl):
        vals = [v for k, vs in tbl.items() if "neg" in k.lower() for v in vs]
        if not vals:
            return None
        return copy_bytes / (max(vals) * 1024.0)
    ff, fw = copy_factor(cf), copy_factor(cw)
    kernels = {}
    for name in set(fetch) | set(write):
        f = fetch.get(name, [])
        w = write.get(name, [])
        if not f or not w:
            continue
        kernels[name] = {
            "fetch_kib_per_dispatch": sum(f) / len(f),
            "write_kib_per_dispatch": sum(w) / len(w),
            "dispatches": len(f),
            "hbm_bytes_per_dispatch": (sum(f) / len(f) * 1024.0 * (ff or 1.0) +
                                       sum(w) / len(w) * 1024.0 * (fw or 1.0)),
        }
    doc = {"copy_factor_fetch": ff, "copy_factor_write": fw,
           "gemm_source_sha": sha(GEMM_SOURCES), "quant_source_sha": sha(QUANT_SOURCES),
           "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
    print(f"wrote {TRAFFIC_FILE}: {len(kernels)} kernels")


def ingest_mfma(csv_path):
    """Write the matrix-core file from one rocprofv3 pass with the derived
    MfmaUtil (busy cycles of the MFMA units over GPU-active cycles x SIMDs)
    and SQ_INSTS_VALU_MFMA_MOPS_F8 (FP8 multiply-add operations / 512): per
    kernel, the duration-weighted MfmaUtil and the FP8 FLOP per dispatch."""
    import csv
    per = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            d = per.setdefault(row["Dispatch_Id"], {"name": row["Kernel_Name"],
                                                    "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
            d[row["Counter_Name"]] = float(row["Counter_Value"])
    kernels = {}
    for d in per.values():
        if "MfmaUtil" not in d:
            continue
        k = kernels.setdefault(d["name"], {"dispatches": 0, "ns": 0, "util_ns": 0.0, "f8_flop": 0.0})
        k["dispatches"] += 1
        k["ns"] += d["ns"]
        k["util_ns"] += d["MfmaUtil"] * d["ns"]
        k["f8_flop"] += d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) * 512.0
    out = {name: {"dispatches": k["dispatches"],
                  "mfma_util_pct": k["util_ns"] / k["ns"] if k["ns"] else 0.0,
                  "f8_flop_per_dispatch": k["f8_flop"] / k["dispatches"]}
           for name, k in kernels.items()}
    doc = {"gemm_source_sha": sha(GEMM_SOURCES), "quant_source_sha": sha(QUANT_SOURCES), "kernels": out}
    with open(MFMA_FILE, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
    print(f"wrote {MFMA_FILE}: {len(out)} kernels")


def _profile_entry(path, symbol_prefix):
    """The entry of a counter file for a kernel, or None if the file is absent
    or its counters were taken on a different version of the kernel code."""
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    src = GEMM_SOURCES if "gemm" in symbol_prefix else QUANT_SOURCES
    key = "gemm_source_sha" if "gemm" in symbol_prefix else "quant_source_sha"
    if doc.get(key) != sha(src):
        return None
    for name, v in doc.get("kernels", {}).items():
        if name.startswith(symbol_prefix):
            return v
    return None


def mfma_busy_for(symbol_prefix):
    """Duration-weighted MfmaUtil (%) of a kernel from the counter file, or None."""
    v = _profile_entry(MFMA_FILE, symbol_prefix)
    return round(v["mfma_util_pct"], 2) if v else None


def traffic_for(symbol_prefix):
    """HBM bytes per dispatch for a kernel, or None if the counters are absent
    or were taken on a different version of the kernel code."""
    v = _profile_entry(TRAFFIC_FILE, symbol_prefix)
    return v["hbm_bytes_per_dispatch"] if v else None


# ---- BF16 comparator ------------------------------------------------------------

def bf16_reference(torch, layers, steps):
    """The same 12 products as plain BF16 GEMMs of the vendor library
    (torch.matmul -> hipBLASLt / rocBLAS), bf16 outputs, with the transposed
    operands materialized beforehand (outside the timing).  This is the
    unquantized linear layer the FP8 path replaces; it is context for the
    FP8/BF16 speedup, not part of the measured step."""
    bufs = []
    for L in layers:
        bufs.append((L.x, L.w.t().contiguous(), L.dy, L.w, L.dy.t().contiguous(),
                     torch.empty_like(L.y), torch.empty_like(L.dx),
                     torch.empty((L.dout, L.din), dtype=torch.bfloat16, device="cuda:0")))

    def step():
        for x, wt, dy, w, dyt, y, dx, dw in bufs:
            torch.matmul(x, wt, out=y)          # Y  = X . W^T
            torch.matmul(dy, w, out=dx)         # dX = dY . W
            torch.matmul(dyt, x, out=dw)        # dW = dY^T . X
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = sum(2.0 * L.T * L.din * L.dout * 3 for L in layers)
    del bufs
    return ms, flops / (ms * 1e-3) / 1e12


def bf16_tiled(torch, pf, layers, steps, stream):
    """The same 12 products through this library's BF16 comparator GEMM
    (puro_bf16_gemm_nt: the FP8 path's own tiling on the bf16 matrix cores,
    no block scales), bf16 outputs, with the transposed operands materialized
    beforehand (outside the timing).  Kernel-for-kernel context for the FP8
    speedup, not part of the measured step."""
    P = lambda t: t.data_ptr()
    calls = []
    keep = []
    for L in layers:
        wt, dyt, xt = L.w.t().contiguous(), L.dy.t().contiguous(), L.x.t().contiguous()
        y, dx = torch.empty_like(L.y), torch.empty_like(L.dx)
        dw = torch.empty((L.dout, L.din), dtype=torch.bfloat16, device="cuda:0")
        shapes = [(L.T, L.dout, L.din, L.x, L.w, y),      # Y  = X . W^T
                  (L.T, L.din, L.dout, L.dy, wt, dx),     # dX = dY . W   (B = W^T)
                  (L.dout, L.din, L.T, dyt, xt, dw)]      # dW = dY^T . X (A = dY^T, B = X^T)
        need = max(pf.puro_bf16_gemm_nt_workspace_bytes(M, N, K) for M, N, K, *_ in shapes)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0")
        keep += [wt, dyt, xt, y, dx, dw, ws]
        for M, N, K, a, b, c in shapes:
            calls.append((M, N, K, P(a), P(b), P(c), P(ws), ws.numel()))

    def step():
        for M, N, K, a, b, c, w, wb in calls:
            check(pf, pf.puro_bf16_gemm_nt(M, N, K, a, b, c, w, wb, stream), "bf16 comparator")
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = sum(2.0 * M * N * K for M, N, K, *_ in calls)
    del keep
    return ms, flops / (ms * 1e-3) / 1e12


def fp8_tensorwise_reference(torch, layers, steps):
    """The same 12 products through the vendor library's FP8 GEMM
    (torch._scaled_mm -> hipBLASLt) on the codes the step's quantizers wrote,
    with ONE scale per tensor: no per-block scales and no fold, so it is not
    the block-scaled method.  It shows what a tuned FP8 GEMM without block
    scales takes on these shapes; context, not part of the measured step.
    Outputs are bf16 for FWD / DGRAD and FP32 for WGRAD where the vendor path
    serves FP32 (bf16 otherwise, reported).  Returns None if this torch build
    has no FP8 GEMM."""
    f8 = getattr(torch, "float8_e4m3fn", None)
    if f8 is None or not hasattr(torch, "_scaled_mm"):
        return None
    one = torch.ones((), dtype=torch.float32, device="cuda:0")
    calls = []
    wgrad_dtype = torch.float32
    for L in layers:
        calls.append((L.qx.view(f8), L.qw.view(f8), torch.bfloat16))      # Y  = X . W^T
        calls.append((L.qdy.view(f8), L.qtw.view(f8), torch.bfloat16))    # dX = dY . W
        calls.append((L.qtdy.view(f8), L.qtx.view(f8), None))             # dW = dY^T . X
    try:
        a, b, _ = calls[2]
        torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.float32)
    except (RuntimeError, TypeError, ValueError, NotImplementedError):
        wgrad_dtype = torch.bfloat16
    try:
        def step():
            for a, b, dt in calls:
                torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=dt or wgrad_dtype)
        for _ in range(3):
            step()
    except (RuntimeError, TypeError, ValueError, NotImplementedError):
        return None             # this torch build has no usable FP8 GEMM: context leg omitted
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = sum(2.0 * a.shape[0] * b.shape[0] * a.shape[1] for a, b, _ in calls)
    return ms, flops / (ms * 1e-3) / 1e12, str(wgrad_dtype).replace("torch.", "")


# ---- CPU baseline --------------------------------------------------------------

def cpu_baseline(specs, host_tensors, tokens):
    """The oracle (quantize + block-scaled GEMM, all three modes) on the first
    `tokens` tokens of every linear layer; GEMM FLOP of that slice / time."""
    import numpy as np
    import oracle
    import synth
    oracle.build(force=False)
    # the host's share of cores: OMP_NUM_THREADS where the host sets it
    oracle.set_threads(max(1, min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", "16")))))
    flops = 0.0
    t0 = time.perf_counter()
    for spec, t in zip(specs, host_tensors):
        x = synth.bits(t["x"][:tokens])
        w = synth.bits(t["w"])
        dy = synth.bits(t["dy"][:tokens])
        qx, sx = oracle.quant_rowwise(x)
        qtx, stx = oracle.quant_colwise(x)
        qw, qtw, sw = oracle.quant_weight(w)
        qdy, sdy = oracle.quant_rowwise(dy)
        qtdy, stdy = oracle.quant_colwise(dy)
        oracle.gemm_blockscaled(oracle.MODE_FWD, qx, sx, qw, sw)
        oracle.gemm_blockscaled(oracle.MODE_DGRAD, qdy, sdy, qtw, sw)
        oracle.gemm_blockscaled(oracle.MODE_WGRAD, qtdy, stdy, qtx, stx)
        tp = qtx.shape[1]
        flops += 2.0 * tokens * spec.d_out * spec.d_in * 2 + 2.0 * spec.d_out * spec.d_in * tp
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.get_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": (f"first {tokens} tokens of each of the {len(specs)} linear layers: "
                       f"quantize X, dY (1x128 and 128x1), W (128x128) and the FWD, DGRAD and "
                       f"WGRAD GEMMs of that slice ({flops / 1e9:.1f} GFLOP)")}


# ---- main --------------------------------------------------------------------------

def copy_calibration():
    """A plain elementwise copy of known size for calibrating the HBM byte
    counters: y = -x over 2^28 float32 (1 GiB read, 1 GiB written)."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print("copy calibration: 3 x neg over 1 GiB float32", flush=True)


def main():
    args = parse_args()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return 0
    if args.ingest_mfma:
        ingest_mfma(args.ingest_mfma)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the FP8 linear-layer path is measured on a single "
              f"MI355X (--gpus {args.gpus} is not supported; data-parallel sharding only "
              f"replicates this per-GPU work).", file=sys.stderr)
        return 2
    import torch
    if args.copy_calibration:
        copy_calibration()
        return 0

    import fp8_block_scaled_tile_amd as pf
    import synth

    wl = synth.workload(args.workload)
    specs = list(wl.linears)
    t_gen = time.perf_counter()
    host_tensors = [synth.linear_inputs(s, seed=args.seed) for s in specs]
    gen_s = time.perf_counter() - t_gen
    layers = [Linear(torch, pf, s, t) for s, t in zip(specs, host_tensors)]
    if args.no_cpu_baseline or args.cpu_tokens <= 0:
        del host_tensors
        host_tensors = None
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    step_flops = sum(L.flops() for L in layers)

    for _ in range(args.warmup):
        run_step(pf, layers, stream)
    torch.cuda.synchronize()

    # timed region: K steps.  Only the launches of the two largest GEMM
    # classes (FWD and DGRAD, bf16 out) are bracketed by events on their
    # stream, for the roofline of the dominant kernel; events around all 26
    # launches would cost the step 1-1.5%.
    def recorder(events, classes=None):
        def rec(name, work):
            if classes is not None and name not in classes:
                return None
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            events.append((name, work, ev))
            return ev
        return rec

    timed_events = []
    rec = recorder(timed_events, ROOFLINE_CLASSES)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(pf, layers, stream, rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps
    value = step_flops / (wall / args.steps) / 1e12

    # per-kernel breakdown: the same K steps again, every launch bracketed
    all_events = []
    rec_all = recorder(all_events)
    t1 = time.perf_counter()
    for _ in range(args.steps):
        run_step(pf, layers, stream, rec_all)
    torch.cuda.synchronize()
    ms_all_events = (time.perf_counter() - t1) * 1e3 / args.steps

    def per_class(events):
        per = {}
        for name, work, (e0, e1) in events:
            d = per.setdefault(name, {"launches": 0, "ms": 0.0, "work": 0.0})
            d["launches"] += 1
            d["ms"] += e0.elapsed_time(e1)
            d["work"] += work
        return per

    def describe(name, d):
        avg_ms = d["ms"] / d["launches"]
        avg_work = d["work"] / d["launches"]
        if name.startswith("gemm"):
            rate = avg_work / (avg_ms * 1e-3) / 1e12
            return {"symbol": KERNEL_SYMBOLS[name], "launches_per_step": d["launches"] // args.steps,
                    "avg_ms": round(avg_ms, 4), "avg_gflop": round(avg_work / 1e9, 2),
                    "tflops": round(rate, 1), "frac_fp8_peak": round(rate / FP8_PEAK_TFLOPS, 4),
                    "ms_per_step": round(d["ms"] / args.steps, 4)}
        rate = avg_work / (avg_ms * 1e-3) / 1e9
        return {"symbol": KERNEL_SYMBOLS[name], "launches_per_step": d["launches"] // args.steps,
                "avg_ms": round(avg_ms, 4), "avg_mb": round(avg_work / 1e6, 2),
                "gbps": round(rate, 1), "frac_hbm_peak": round(rate / HBM_PEAK_GBPS, 4),
                "ms_per_step": round(d["ms"] / args.steps, 4)}

    kernels = {name: describe(name, d) for name, d in per_class(all_events).items()}
    timed = {name: describe(name, d) for name, d in per_class(timed_events).items()}
    dom = max(timed, key=lambda k: timed[k]["ms_per_step"])
    dk = timed[dom]
    traffic = traffic_for(dk["symbol"])
    roofline = {"bound": "mfma", "achieved": dk["tflops"], "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dk["tflops"] / FP8_PEAK_TFLOPS, 4),
                "traffic": traffic, "mfma_busy_pct": mfma_busy_for(dk["symbol"]),
                "kernel": dk["symbol"], "launch_class": dom,
                "algorithmic_gflop_per_launch": dk["avg_gflop"], "avg_ms": dk["avg_ms"],
                "timed_in": "the timed region"}
    gemm_ms = sum(v["ms_per_step"] for k, v in kernels.items() if k.startswith("gemm"))
    quant_ms = sum(v["ms_per_step"] for k, v in kernels.items() if k.startswith("quant"))

    bf16 = None
    bf16_own = None
    if not args.no_bf16_reference:
        bms, btf = bf16_reference(torch, layers, args.steps)
        bf16 = {"value": round(btf, 1), "unit": "TFLOP/s", "ms_per_step": round(bms, 4),
                "kind": "vendor BF16 GEMM (torch.matmul -> hipBLASLt/rocBLAS), same 12 products, "
                        "bf16 outputs, transposed operands pre-materialized; context, not timed above",
                "fp8_step_speedup": round(bms / ms_per_step, 3),
                "fp8_gemm_speedup": round(bms / gemm_ms, 3) if gemm_ms else None}
        tms, ttf = bf16_tiled(torch, pf, layers, args.steps, stream)
        bf16_own = {"value": round(ttf, 1), "unit": "TFLOP/s", "ms_per_step": round(tms, 4),
                    "kind": "this library's BF16 comparator GEMM (the FP8 path's tiling on bf16 "
                            "matrix cores, no block scales), same 12 products, bf16 outputs, "
                            "transposed operands pre-materialized; context, not timed above",
                    "fp8_step_speedup": round(tms / ms_per_step, 3),
                    "fp8_gemm_speedup": round(tms / gemm_ms, 3) if gemm_ms else None}

    fp8_vendor = None
    if not args.no_bf16_reference:
        ref = fp8_tensorwise_reference(torch, layers, args.steps)
        if ref is not None:
            vms, vtf, wdt = ref
            fp8_vendor = {"value": round(vtf, 1), "unit": "TFLOP/s", "ms_per_step": round(vms, 4),
                          "kind": "vendor FP8 GEMM (torch._scaled_mm -> hipBLASLt) with one scale "
                                  "per tensor (no block scales, not the block-scaled method), "
                                  "same 12 products on the step's FP8 codes, bf16 FWD/DGRAD "
                                  f"outputs, {wdt} WGRAD output; context, not timed above",
                          "block_scaled_gemm_ratio": round(vms / gemm_ms, 3) if gemm_ms else None}

    produce = None
    if not args.no_produce:
        produce = produce_bench(torch, pf, spec0_tokens(specs), 2048, 8192, stream, args.produce_iters,
                                args.seed)

    cold = None
    copy_ref = None
    if not args.no_cold_stats:
        cold = cold_kernel_stats(torch, pf, layers, stream, args.cold_iters)
        copy_ref = hbm_copy_reference(torch)

    cpu = None
    if host_tensors is not None:
        cpu = cpu_baseline(specs, host_tensors, args.cpu_tokens)

    spec0 = specs[0]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": spec0.tokens, "hidden": 2048, "heads": 16,
                   "ffn": 8192, "linears": {s.name: [s.d_in, s.d_out] for s in specs},
                   "gemm_tflop_per_step": round(step_flops / 1e12, 4),
                   "parallelism": "single GPU"},
        "pct_of_fp8_peak": round(100.0 * value / FP8_PEAK_TFLOPS, 2),
        "gemm_only_tflops": round(step_flops / (gemm_ms * 1e-3) / 1e12, 1) if gemm_ms else None,
        "ms_per_step_all_events": round(ms_all_events, 4),
        "gemm_ms_per_step": round(gemm_ms, 4),
        "quant_ms_per_step": round(quant_ms, 4),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "bf16_reference": bf16,
        "bf16_tiled": bf16_own,
        "fp8_tensorwise_reference": fp8_vendor,
        "produce": produce,
        "kernels_cold": cold,
        "hbm_copy_reference": copy_ref,
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
