"""Host logic of bench.py: the step enqueues every layer's own launches, in
order, with that layer's shapes (checked with a stand-in binding, no GPU)."""
from __future__ import annotations

import sys
import types

import bench


class _Buf:
    def data_ptr(self):
        return 0

    def numel(self):
        return 16


def _layer(name, T, din, dout):
    L = types.SimpleNamespace(spec=types.SimpleNamespace(name=name), T=T, Tp=T, din=din, dout=dout)
    for a in ("x", "qx", "sx", "qtx", "stx", "w", "qw", "qtw", "sw", "y", "dy", "qdy", "sdy",
              "qtdy", "stdy", "dx", "dw", "ws"):
        setattr(L, a, _Buf())
    L.gemms = [("gemm_fwd_bf16", 0, T, dout, din), ("gemm_dgrad_bf16", 1, T, din, dout),
               ("gemm_wgrad_fp32", 2, dout, din, T)]
    return L


def test_step_calls_bind_each_layer():
    seen = []
    pf = types.SimpleNamespace(
        GEMM_FWD=0, GEMM_DGRAD=1, GEMM_WGRAD=2, OUT_BF16=0, OUT_FP32=1,
        puro_fp8_quant_act=lambda x, r, c, *a: seen.append(("act", r, c)) or 0,
        puro_fp8_quant_weight=lambda w, n, k, *a: seen.append(("weight", n, k)) or 0,
        puro_fp8_gemm_blockscaled=lambda m, M, N, K, *a: seen.append(("gemm", m, M, N, K)) or 0)
    layers = [_layer("a", 256, 128, 384), _layer("b", 512, 256, 128)]
    calls = bench.step_calls(pf, layers, None)
    assert [c[0] for c in calls] == ["a"] * 6 + ["b"] * 6
    for _, _, _, fn in calls:
        assert fn() == 0
    expect = []
    for T, din, dout in ((256, 128, 384), (512, 256, 128)):
        expect += [("act", T, din), ("weight", dout, din), ("gemm", 0, T, dout, din),
                   ("act", T, dout), ("gemm", 1, T, din, dout), ("gemm", 2, dout, din, T)]
    assert seen == expect
    works = [c[2] for c in calls]
    assert works[2] == 2.0 * 256 * 384 * 128 and works[8] == 2.0 * 512 * 128 * 256


def test_ingest_mfma_weights_by_duration_and_gates_on_code(tmp_path, monkeypatch):
    """The matrix-core file: MfmaUtil averaged with each dispatch's duration as
    weight, MOPS x 512 as FLOP, and the entry withheld once the kernel code
    differs from the code the counters were taken on."""
    name = "void puro::gemm_bs_kernel<0, 0>(unsigned char const*, int)"
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    rows = [(1, "MfmaUtil", 40.0, 0, 100), (1, "SQ_INSTS_VALU_MFMA_MOPS_F8", 1e6, 0, 100),
            (2, "MfmaUtil", 60.0, 1000, 1300), (2, "SQ_INSTS_VALU_MFMA_MOPS_F8", 1e6, 1000, 1300),
            (3, "GRBM_GUI_ACTIVE", 5.0, 2000, 2010)]
    csv_path = tmp_path / "c.csv"
    csv_path.write_text(head + "".join(f'{d},"{name}",{c},{v},{a},{b}\n' for d, c, v, a, b in rows))
    monkeypatch.setattr(bench, "MFMA_FILE", str(tmp_path / "m.json"))
    bench.ingest_mfma(str(csv_path))
    assert bench.mfma_busy_for("void puro::gemm_bs_kernel<0, 0>") == 55.0
    entry = bench._profile_entry(bench.MFMA_FILE, "void puro::gemm_bs_kernel<0, 0>")
    assert entry["dispatches"] == 2 and entry["f8_flop_per_dispatch"] == 512e6
    # a comment edit keeps the entry, a code edit drops it
    src = tmp_path / "gemm.hip"
    src.write_text(open(bench.GEMM_SOURCES[0]).read() + "\n// a comment\n")
    monkeypatch.setattr(bench, "GEMM_SOURCES", [str(src)] + bench.GEMM_SOURCES[1:])
    assert bench.mfma_busy_for("void puro::gemm_bs_kernel<0, 0>") == 55.0
    src.write_text(open(str(src)).read() + "int changed_code;\n")
    assert bench.mfma_busy_for("void puro::gemm_bs_kernel<0, 0>") is None


def test_ingest_pmc_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    """The traffic file: per kernel, FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, averaged over dispatches) scaled by what the same counters read
    for the 1 GiB copy (bytes expected / bytes counted)."""
    head = "Kernel_Name,Counter_Value\n"
    k = "void puro::gemm_bs_kernel<0, 0>(int)"
    neg = "void at::native::neg_kernel(float)"

    def csv(name, rows):
        path = tmp_path / name
        path.write_text(head + "".join(f'"{n}",{v}\n' for n, v in rows))
        return str(path)

    fetch = csv("f.csv", [(k, 1000.0), (k, 3000.0)])
    write = csv("w.csv", [(k, 500.0), (k, 500.0)])
    copy_f = csv("cf.csv", [(neg, 524288.0)])          # half of 1 GiB counted -> factor 2
    copy_w = csv("cw.csv", [(neg, 1048576.0)])         # all of it -> factor 1
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    bench.ingest_pmc(fetch, write, copy_f, copy_w)
    import json
    doc = json.load(open(bench.TRAFFIC_FILE))
    assert doc["copy_factor_fetch"] == 2.0 and doc["copy_factor_write"] == 1.0
    e = doc["kernels"][k]
    assert e["dispatches"] == 2
    assert e["hbm_bytes_per_dispatch"] == 2000.0 * 1024 * 2.0 + 500.0 * 1024 * 1.0
    assert bench.traffic_for("void puro::gemm_bs_kernel<0, 0>") == e["hbm_bytes_per_dispatch"]


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    """bench.py measures one GPU; --gpus N > 1 exits with status 2 and says
    why, before touching the GPU."""
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    err = capsys.readouterr().err
    assert "one GPU" in err or "single" in err


def test_roofline_classes_are_gemm_classes():
    """The classes timed inside the timed region are GEMM launch classes with
    kernel symbols, so the roofline always names a GEMM kernel."""
    for c in bench.ROOFLINE_CLASSES:
        assert c.startswith("gemm") and c in bench.KERNEL_SYMBOLS


def test_vendor_fp8_leg_is_omitted_without_fp8_support():
    """A torch build without an FP8 dtype or _scaled_mm gives no context leg
    (None) rather than an error, so the bench line is still printed."""
    assert bench.fp8_tensorwise_reference(types.SimpleNamespace(), [], 1) is None
    no_mm = types.SimpleNamespace(float8_e4m3fn=object())
    assert bench.fp8_tensorwise_reference(no_mm, [], 1) is None
