"""Host logic of bench.py: the step enqueues every layer's own launches, in
order, with that layer's shapes (checked with a stand-in binding, no GPU)."""
from __future__ import annotations

import sys
import types

import pytest

import bench


@pytest.fixture(autouse=True)
def _counter_files_in_tmp(tmp_path, monkeypatch):
    """Every test here reads and writes counter files under its own temporary
    directory, never the committed ones."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", bench.traffic_file())
    monkeypatch.setattr(bench, "MFMA_FILE", bench.mfma_file())


class _Buf:
    def data_ptr(self):
        return 0

    def numel(self):
        return 16


class _Ptr(_Buf):
    def __init__(self, v):
        self.v = v

    def data_ptr(self):
        return self.v


def _layer(name, T, din, dout, fwd_mode=0, dgrad_mode=1, fwd=True, dgrad=True, wgrad=True):
    spec = types.SimpleNamespace(name=name, fwd=fwd, dgrad=dgrad, wgrad=wgrad)
    L = types.SimpleNamespace(spec=spec, T=T, Tp=T, din=din, dout=dout)
    for a in ("x", "w", "sw", "y", "dy", "dx", "dw", "ws"):
        setattr(L, a, _Buf())
    L.x_row, L.x_col, L.dy_row, L.dy_col = fwd, wgrad, dgrad, wgrad
    L.qx, L.sx = (_Buf(), _Buf()) if fwd else (None, None)
    L.qtx, L.stx = (_Buf(), _Buf()) if wgrad else (None, None)
    L.qdy, L.sdy = (_Buf(), _Buf()) if dgrad else (None, None)
    L.qtdy, L.stdy = (_Buf(), _Buf()) if wgrad else (None, None)
    L.fwd_mode, L.dgrad_mode = fwd_mode, dgrad_mode
    L.need_q = (fwd and fwd_mode == 0) or (dgrad and dgrad_mode == 3)
    L.need_qt = (fwd and fwd_mode == 4) or (dgrad and dgrad_mode == 1)
    L.qw = _Ptr(16) if L.need_q else None          # tell the two weight code copies apart
    L.qtw = _Ptr(32) if L.need_qt else None
    L.fwd_b = L.qw if fwd_mode == 0 else L.qtw
    L.dgrad_b = L.qtw if dgrad_mode == 1 else L.qw
    L.fwd_fp32 = False
    L.gemms = ([("fwd", "gemm_fwd_bf16", fwd_mode, T, dout, din)] * fwd
               + [("dgrad", "gemm_dgrad_bf16", dgrad_mode, T, din, dout)] * dgrad
               + [("wgrad", "gemm_wgrad_fp32", 2, dout, din, T)] * wgrad)
    L.gemm = lambda kind: next(g for g in L.gemms if g[0] == kind)
    return L


def _pf(seen):
    return types.SimpleNamespace(
        GEMM_FWD=0, GEMM_DGRAD=1, GEMM_WGRAD=2, GEMM_DGRAD_W=3, GEMM_FWD_T=4, OUT_BF16=0,
        OUT_FP32=1,
        puro_fp8_quant_act=lambda x, r, c, q, s, qt, st, stream:
            seen.append(("act", r, c, q is not None, qt is not None)) or 0,
        puro_fp8_quant_weight=lambda w, n, k, q, qt, s, st: seen.append(("weight", n, k, q, qt)) or 0,
        puro_fp8_gemm_blockscaled=lambda m, M, N, K, a, sa, b, *r: seen.append(("gemm", m, M, N, K, b)) or 0)


def test_step_calls_bind_each_layer():
    """Each layer's launches, in order, with its own shapes, GEMM modes and
    weight code copies: layer a runs FWD + DGRAD (reads q and q^T), layer b
    FWD_T + DGRAD (reads q^T only, so the weight quantizer skips q)."""
    seen = []
    pf = _pf(seen)
    layers = [_layer("a", 256, 128, 384), _layer("b", 512, 256, 128, fwd_mode=4, dgrad_mode=1)]
    calls = bench.step_calls(pf, layers, None)
    assert [c[0] for c in calls] == ["a"] * 6 + ["b"] * 6
    for _, _, _, fn in calls:
        assert fn() == 0
    A = lambda r, c: ("act", r, c, True, True)
    expect = [A(256, 128), ("weight", 384, 128, 16, 32), ("gemm", 0, 256, 384, 128, 16),
              A(256, 384), ("gemm", 1, 256, 128, 384, 32), ("gemm", 2, 384, 128, 256, 0),
              A(512, 256), ("weight", 128, 256, None, 32), ("gemm", 4, 512, 128, 256, 32),
              A(512, 128), ("gemm", 1, 512, 256, 128, 32), ("gemm", 2, 128, 256, 512, 0)]
    assert seen == expect
    works = [c[2] for c in calls]
    assert works[2] == 2.0 * 256 * 384 * 128 and works[8] == 2.0 * 512 * 128 * 256
    assert works[1] == bench.weight_bytes(384, 128, 2) and works[7] == bench.weight_bytes(128, 256, 1)


def test_step_calls_follow_the_layer_gemm_set():
    """A forward-only layer quantizes X row-wise only and W without the
    transposed copy; a backward-only layer (DGRAD from the weight's codes +
    WGRAD) quantizes dY both ways, X column-wise only, W once."""
    seen = []
    pf = _pf(seen)
    fwd_only = _layer("qkv", 16384, 2048, 6144, dgrad=False, wgrad=False)
    bwd_only = _layer("down", 16384, 8192, 2048, dgrad_mode=3, fwd=False)
    calls = bench.step_calls(pf, [fwd_only, bwd_only], None)
    for _, _, _, fn in calls:
        assert fn() == 0
    assert [c[1] for c in calls] == ["quant_act_row", "quant_weight", "gemm_fwd_bf16",
                                     "quant_act_col", "quant_weight", "quant_act_dual",
                                     "gemm_dgrad_bf16", "gemm_wgrad_fp32"]
    assert seen == [("act", 16384, 2048, True, False), ("weight", 6144, 2048, 16, None),
                    ("gemm", 0, 16384, 6144, 2048, 16),
                    ("act", 16384, 8192, False, True), ("weight", 2048, 8192, 16, None),
                    ("act", 16384, 2048, True, True), ("gemm", 3, 16384, 8192, 2048, 16),
                    ("gemm", 2, 2048, 8192, 16384, 0)]
    assert calls[0][2] == bench.act_bytes(16384, 2048, True, False) == 16384 * 2048 * 3 + 16384 * 16 * 4
    assert calls[5][2] == bench.act_dual_bytes(16384, 2048)


def test_step_calls_grouped_weights():
    """With grouped weights the step starts with one launch over every
    layer's weight (each with the code copies its GEMMs read) and the layers
    launch no weight quantizer of their own."""
    import ctypes
    seen = []
    pf = _pf(seen)

    class Desc(ctypes.Structure):
        _fields_ = [("w", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                    ("q", ctypes.c_void_p), ("qt", ctypes.c_void_p), ("s", ctypes.c_void_p)]
    pf.WeightDesc = Desc
    pf.puro_fp8_quant_weight_grouped = lambda d, n, st: seen.append(
        ("grouped", n, [(d[i].n, d[i].k, d[i].q, d[i].qt) for i in range(n)])) or 0
    layers = [_layer("a", 256, 128, 384, dgrad_mode=3), _layer("b", 512, 256, 128, fwd_mode=4)]
    calls = bench.step_calls(pf, layers, None, grouped_weights=True)
    assert [c[1] for c in calls][:1] == ["quant_weight_grouped_t"]
    assert not any(c[1].startswith("quant_weight") for c in calls[1:])
    for _, _, _, fn in calls:
        assert fn() == 0
    assert seen[0] == ("grouped", 2, [(384, 128, 16, None), (128, 256, None, 32)])
    assert calls[0][2] == bench.weight_bytes(384, 128, 1) + bench.weight_bytes(128, 256, 1)
    # one weight only: the per-layer launch
    one = bench.step_calls(pf, layers[:1], None, grouped_weights=True)
    assert [c[1] for c in one][1] == "quant_weight"


def test_counter_files_are_per_workload():
    assert bench.traffic_file() == bench.TRAFFIC_FILE
    assert bench.traffic_file("qkv_fwd").endswith("profiles/traffic_qkv_fwd.json")
    assert bench.mfma_file("down_bwd").endswith("profiles/mfma_down_bwd.json")


def test_configs_name_the_workloads():
    import synth
    assert bench.CONFIGS["c5"] == "block_stack"
    for name in bench.CONFIGS.values():
        synth.workload(name)


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
    monkeypatch.setattr(bench, "mfma_file", lambda workload="block_stack": str(tmp_path / "m.json"))
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


def test_ingest_mfma_clock_from_gpu_active_cycles(tmp_path, monkeypatch):
    """The clock of a kernel: GRBM_GUI_ACTIVE (summed over the XCDs the agent
    table names) per XCD over the dispatches' duration; none for kernels of
    under 100 us on average, or without the agent table."""
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    long_k = "void puro::gemm_bs_kernel<0, 0>(int)"
    short_k = "void puro::quant_block_kernel<true, true, false, false>(int)"
    rows = []
    for d, (name, ns) in enumerate([(long_k, 200_000), (long_k, 400_000), (short_k, 20_000)], 1):
        rows += [(d, name, "MfmaUtil", 10.0, ns), (d, name, "GRBM_GUI_ACTIVE", 8 * 2.0 * ns, ns)]
    pc = tmp_path / "bench_counter_collection.csv"
    pc.write_text(head + "".join(f'{d},"{n}",{c},{v},0,{ns}\n' for d, n, c, v, ns in rows))
    monkeypatch.setattr(bench, "mfma_file", lambda workload="block_stack": str(tmp_path / "m.json"))
    bench.ingest_mfma(str(pc))
    assert bench.sclk_for(long_k.split("(")[0]) is None          # no agent table: no XCD count
    (tmp_path / "bench_agent_info.csv").write_text("Name,Num_Xcc\ngfx950,8\n")
    bench.ingest_mfma(str(pc))
    assert bench.sclk_for(long_k.split("(")[0]) == 2.0
    assert bench.sclk_for(short_k.split("(")[0]) is None


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
    monkeypatch.setattr(bench, "traffic_file", lambda workload="block_stack": str(tmp_path / "t.json"))
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


def test_dominant_class_is_the_one_with_most_time():
    """The roofline's kernel: the class with the most total time over the
    warm-up's bracketed launches (several launches of one class add up)."""
    t = [("gemm_fwd_bf16", 0.5), ("gemm_dgrad_w_bf16", 0.9), ("gemm_fwd_bf16", 0.5),
         ("gemm_wgrad_fp32", 0.95)]
    assert bench.dominant_class(t) == "gemm_fwd_bf16"
    assert bench.dominant_class(t[1:2] + t[3:]) == "gemm_wgrad_fp32"
    assert bench.dominant_class([]) is None
    for c in ("gemm_fwd_bf16", "gemm_fwd_t_bf16", "gemm_dgrad_w_bf16", "gemm_wgrad_fp32",
              "gemm_wgrad_splitk"):
        assert c in bench.KERNEL_SYMBOLS


def test_vendor_fp8_leg_is_omitted_without_fp8_support():
    """A torch build without an FP8 dtype or _scaled_mm gives no context leg
    (None) rather than an error, so the bench line is still printed."""
    assert bench.fp8_tensorwise_reference(types.SimpleNamespace(), None, [], 1) is None
    no_mm = types.SimpleNamespace(float8_e4m3fn=object())
    assert bench.fp8_tensorwise_reference(no_mm, None, [], 1) is None
