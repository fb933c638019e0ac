"""Host-side checks of bench.py's contract logic (no GPU): the one-GPU guard, the source-hash
gate on the roofline's traffic figure, and the counter calibration that turns rocprofv3's
FETCH_SIZE / WRITE_SIZE into HBM bytes."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (bench.py imports torch only inside main)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    path = tmp_path / "hbm_traffic.json"
    path.write_text(json.dumps({"kernels": {"gemm_i8_prefill": {"source_hash": "abc", "bytes_per_launch": 123.0}}}))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    assert bench.traffic_from_profiles("gemm_i8_prefill", "abc") == 123.0
    assert bench.traffic_from_profiles("gemm_i8_prefill", "abd") is None      # kernel changed since
    assert bench.traffic_from_profiles("rotate_quant_prefill", "abc") is None
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "missing.json"))
    assert bench.traffic_from_profiles("gemm_i8_prefill", "abc") is None


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_calibrates_against_the_copy(tmp_path, monkeypatch, capsys):
    gemm = "void convrot::(anonymous namespace)::gemm_i8_kernel<(convrot::Epi)0, true>(GemmParams)"
    rq = "void convrot::rotate_quant_kernel<false, 8, 1, 8>(convrot::RQParams)"
    copy = "__amd_rocclr_copyBuffer"
    kib = bench.COPY_PROBE_BYTES / 1024
    f, w, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    # per-dispatch medians: gemm 271000 KiB fetched, 131000 written; the copy's counters read half
    # its size for FETCH_SIZE and all of it for WRITE_SIZE
    _counter_csv(f, [(gemm, "FETCH_SIZE", 270000), (gemm, "FETCH_SIZE", 272000), (gemm, "FETCH_SIZE", 271000),
                     (rq, "FETCH_SIZE", 21500)])
    _counter_csv(w, [(gemm, "WRITE_SIZE", 131000), (rq, "WRITE_SIZE", 21550)])
    _counter_csv(cf, [(copy, "FETCH_SIZE", kib / 2)])
    _counter_csv(cw, [(copy, "WRITE_SIZE", kib)])
    out_path = tmp_path / "profiles" / "hbm_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out_path))
    bench.pmc_summary(f, w, cf, cw)
    capsys.readouterr()
    d = json.loads(out_path.read_text())
    assert d["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert d["calibration"]["write_factor"] == pytest.approx(1.0)
    g = d["kernels"]["gemm_i8_prefill"]
    assert g["fetch_kib_raw"] == 271000 and g["write_kib_raw"] == 131000
    assert g["fetch_bytes"] == pytest.approx(271000 * 1024 * 2.0)
    assert g["write_bytes"] == pytest.approx(131000 * 1024)
    assert g["bytes_per_launch"] == pytest.approx(g["fetch_bytes"] + g["write_bytes"])
    assert g["source_hash"] == bench.src_hash("gemm_i8.hip")
    assert d["kernels"]["rotate_quant_prefill"]["source_hash"] == bench.src_hash("rotate_quant.hip")
    assert "copy" not in d["kernels"]


def test_counter_table_means_and_derived_rows(tmp_path, capsys):
    gemm = "void convrot::(anonymous namespace)::gemm_i8_kernel<(convrot::Epi)0, true>(convrot::(anonymous namespace)::GemmParams)"
    torch_kernel = "void at::native::vectorized_elementwise_kernel<4>(int)"
    a, b = str(tmp_path / "a.csv"), str(tmp_path / "b.csv")
    _counter_csv(a, [(gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 300.0), (gemm, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0),
                     (gemm, "GRBM_GUI_ACTIVE", 8 * 800.0), (gemm, "GRBM_GUI_ACTIVE", 8 * 800.0),
                     (torch_kernel, "GRBM_GUI_ACTIVE", 5.0)])
    _counter_csv(b, [(gemm, "TCC_HIT_sum", 30.0), (gemm, "TCC_MISS_sum", 10.0)])
    bench.counter_table([a, b])
    out = capsys.readouterr().out
    assert "`gemm_i8_kernel<(Epi)0, true>`" in out and "vectorized_elementwise" not in out
    rows = {ln.split("|")[1].strip(): ln.split("|")[2].strip() for ln in out.splitlines() if ln.startswith("| ")}
    assert rows["dispatches"] == "2"
    assert float(rows["SQ_VALU_MFMA_BUSY_CYCLES"]) == pytest.approx(1024 * 400.0, rel=1e-3)
    assert float(rows["*MFMA-busy fraction*"]) == pytest.approx(0.5)
    assert float(rows["*L2 hit rate*"]) == pytest.approx(0.75)


def test_trace_table_groups_by_kernel_and_launch_shape(tmp_path, capsys):
    path = tmp_path / "kernel_trace.csv"
    gemm = "void convrot::(anonymous namespace)::gemm_i8_kernel<(convrot::Epi)0, true>(convrot::(anonymous namespace)::GemmParams)"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Workgroup_Size", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, (dur, grid) in enumerate([(300000, 131072), (310000, 131072), (20000, 4096)]):
            w.writerow({"Kernel_Name": gemm, "Grid_Size": grid, "Workgroup_Size": 512,
                        "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + dur})
    bench.trace_table(str(path))
    out = capsys.readouterr().out
    assert "| `gemm_i8_kernel<(Epi)0, true>` | 3 | 210.00 | 300.00 | 20.00 | 310.00 |" in out
    assert "| `gemm_i8_kernel<(Epi)0, true>` | 131072 | 512 | 2 | 305.00 |" in out
