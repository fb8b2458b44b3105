"""Host logic of bench.py (no GPU): the rocprofv3 summary (kernel statistics, per-workload
kernel time from ROCTx ranges, counter figures and calibrated traffic), the roofline
objects, and the reading of committed summaries."""

import csv
import os

import pytest

import bench


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


KT = ["Kind", "Agent_Id", "Queue_Id", "Kernel_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp",
      "End_Timestamp", "Grid_Size"]
GEMM = "void bitmm::(anonymous namespace)::gather_qmm_kernel<4>(bitmm::GatherParams)"
PREP = "bitmm::(anonymous namespace)::gather_prepare_kernel(int const*, int, int, unsigned int*)"
OTHER = "void at::native::vectorized_elementwise_kernel<4>(int)"


def test_trace_summary_per_workload(tmp_path):
    rows = []
    t = 1000
    # two launches of (prepare 5 us, gemm 55 us) inside the range, one outside it
    for i in range(3):
        rows.append(["KERNEL_DISPATCH", 1, 1, 1, PREP, i, t, t + 5000, 1024])
        rows.append(["KERNEL_DISPATCH", 1, 1, 2, GEMM, i, t + 6000, t + 61000, 3072])
        t += 100000
    rows.append(["KERNEL_DISPATCH", 1, 1, 3, OTHER, 9, 50, 60, 64])
    _write(str(tmp_path / "host" / "1_kernel_trace.csv"), KT, rows)
    _write(str(tmp_path / "host" / "1_marker_api_trace.csv"),
           ["Domain", "Function", "Message", "Start_Timestamp", "End_Timestamp"],
           [["MARKER_CORE_API", "roctxRangePushA", "bitmm:gather_up", 900, 200000 + 900]])
    bj = tmp_path / "bench.json"
    bj.write_text('noise\n{"suite": [{"workload": "gather_up", "us_per_launch": 64.0}]}\n')
    text = bench.summarize_profile(str(tmp_path), str(bj), "rocprofv3 --kernel-trace -- python3 bench.py")
    kv = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    assert kv["kernel_sources_sha256_16"] == bench.kernel_sources_hash()
    assert kv["wl.gather_up.launches"] == "2"
    assert float(kv["wl.gather_up.kernel_us_per_launch"]) == pytest.approx(60.0)
    assert float(kv["wl.gather_up.kernel_share_of_untraced_pct"]) == pytest.approx(93.75, abs=0.1)
    assert "# command" in text and "bench.py" in text


CC = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
      "Kernel_Id", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value"]


def test_counter_summary_calibration_and_derived(tmp_path):
    copy = bench.COPY_KERNEL + "(void*)"
    fetch_rows, write_rows, sq_rows = [], [], []
    for d in range(5):   # calibration copies of 256 MiB, first in the run: FETCH reads half, WRITE all
        fetch_rows.append([d, d, 1, 1, 1, 1, 131072, 7, copy, 256, "FETCH_SIZE", 131072.0])
        write_rows.append([d, d, 1, 1, 1, 1, 131072, 7, copy, 256, "WRITE_SIZE", 262144.0])
    fetch_rows.append([5, 5, 1, 1, 1, 1, 131072, 7, copy, 256, "FETCH_SIZE", 3.0])  # a later, smaller copy
    for d in range(10, 14):
        fetch_rows.append([d, d, 1, 1, 1, 1, 3072, 2, GEMM, 256, "FETCH_SIZE", 1000.0])
        fetch_rows.append([d + 10, d + 10, 1, 1, 1, 1, 1024, 3, PREP, 1024, "FETCH_SIZE", 10.0])
        write_rows.append([d, d, 1, 1, 1, 1, 3072, 2, GEMM, 256, "WRITE_SIZE", 300.0])
        write_rows.append([d + 10, d + 10, 1, 1, 1, 1, 1024, 3, PREP, 1024, "WRITE_SIZE", 1.0])
        sq_rows.append([d, d, 1, 1, 1, 1, 3072, 2, GEMM, 256, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0])
        sq_rows.append([d, d, 1, 1, 1, 1, 3072, 2, GEMM, 256, "GRBM_GUI_ACTIVE", 2000.0 * bench.XCD_NUM])
        sq_rows.append([d, d, 1, 1, 1, 1, 3072, 2, GEMM, 256, "SQ_ACTIVE_INST_VALU", 256000.0])
        sq_rows.append([d + 10, d + 10, 1, 1, 1, 1, 1024, 3, PREP, 1024, "GRBM_GUI_ACTIVE", 100.0 * bench.XCD_NUM])
    # the passes come from separate runs whose dispatch ids collide
    _write(str(tmp_path / "fetch" / "h" / "1_counter_collection.csv"), CC, fetch_rows)
    _write(str(tmp_path / "write" / "h" / "2_counter_collection.csv"), CC, write_rows)
    _write(str(tmp_path / "sq" / "h" / "3_counter_collection.csv"), CC, sq_rows)
    text = bench.summarize_profile(str(tmp_path), None, None, algorithmic_bytes=2048 * 1024)
    kv = {k.strip(): v.strip() for k, v in
          (line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith("#"))}
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    # (1000 + 10) KiB * 2 + (300 + 1) KiB * 1 per call
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx((2020 + 301) * 1024)
    assert float(kv["traffic_over_algorithmic"]) == pytest.approx((2020 + 301) / 2048, rel=1e-4)
    # the longest kernel's figures: 512000 / (2000 * 1024 SIMDs) and 256000 / 256 CUs / 2000
    assert float(kv["MfmaUtil_pct"]) == pytest.approx(25.0)
    assert float(kv["VALUBusy_pct"]) == pytest.approx(50.0)


def test_roofline_objects():
    r = bench.roofline_obj("hbm", 40_000_000, 1, 10e-6, {"read_GB_s": {"41943040": 5000.0, "1073741824": 7000.0}})
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(0.5)
    assert r["measured_read_GB_s_at"]["bytes"] == 41943040 and r["frac_of_measured"] == pytest.approx(0.8)
    m = bench.roofline_obj("mfma", 1, 85e9, 100e-6, {"mfma_bf16_TFLOP_s": 2000.0})
    assert m["bound"] == "mfma" and m["achieved"] == pytest.approx(850.0) and m["frac"] == pytest.approx(0.34)
    assert m["frac_of_measured"] == pytest.approx(0.425)


def test_suite_names_match_inputs():
    from bit_matmul_amd import inputs as I
    specs = bench.suite_specs(I)
    names = bench.suite_names()
    assert len(specs) == len(names) == len(set(names))
    # the cheap ones are built here; the others are checked by bench.py itself at run time
    for (kind, make, bound), name in zip(specs, names):
        assert bound in ("hbm", "mfma")
        if name.startswith(("qmv_M1", "qmm_M3")):
            assert make().name == name


def test_read_summary_requires_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "x.txt").write_text("# c\nkernel_sources_sha256_16: deadbeef\nfoo: 1.5\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_summary("x", "deadbeef")["foo"] == "1.5"
    assert bench.read_summary("x", "other") is None
    assert bench.read_summary("missing", "deadbeef") is None
