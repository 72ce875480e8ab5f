"""Host-side checks of the measurement tools: the rocprofv3 summary readers
(on small synthetic CSV files laid out as rocprofv3 writes them) and the
bench's algorithmic work counts and its one-GPU guard."""

import csv
import os
import subprocess
import sys

import pytest

from matrix_aware_optimizer_muon_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

BX = "void muon::ns_gemm_kernel<false, 2, 1, false>(muon::UnitDev const*, muon::GemmTask const*, muon::GemmParams)"
GRAM = "void muon::ns_gemm_kernel<false, 0, 0, false>(muon::UnitDev const*, muon::GemmTask const*, muon::GemmParams)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_kernel_kind_names():
    assert P.kernel_kind(BX) == "bx"
    assert P.kernel_kind(GRAM) == "gram"
    assert P.kernel_kind("void muon::ns_gemm_kernel<true, 1, 0, false>(...)") == "square/f32"
    assert P.kernel_kind("void muon::ns_gemm_kernel<false, 2, 1, true>(...)") == "bx"
    assert P.kernel_kind("_ZN4muon14ns_gemm_kernelILb1ELi2ELi0ELb0EEEvPKNS_7UnitDevE") == "bx/f32"
    assert P.kernel_kind("void muon::momentum_kernel<false>(...)") == "momentum"
    assert P.kernel_kind(COPY) == "copy"
    assert P.kernel_kind("void muon::update_kernel<false>(...)") == "update"
    assert P.kernel_kind("muon::(anonymous namespace)::syrk_update_kernel(double*, double*)") == "syrk_update_kernel"


def test_alone_dispatches():
    # two overlapping launches (two streams), then serial ones
    assert P._alone([(0, 1), (2, 3), (2.5, 4), (5, 6)]) == [True, False, False, True]
    # a long launch overlapping two short ones further on
    assert P._alone([(0, 10), (1, 2), (3, 4), (11, 12)]) == [False, False, False, True]
    assert P._alone([]) == []


def test_trace_table_separates_overlapping_dispatches(tmp_path):
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X",
              "Group_Segment_Size"]
    us = 1000   # timestamps in ns
    rows = [  # a two-stream phase: both launches take 200 us side by side
        {"Kernel_Name": BX, "Start_Timestamp": 0, "End_Timestamp": 200 * us},
        {"Kernel_Name": BX, "Start_Timestamp": 5 * us, "End_Timestamp": 205 * us},
        # the same launches one after the other on one stream: 110 us each
        {"Kernel_Name": BX, "Start_Timestamp": 300 * us, "End_Timestamp": 410 * us},
        {"Kernel_Name": BX, "Start_Timestamp": 420 * us, "End_Timestamp": 530 * us},
        {"Kernel_Name": GRAM, "Start_Timestamp": 540 * us, "End_Timestamp": 600 * us},
    ]
    for r in rows:
        r.update({"Workgroup_Size_X": 512, "Grid_Size_X": 512 * 300, "Group_Segment_Size": 65536})
    _write(str(tmp_path / "run" / "run_kernel_trace.csv"), fields, rows)
    t = P.trace_table(str(tmp_path))
    assert t["bx"]["calls"] == 4 and t["bx"]["alone_calls"] == 2
    assert t["bx"]["avg_us"] == pytest.approx((200 + 200 + 110 + 110) / 4)
    assert t["bx"]["alone_avg_us"] == pytest.approx(110)
    assert t["bx"]["grid"] == 300 and t["bx"]["lds"] == 65536
    assert t["gram"]["alone_avg_us"] == pytest.approx(60)
    md = P.trace_markdown(str(tmp_path), "t", "cmd")
    assert "| bx | 4 |" in md and "alone avg" in md


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]

    def counters(d, name, rows):
        _write(str(tmp_path / d / "run_counter_collection.csv"), fields,
               [{"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": name, "Counter_Value": v}
                for i, k, v in rows])
    # two bx dispatches; counter values of one dispatch come in two instances
    counters("f", "FETCH_SIZE", [(1, BX, 100.0), (1, BX, 100.0), (2, BX, 300.0)])
    counters("w", "WRITE_SIZE", [(1, BX, 50.0), (2, BX, 150.0)])
    # a 1 MiB copy for which FETCH_SIZE reads half the bytes and WRITE_SIZE all
    counters("cf", "FETCH_SIZE", [(1, COPY, 512.0)])
    counters("cw", "WRITE_SIZE", [(1, COPY, 1024.0)])
    d = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                  1 << 20, ["cmd"])
    assert d["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert d["calibration"]["write_scale"] == pytest.approx(1.0)
    assert d["per_launch_read_bytes"]["bx"] == 2 * 250 * 1024      # mean of 200 and 300 KiB, x2
    assert d["per_launch_write_bytes"]["bx"] == 100 * 1024
    assert d["per_launch_bytes"]["bx"] == 600 * 1024
    assert d["kernel_source_hash"] == P.kernel_source_hash()


def test_mfma_table_from_counters(tmp_path):
    _write(str(tmp_path / "run_agent_info.csv"), ["Simd_Count", "Num_Xcc", "Max_Engine_Clk_Fcompute"],
           [{"Simd_Count": 0, "Num_Xcc": 0, "Max_Engine_Clk_Fcompute": 0},      # the CPU agent
            {"Simd_Count": 1024, "Num_Xcc": 8, "Max_Engine_Clk_Fcompute": 2400}])
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    us = 1000
    rows = []
    # two bx dispatches of 100 us: 50 G MFMA flops each, active 2 GHz on
    # each of 8 XCDs, MFMA busy a quarter of the SIMD cycles
    for d, t0 in ((1, 0), (2, 200 * us)):
        for c, v in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 50e9 / 512), ("GRBM_GUI_ACTIVE", 8 * 2e9 * 100e-6),
                     ("SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * 2e9 * 100e-6)):
            rows.append({"Dispatch_Id": d, "Kernel_Name": BX, "Counter_Name": c, "Counter_Value": v,
                         "Start_Timestamp": t0, "End_Timestamp": t0 + 100 * us})
    # a copy does no MFMA work and is left out
    rows.append({"Dispatch_Id": 3, "Kernel_Name": COPY, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "Counter_Value": 0, "Start_Timestamp": 0, "End_Timestamp": 1})
    _write(str(tmp_path / "run_counter_collection.csv"), fields, rows)
    t = P.mfma_table(str(tmp_path), 2500.0)
    assert set(t) == {"bx"}
    e = t["bx"]
    assert e["dispatches"] == 2 and e["gflop"] == pytest.approx(50.0) and e["avg_us"] == pytest.approx(100.0)
    assert e["tflops"] == pytest.approx(500.0) and e["frac"] == pytest.approx(0.2)
    assert e["busy_pct"] == pytest.approx(25.0)
    assert "| bx | 2 | 50.00 | 100.0 | 500 | 20.0 | 25.0 |" in P.mfma_markdown(str(tmp_path), "t", "cmd", 2500.0)


def test_step_windows_busy_share_and_queue_gaps(tmp_path):
    d = tmp_path / "trace"
    mom = "void muon::momentum_kernel<false>(muon::UnitDev const*, muon::EwTask const*, muon::K1Params)"
    fields = ["Kernel_Name", "Queue_Id", "Start_Timestamp", "End_Timestamp"]
    # step 1: two lanes on two queues, back to back; step 2: one queue with a
    # 10 us gap between its two launches and a 5 us gap before the next lane
    ev = [(mom, 1, 0, 100), (mom, 2, 0, 100), (BX, 1, 100, 300), (GRAM, 2, 100, 300),
          (mom, 1, 1000, 1100), (BX, 1, 1110, 1300), (mom, 1, 1305, 1400), (GRAM, 1, 1400, 2000)]
    rows = [{"Kernel_Name": k, "Queue_Id": q, "Start_Timestamp": a * 1000, "End_Timestamp": b * 1000}
            for k, q, a, b in ev]
    _write(str(d / "run_kernel_trace.csv"), fields, rows)
    st = P.step_windows(str(d))
    assert len(st) == 2
    assert st[0]["queues"] == 2 and st[0]["dispatches"] == 4
    assert abs(st[0]["us"] - 1000.0) < 1e-9 and abs(st[0]["busy_us"] - 300.0) < 1e-9
    assert st[0]["queue_gap_us"] == {"1": 700.0, "2": 0.0}
    assert st[1]["queues"] == 1 and st[1]["dispatches"] == 4
    assert abs(st[1]["busy_us"] - 985.0) < 1e-9 and st[1]["queue_gap_us"] == {"1": 15.0}


def test_lds_table_shares(tmp_path):
    d = tmp_path / "lds"
    _write(str(d / "run_agent_info.csv"), ["Simd_Count", "Num_Xcc", "Max_Engine_Clk_Fcompute"],
           [{"Simd_Count": 1024, "Num_Xcc": 8, "Max_Engine_Clk_Fcompute": 2400}])
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    vals = {"SQ_LDS_IDX_ACTIVE": 2560.0, "SQ_LDS_BANK_CONFLICT": 256.0, "SQ_INSTS_LDS": 300.0,
            "SQ_INSTS_MFMA": 200.0, "SQ_WAIT_INST_LDS": 30.0, "SQ_WAIT_INST_ANY": 250.0, "SQ_WAVE_CYCLES": 1000.0,
            "GRBM_GUI_ACTIVE": 800.0}
    rows = [{"Dispatch_Id": 1, "Kernel_Name": BX, "Counter_Name": c, "Counter_Value": v,
             "Start_Timestamp": 0, "End_Timestamp": 5000} for c, v in vals.items()]
    _write(str(d / "run_counter_collection.csv"), fields, rows)
    e = P.lds_table(str(d))["bx"]
    # 2560 LDS cycles over 256 CUs x (800 / 8) cycles: 10 %
    assert abs(e["lds_busy_pct"] - 10.0) < 1e-9 and abs(e["conflict_pct"] - 10.0) < 1e-9
    assert abs(e["lds_per_mfma"] - 1.5) < 1e-12 and abs(e["wait_lds_pct"] - 3.0) < 1e-9
    assert abs(e["wait_any_pct"] - 25.0) < 1e-9 and abs(e["avg_us"] - 5.0) < 1e-9


def test_marker_table_counts_and_means(tmp_path):
    d = tmp_path / "markers"
    fields = ["Domain", "Function", "Process_Id", "Thread_Id", "Correlation_Id", "Start_Timestamp", "End_Timestamp"]
    rows = [{"Domain": "MARKER_CORE_RANGE_API", "Function": n, "Process_Id": 1, "Thread_Id": 1,
             "Correlation_Id": i, "Start_Timestamp": t0, "End_Timestamp": t0 + dur}
            for i, (n, t0, dur) in enumerate([("muon.step", 0, 9000), ("muon.gram", 10, 2000),
                                              ("muon.gram", 5000, 4000), ("muon.bx", 9000, 1500)])]
    _write(str(d / "run_marker_api_trace.csv"), fields, rows)
    text = P.markers_markdown(str(d), "roctx", ["cmd"])
    lines = [l for l in text.splitlines() if l.startswith("| `")]
    # largest total first; means in microseconds (timestamps in ns)
    assert lines == ["| `muon.step` | 1 | 9.0 |", "| `muon.gram` | 2 | 3.0 |", "| `muon.bx` | 1 | 1.5 |"]


def test_blas_table_from_bench_lines(tmp_path):
    import json
    line = {"gpu_clock_mhz": 2000, "blas_context": {
        "library": "torch.bmm bf16", "shapes": 1,
        "gram": {"vendor_ms": 0.2, "vendor_tflops": 500.0, "vendor_frac_bf16_peak": 0.2, "library_ms": 0.1},
        "square": {"vendor_ms": 0.1, "vendor_tflops": 400.0, "vendor_frac_bf16_peak": 0.16, "library_ms": 0.1},
        "bx": {"vendor_ms": 0.3, "vendor_tflops": 600.0, "vendor_frac_bf16_peak": 0.24, "library_ms": 0.4}}}
    f = tmp_path / "blas_square.json"
    f.write_text("warning text\n" + json.dumps(line) + "\n")
    text = P.blas_markdown([str(f)], ["cmd"])
    rows = [l for l in text.splitlines() if l.startswith("| one 4096x4096")]
    assert [r.split(" | ")[1] for r in rows] == ["gram", "square", "bx"]
    assert rows[0].endswith("| 2.00 |") and rows[2].endswith("| 0.75 |")
    assert "square 2000" in text and P.kernel_source_hash() in text


def test_bench_work_counts():
    # symmetric products: Gram m(m+1)n, square m^2(m+1), update 2m^2n
    f = bench.ns_flops(768, 3072)
    assert f == {"gram": 768 * 769 * 3072, "square": 768 * 768 * 769, "bx": 2 * 768 * 768 * 3072}
    m, n = 256, 512
    # one iteration: B X reads B, X hi and its int8 correction, and reads and
    # writes the weight; no X master is written
    b1 = bench.ns_bytes(m, n, 2, 2, 1)
    assert b1["bx"] == 2 * m * m + 3 * m * n + 4 * m * n
    assert b1["gram"] == 2 * m * n + 2 * m * m and b1["square"] == 4 * m * m
    # five iterations: four write the 3-byte master, the last the weight
    b5 = bench.ns_bytes(m, n, 2, 2, 5)
    assert b5["bx"] == pytest.approx((4 * (2 * m * m + 6 * m * n) + b1["bx"]) / 5)
    # float32 NS: X is one float, no correction
    b = bench.ns_bytes(m, n, 4, 4, 1)
    assert b["bx"] == 4 * m * m + 4 * m * n + 8 * m * n


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "one GPU" in r.stderr
