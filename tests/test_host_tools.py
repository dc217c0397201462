"""Host-side tooling (no GPU): the rocprofv3 summaries behind the committed
profiles, on small synthetic CSVs of the rocprofv3 layout, and bench.py's
refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

from audio_encoder_tower_amd import rocprof_summary as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
K = "void aenc::gemm_bf16_256_kernel<2, false>(aenc::GemmArgs)"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_trace_labels_dispatches_of_one_kernel_in_turn(tmp_path):
    # four dispatches of the same kernel and grid: 1, 2, 3, 4 ms, labelled a, b, a, b
    rows = [{"Dispatch_Id": i + 1, "Kernel_Name": K, "Grid_Size": 241664,
             "Start_Timestamp": 0, "End_Timestamp": int((i + 1) * 1e6)} for i in range(4)]
    rows.append({"Dispatch_Id": 5, "Kernel_Name": "void aenc::layernorm_kernel<unsigned short, false>(float const*)",
                 "Grid_Size": 1539840, "Start_Timestamp": 0, "End_Timestamp": int(0.5e6)})
    _write(str(tmp_path / "run" / "x_kernel_trace.csv"), rows)
    out = rs.trace(str(tmp_path), {"gemm_bf16_256_kernel<2, false>": ["a", "b"]})
    lines = {l.split(" | ")[0].lstrip("| "): l for l in out.splitlines()[2:]}
    a = lines["gemm_bf16_256_kernel<2, false> [a]"].split(" | ")
    b = lines["gemm_bf16_256_kernel<2, false> [b]"].split(" | ")
    # columns: kernel, grid, calls, avg, min, max, share
    assert a[2] == "2" and float(a[3]) == pytest.approx(2.0) and float(a[4]) == 1.0 and float(a[5]) == 3.0
    assert b[2] == "2" and float(b[3]) == pytest.approx(3.0)
    assert float(b[6].rstrip("% |")) == pytest.approx(100 * 6 / 10.5, abs=0.05)
    assert "layernorm_kernel<unsigned short, false>" in lines


def test_counters_derived_columns(tmp_path):
    # one dispatch of 1 ms: GRBM_GUI_ACTIVE over 8 XCDs = 2e6 cycles each -> 2.00 GHz;
    # MFMA busy = 1.024e9 / (2e6 x 1024 SIMDs) = 0.5; CU busy = 2.56e8 / (2e6 x 256) = 0.5
    base = {"Dispatch_Id": 7, "Kernel_Name": K, "Grid_Size": 241664, "Start_Timestamp": 1000,
            "End_Timestamp": 1000 + int(1e6)}
    rows = [dict(base, Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=8 * 2e6),
            dict(base, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=1.024e9),
            dict(base, Counter_Name="SQ_BUSY_CU_CYCLES", Counter_Value=2.56e8)]
    _write(str(tmp_path / "run" / "x_counter_collection.csv"), rows)
    out = rs.counters(str(tmp_path))
    head = [c.strip() for c in out.splitlines()[0].strip("|").split("|")]
    row = [c.strip() for c in out.splitlines()[2].strip("|").split("|")]
    got = dict(zip(head, row))
    assert got["clock GHz"] == "2.00" and got["MFMA busy"] == "0.500" and got["CU busy"] == "0.500"
    assert got["dispatches"] == "1" and float(got["avg ms (profiled)"]) == pytest.approx(1.0)


def test_traffic_scales_by_the_copy_kernel(tmp_path):
    # the copy kernel moved 64 MiB each way but the counters read 0.5x (fetch) and 2x (write)
    def run(d, counter, copy_kib, step_kib):
        rows = [{"Dispatch_Id": 1, "Kernel_Name": "void aenc::copy_kernel(unsigned int*)", "Grid_Size": 65536,
                 "Counter_Name": counter, "Counter_Value": copy_kib},
                {"Dispatch_Id": 2, "Kernel_Name": K, "Grid_Size": 241664, "Counter_Name": counter,
                 "Counter_Value": step_kib}]
        _write(str(tmp_path / d / "x_counter_collection.csv"), rows)
    run("f", "FETCH_SIZE", 0.5 * 64 * 1024, 1000.0)
    run("w", "WRITE_SIZE", 2.0 * 64 * 1024, 300.0)
    out = json.loads(rs.traffic(str(tmp_path / "f"), str(tmp_path / "w"), 64,
                                {"fc2": ("gemm_bf16_256_kernel<2, false>", 241664)}))
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(0.5)
    k = out["kernels"]["fc2"]
    assert k["fetch_bytes"] == 2000 * 1024 and k["write_bytes"] == 150 * 1024
    assert k["bytes_per_launch"] == 2150 * 1024 and len(k["source_digest"]) == 16


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr and res.stdout == ""
