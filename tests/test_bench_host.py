"""Host-side logic of bench.py, on the CPU: the one-GPU contract and the
turning of rocprofv3 CSV output into the traffic figure the bench reports.

The profile summary is fed small hand-written CSV files in rocprofv3's
column layout: a calibration copy whose counters read a known fraction of
its bytes, and two GEMM dispatches, so the scale factors and the scaled
bytes per launch can be checked by hand.
"""

import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

GEMM1 = "_ZN5tpmlp12_GLOBAL__N_114gemm_bf16_mfmaINS0_3CfgILi256ELi256ELi5EEELi0ELb0EDF16bLi0EEEvNS0_10FastParamsE"
GEMM2 = "_ZN5tpmlp12_GLOBAL__N_114gemm_bf16_mfmaINS0_3CfgILi256ELi256ELi5EEELi1ELb0EDF16bLi0EEEvNS0_10FastParamsE"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda(float)>"


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _counter_rows(name, per_kernel):
    # two rows per dispatch (the counter is reported per XCD group and summed)
    rows = []
    for disp, (kernel, value) in enumerate(per_kernel):
        for part in (0.25, 0.75):
            rows.append({"Kernel_Name": kernel, "Dispatch_Id": disp, "Counter_Name": name,
                         "Counter_Value": value * part})
    return rows


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                          "--warmup", "0"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_profile_summary_scales_the_counters(tmp_path, monkeypatch):
    traffic_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic_file))
    calib_read_kib = bench.CALIB_ELEMS * 2 / 1024
    calib_write_kib = bench.CALIB_ELEMS * 4 / 1024
    trace, fetch, write = tmp_path / "trace", tmp_path / "fetch", tmp_path / "write"
    _write_csv(str(trace / "t_kernel_stats.csv"), ["Name", "Calls", "AverageNs"],
               [{"Name": GEMM1, "Calls": 2, "AverageNs": 1500000}, {"Name": GEMM2, "Calls": 2, "AverageNs": 1400000}])
    _write_csv(str(trace / "t_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [{"Kernel_Name": GEMM1, "Start_Timestamp": 0, "End_Timestamp": 1_500_000},
                {"Kernel_Name": GEMM1, "Start_Timestamp": 0, "End_Timestamp": 1_700_000},
                {"Kernel_Name": GEMM2, "Start_Timestamp": 0, "End_Timestamp": 1_400_000}])
    fields = ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    # the counters see a quarter of the copy's reads and half of its writes
    _write_csv(str(fetch / "f_counter_collection.csv"), fields,
               _counter_rows("FETCH_SIZE", [(COPY, calib_read_kib / 4), (GEMM1, 1000.0), (GEMM2, 3000.0)]))
    _write_csv(str(write / "w_counter_collection.csv"), fields,
               _counter_rows("WRITE_SIZE", [(COPY, calib_write_kib / 2), (GEMM1, 500.0), (GEMM2, 100.0)]))
    bench.summarize_profiles(str(trace), str(fetch), str(write), "wl_test", str(tmp_path / "out"), "cmd")

    data = json.loads(traffic_file.read_text())["wl_test"]
    assert abs(data["read_scale"] - 4.0) < 1e-12 and abs(data["write_scale"] - 2.0) < 1e-12
    assert data["gemm1"]["l2_fabric_bytes_per_launch"] == (1000.0 * 4 + 500.0 * 2) * 1024
    assert data["gemm2"]["l2_fabric_bytes_per_launch"] == (3000.0 * 4 + 100.0 * 2) * 1024
    assert data["gemm1"]["kind"] == bench.TRAFFIC_KIND
    md = (tmp_path / "out" / "tpmlp_forward_wl_test.md").read_text()
    assert "| gemm1 | 2 | 1600.0 | 1500.0 | 1700.0 |" in md
    assert "| gemm2 | 1 | 1400.0 | 1400.0 | 1400.0 |" in md

    # the bench reports the figure only while the kernel source is the one profiled
    assert bench._traffic("wl_test", "gemm1", 1.0) == (1000.0 * 4 + 500.0 * 2) * 1024
    full = json.loads(traffic_file.read_text())
    full["wl_test"]["gemm1"]["source_sha256"] = "0" * 64
    traffic_file.write_text(json.dumps(full))
    assert bench._traffic("wl_test", "gemm1", 1.0) is None
    assert bench._traffic("other_workload", "gemm1", 1.0) is None
