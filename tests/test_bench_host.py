"""Host logic of bench.py that needs no GPU: the traffic summary read from
rocprofv3 counter CSVs, and the refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        for i, (name, grid, val) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": "Agent 1",
                        "Queue_Id": 1, "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid,
                        "Kernel_Id": 1, "Kernel_Name": name, "Workgroup_Size": 256,
                        "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 64,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 32, "Counter_Name": counter,
                        "Counter_Value": val, "Start_Timestamp": 0, "End_Timestamp": 1})


def test_traffic_counts_the_ffn_dispatches_only(tmp_path):
    """Copies calibrate the counter (512 MiB read as 256 MiB of FETCH_SIZE =>
    factor 2; a small copy is not a calibration copy); the per-call figure is
    the mean over dispatches of each FFN kernel, summed over the kernels;
    other kernels are ignored."""
    copy = "__amd_rocclr_copyBuffer"
    g1 = "void moe::ffn_decode_kernel<1, 1, 2>(moe::FfnArgs)"
    g2 = "void moe::ffn_decode_kernel<2, 2, 2>(moe::FfnArgs)"
    small = [(copy, 4096, 10.0)]
    cal = [(copy, 1 << 20, 262144.0)] * 3
    fetch = small + cal + [(g1, 1096, 130.0), (g1, 1096, 134.0), (g2, 500, 60.0),
                           (g2, 500, 62.0),
                           ("void moe::route_permute_kernel<5>(moe::FusedRouteArgs)", 72, 9.0)]
    write = small + [(copy, 1 << 20, 524288.0)] * 3 + [(g1, 1096, 2.0), (g2, 500, 4.0)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _csv(fp, "FETCH_SIZE", fetch)
    _csv(wp, "WRITE_SIZE", write)
    res = bench.traffic_from_csv(str(fp), str(wp), 512)
    f, w = res["fetch"], res["write"]
    assert f["bytes_per_counter_byte"] == pytest.approx(2.0)
    assert w["bytes_per_counter_byte"] == pytest.approx(1.0)
    assert f["ffn_kib_per_call"] == pytest.approx(132.0 + 61.0)
    assert w["ffn_kib_per_call"] == pytest.approx(2.0 + 4.0)
    assert f["dispatches"] == {g1: 2, g2: 2}
    assert res["traffic_bytes_per_call"] == pytest.approx((193.0 * 2 + 6.0) * 1024)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
