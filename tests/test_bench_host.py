"""Host-side logic of bench.py: the one-GPU guard and the HBM-traffic
summary (counter KiB scaled by what the same counter reads for a copy of
known size)."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path):
    import bench
    copy_kib = bench.COPY_BYTES / 1024.0
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    # FETCH_SIZE reads half the copy's bytes (factor 2), WRITE_SIZE all of them
    # (factor 1); the attention kernel's median over its dispatches is taken
    _write(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_kib / 2)] +
           [("void ca::cascade_phases_kernel<128, 1>(ca::TileArgs)", v) for v in (100.0, 300.0, 200.0)] +
           [("void ca::merge_kernel<128, false, 1>(ca::MergeArgs)", 10.0)])
    _write(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib)] +
           [("void ca::cascade_phases_kernel<128, 1>(ca::TileArgs)", 40.0)] * 3 +
           [("void ca::merge_kernel<128, false, 1>(ca::MergeArgs)", 5.0)])
    rec = bench.summarize_pmc(fetch, write, "worked_decode", 3)
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    k = rec["kernels"]["cascade_phases_kernel"]
    assert k["fetch_kib_raw"] == 200.0
    assert k["fetch_bytes"] == pytest.approx(200.0 * 1024 * 2)
    assert k["write_bytes"] == pytest.approx(40.0 * 1024)
    assert k["hbm_bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2 + 40.0 * 1024)
    m = rec["kernels"]["merge_kernel"]
    assert m["hbm_bytes_per_launch"] == pytest.approx(10.0 * 1024 * 2 + 5.0 * 1024)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    assert fetch in rec["command"] and write in rec["command"]

