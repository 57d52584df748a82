"""Host-side parts of bench.py: the HBM traffic record built from rocprofv3
counter files (no GPU; synthetic counter CSVs in rocprofv3's column layout)."""

import csv
import json
import os

import bench

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
        "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
        "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
        "End_Timestamp"]


def _write(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, COLS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({c: 0 for c in COLS} | {"Dispatch_Id": i + 1, "Kernel_Name": name,
                                               "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_scales_counters_by_the_copy(tmp_path):
    k = f"void pa::(anonymous namespace)::{bench.STEP_KERNEL}(unsigned short const*)"
    other = "void pa::(anonymous namespace)::combine_kernel<128, 16>(unsigned short*)"
    d = [str(tmp_path / n) for n in ("fs", "ws", "fc", "wc")]
    # two step-kernel dispatches (mean 1000 KiB fetched) among other kernels
    _write(d[0], "FETCH_SIZE", [(k, 900.0), (other, 5.0), (k, 1100.0)])
    _write(d[1], "WRITE_SIZE", [(k, 10.0), (k, 30.0), (other, 7.0)])
    # a 1 GiB copy whose FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    _write(d[2], "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 524288.0)])
    _write(d[3], "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1048576.0)])
    out = tmp_path / "traffic.json"
    bench.write_traffic(d, str(out))
    rec = json.load(open(out))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_read_bytes_per_launch"] == 1000 * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == 20 * 1024
    assert rec["hbm_bytes_per_launch"] == 1000 * 1024 * 2 + 20 * 1024
    assert rec["launches"] == 2
    assert rec["kernel"] == bench.STEP_KERNEL
    assert rec["source_sha256_16"] == bench.kernel_source_hash("k_decode.hip")



def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says why."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
