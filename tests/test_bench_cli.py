"""bench.py's command-line contract that needs no GPU: the one-GPU rule and the
rocprofv3 CSV summariser."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "--gpus must be 1" in line["error"]


def test_summarize_reads_rocprof_csv(tmp_path):
    kt = tmp_path / "kt"
    kt.mkdir()
    with open(kt / "kt_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void wf::wf_dense_fwd<128>(unsigned short const*)", 4, 148e6, 37e6, 92.5, 36e6, 39e6, 1e6])
    fs = tmp_path / "FETCH_SIZE"
    fs.mkdir()
    with open(fs / "FETCH_SIZE_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for val in (100.0, 300.0):
            w.writerow(["void wf::wf_dense_fwd<128>(unsigned short const*)", "FETCH_SIZE", val])
    r = run_bench("--summarize", str(tmp_path))
    assert r.returncode == 0, r.stderr
    assert "37.0000" in r.stdout and "36.0000" in r.stdout and "39.0000" in r.stdout
    assert "FETCH_SIZE=200" in r.stdout and "n=2" in r.stdout
