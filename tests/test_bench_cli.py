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


def _counter_csv(path, rows):
    path.mkdir()
    with open(path / f"{path.name}_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_traffic_json_calibrates_against_the_copy(tmp_path):
    """Known counter values in, the derived bytes, clock and MFMA busy fraction out."""
    sys.path.insert(0, ROOT)
    import bench
    dense, copy = "void wf::wf_dense_fwd<128, 0>(unsigned short const*)", "__amd_rocclr_copyBuffer"
    (tmp_path / "kt").mkdir()
    with open(tmp_path / "kt" / "kt_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([dense, 2, 80e6, 40e6, 99.0, 40e6, 40e6, 0])
    # the 1 GiB copy reads as half its bytes fetched and all of them written: scales 2 and 1
    _counter_csv(tmp_path / "FETCH_SIZE", [[copy, "FETCH_SIZE", 524288], [dense, "FETCH_SIZE", 1e6],
                                           [dense, "FETCH_SIZE", 1e6]])
    _counter_csv(tmp_path / "WRITE_SIZE", [[copy, "WRITE_SIZE", 1048576], [dense, "WRITE_SIZE", 5e5]])
    # 2 GHz over a 40 ms launch on 8 XCDs; the matrix pipe busy half of the cycles on 1,024 SIMDs
    _counter_csv(tmp_path / "sq1", [[dense, "GRBM_GUI_ACTIVE", 8 * 2e9 * 0.04],
                                    [dense, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * 2e9 * 0.04]])
    out = bench.write_traffic(str(tmp_path), str(tmp_path / "traffic.json"))
    assert out["calibration"]["fetch_scale"] == 2.0 and out["calibration"]["write_scale"] == 1.0
    assert out["bytes_per_launch"] == 1e6 * 1024 * 2 + 5e5 * 1024
    assert out["clock_ghz"] == 2.0 and out["mfma_busy"] == 0.5
    assert json.load(open(tmp_path / "traffic.json")) == out


def test_reported_vsa_flops_follow_the_page_convention():
    """bench.py's fine-stage FLOPs for the page's 78-of-624 operating point give the
    page's roofline figure (padded query tokens left out), printed in tests/golden/."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    golden = json.load(open(os.path.join(ROOT, "tests", "golden", "page4_vsa_480p.json")))
    wl = synth.WORKLOADS["vsa_480p_k78"]
    assert (wl.T, wl.H, wl.W, wl.Hh, wl.D, wl.topk) == (golden["T"], golden["H"], golden["W"], golden["heads"],
                                                        golden["head_dim"], golden["kept_cubes"])
    fl = bench.vsa_flops(wl, golden["cubes"])
    assert round(fl["fine"] / 1e12, 2) == golden["tflop_rounded"]
    # the step's own top-32 figure scales with k
    wl32 = synth.WORKLOADS["vsa_480p"]
    assert bench.vsa_flops(wl32, golden["cubes"])["fine"] * 78 == fl["fine"] * 32


def test_ideal_speedup_is_the_flop_ratio():
    """Dense FLOPs over VSA FLOPs (fine on real queries + coarse scores) at the same shape."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    w480, w720 = synth.WORKLOADS["vsa_480p"], synth.WORKLOADS["vsa_720p"]
    assert abs(bench.ideal_speedup(w480, 624) - 32760 / (64 * 32 + 624 ** 2 / (2 * 32760))) < 1e-9
    assert 15.9 < bench.ideal_speedup(w480, 624) < 16.0
    assert 18.3 < bench.ideal_speedup(w720, 1440) < 18.5
    info = bench.blas_info()
    assert info["threads"] >= 1 and isinstance(info["library"], str)
