"""Host-side pieces of bench.py that run without a GPU."""

import csv
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _counter_csv(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_traffic_scaled_by_copy_kernel(tmp_path, monkeypatch):
    bench = _load_bench()
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    mib = 64
    copy_kib = mib * 1024
    # the copy reads half its bytes on FETCH_SIZE (factor 2) and all of them on WRITE_SIZE (factor 1);
    # a fill kernel in the same run must be ignored
    _counter_csv(tmp_path / "cf", [[1, "fill_kernel", "FETCH_SIZE", 5.0],
                                   [2, "elementwise<neg_kernel_cuda>", "FETCH_SIZE", copy_kib / 2]])
    _counter_csv(tmp_path / "cw", [[1, "fill_kernel", "WRITE_SIZE", copy_kib],
                                   [2, "elementwise<neg_kernel_cuda>", "WRITE_SIZE", copy_kib]])
    # two attention dispatches; the first reports its counter in two instances that add up
    _counter_csv(tmp_path / "f", [[7, "attnring::fwd_bf16_kernel<8>", "FETCH_SIZE", 60.0],
                                  [7, "attnring::fwd_bf16_kernel<8>", "FETCH_SIZE", 40.0],
                                  [9, "attnring::fwd_bf16_kernel<8>", "FETCH_SIZE", 300.0],
                                  [8, "merge_kernel", "FETCH_SIZE", 1e6]])
    _counter_csv(tmp_path / "w", [[7, "attnring::fwd_bf16_kernel<8>", "WRITE_SIZE", 10.0],
                                  [9, "attnring::fwd_bf16_kernel<8>", "WRITE_SIZE", 30.0]])
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                        str(tmp_path / "cw"), workload="ring_64k_rank7", copy_mib=mib)
    rec = json.loads(out.read_text())
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 200.0 * 1024 * 2
    assert rec["write_bytes_per_launch"] == 20.0 * 1024
    assert rec["bytes_per_launch"] == 200.0 * 1024 * 2 + 20.0 * 1024
    assert rec["launches"] == [2, 2]
    assert rec["kernel_source_sha"] == bench.kernel_source_hash()


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "--gpus 2 is not supported" in proc.stderr
