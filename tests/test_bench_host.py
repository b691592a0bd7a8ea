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


def test_counter_summary_clock_and_busy(tmp_path, capsys):
    """--counters-from: the clock comes from one XCD's busy clocks over the traced
    duration, MFMA busy from per-SIMD busy cycles over that clock count."""
    bench = _load_bench()
    folder = tmp_path / "ctr"
    dur_ns = 1_000_000                        # 1 ms per dispatch
    clocks = 1.8e6                            # 1.8 GHz on each XCD
    busy_frac = 0.5
    simds = bench.N_CU * bench.SIMD_PER_CU
    vals = {"GRBM_GUI_ACTIVE": clocks * bench.N_XCD, "SQ_VALU_MFMA_BUSY_CYCLES": busy_frac * clocks * simds,
            "SQ_INSTS_MFMA": 1000.0, "SQ_INSTS_VALU": 8500.0, "SQ_INSTS_LDS": 1500.0,
            "SQ_LDS_BANK_CONFLICT": 0.0, "SQ_LDS_IDX_ACTIVE": 0.25 * clocks * bench.N_CU,
            "SQ_WAVES": 16384.0, "SQ_BUSY_CYCLES": 1.0}
    rows = []
    for disp in (3, 4):
        for name, v in vals.items():
            # each counter split over two hardware instances
            rows.append([disp, "attnring::fwd_bf16_kernel<8>", name, v / 2])
            rows.append([disp, "attnring::fwd_bf16_kernel<8>", name, v / 2])
        rows.append([disp + 10, "other_kernel", "GRBM_GUI_ACTIVE", 1e12])
    _counter_csv(folder, rows)
    with open(folder / "ctr_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerow([3, "attnring::fwd_bf16_kernel<8>", 5_000, 5_000 + dur_ns])
        w.writerow([4, "attnring::fwd_bf16_kernel<8>", 9_000_000, 9_000_000 + dur_ns])
        w.writerow([13, "other_kernel", 0, 10])
    bench.summarize_counters(str(folder))
    rec = json.loads(capsys.readouterr().out)
    assert rec["dispatches"] == 2
    assert abs(rec["avg_duration_us"] - 1000.0) < 1e-9
    assert abs(rec["shader_clock_ghz"] - 1.8) < 1e-9
    assert abs(rec["mfma_busy_pct"] - 50.0) < 1e-9
    assert abs(rec["valu_per_mfma"] - 8.5) < 1e-12 and abs(rec["lds_per_mfma"] - 1.5) < 1e-12
    assert abs(rec["lds_active_pct"] - 25.0) < 1e-9 and rec["lds_bank_conflict_pct"] == 0.0


def test_trace_summary_lists_the_warmup_apart(tmp_path, capsys):
    """--trace-from: dispatches in launch order, the first warmup x launches-per-step are the
    warmup; the rest (timed pass and event-timed pass) give the average launch."""
    bench = _load_bench()
    folder = tmp_path / "kt"
    folder.mkdir()
    per_step, warmup, steps = 8, 2, 3     # ring_64k_rank7: 8 active chunks per ring pass
    durs = [2000.0] * (per_step * warmup) + [1000.0, 500.0] * (per_step * steps)  # microseconds
    with open(folder / "kt_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 10_000
        rows = []
        for i, d in enumerate(durs):
            rows.append([i, "attnring::fwd_bf16_kernel<8>", t, t + int(d * 1e3)])
            t += int(d * 1e3) + 50
        for r in reversed(rows):              # file order must not matter: sorted by start
            w.writerow(r)
        w.writerow([999, "other_kernel", 0, 5])
    bench.summarize_trace(str(folder), "ring_64k_rank7", warmup, steps)
    rec = json.loads(capsys.readouterr().out)
    assert rec["launches_per_step"] == per_step
    assert rec["warmup_dispatches"] == per_step * warmup and rec["warmup_avg_us"] == 2000.0
    assert rec["timed_dispatches"] == 2 * per_step * steps and rec["timed_avg_us"] == 750.0
    assert abs(rec["kernel_ms_per_step"] - 6.0) < 1e-12
    flop = 4 * 64 * 64 * (lambda c: sum(range(7 * c + 1, 8 * c + 1)))(8192) / per_step
    assert rec["flop_per_launch"] == flop


class _FakeJob:
    """A job whose steps take `dt` seconds of host time (no GPU)."""

    def __init__(self, dt):
        self.dt, self.steps = dt, 0

    def run(self):
        self.steps += 1
        import time as _t
        _t.sleep(self.dt)


def test_warmup_extends_to_a_minimum_time(monkeypatch):
    bench = _load_bench()
    import types
    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: None))
    monkeypatch.setitem(sys.modules, "torch", fake_torch)
    job = _FakeJob(0.002)
    n = bench.warm_up(job, 5, min_seconds=0.05)
    assert n == job.steps and 5 < n <= 40            # 5 requested, then enough for ~50 ms
    job = _FakeJob(0.002)
    assert bench.warm_up(job, 5) == 5 == job.steps     # no minimum: exactly the requested steps
    job = _FakeJob(0.02)
    assert bench.warm_up(job, 5, min_seconds=0.05) == 5  # already past the minimum
