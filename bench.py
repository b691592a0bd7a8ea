"""Throughput of one device's share of ring-attention prefill on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for the ring workloads, the device's N ring steps (attention of its query
chunk against every key/value chunk, fully masked chunks skipped) and the LSE
merges; for the prefill workload, one full causal attention call.  Inputs
are resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` is algorithmic TFLOP/s: 4 * head_dim * Hq
flops per causal (query, key) pair (2*d for the score, 2*d for the weighted
sum of values); masked work and softmax arithmetic are not counted.

    python bench.py [--gpus 1] [--steps 50] [--warmup 100] [--workload ring_64k_rank7]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal GQA prefill attention TFLOP/s & % bf16 peak at 32K/64K/100K, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak (2.5 PFLOP/s)
DOMINANT_KERNEL = "fwd_bf16_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16.json")
KERNEL_SOURCES = ["fwd_bf16.hip", "kernels.h", "merge_math.h"]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="ring_64k_rank7")
    ap.add_argument("--extra", default="ring_32k_rank3,prefill_100k,ring_100k_n16_rank15,ring_100k_n16,"
                    "varlen_ulysses_rank7,chunked_prefill_12k,ring_64k_zigzag_rank7",
                    help="comma list of further workloads measured in the same run ('' for none)")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--extra-warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache passes (for profiled runs: only warmup and timed steps launch)")
    ap.add_argument("--trace-from", metavar="FOLDER",
                    help="only summarize the attention kernel's durations in a rocprofv3 --kernel-trace run of "
                         "this script with the same --workload/--warmup/--steps and --extra ''")
    ap.add_argument("--unfused", action="store_true",
                    help="merge each ring step with the separate merge kernel instead of in the step")
    ap.add_argument("--cpu-rows", type=int, default=768,
                    help="query rows of the oracle sample (all heads, all ring steps)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (for counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only derive HBM bytes per attention launch from four rocprofv3 --pmc output "
                         "folders (FETCH_SIZE and WRITE_SIZE of a bench run, then of --calibrate-copy) "
                         "and write them to " + os.path.relpath(TRAFFIC_FILE, ROOT))
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only measure the sustained rate of a large library bf16 GEMM on random data "
                         "(the practical matrix-core ceiling under the board's power limit)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the sustained rate of back-to-back bf16 MFMAs on constant and on "
                         "random operands (the probe library built beside the attention library)")
    ap.add_argument("--mix-ceiling", action="store_true",
                    help="only measure the sustained matrix-core rate of the attention kernel's inner-loop "
                         "instruction mix on constant and on random operands (the probe library)")
    ap.add_argument("--valu-rates", action="store_true",
                    help="only measure issue rates of the softmax's vector instructions and their overlap "
                         "with the matrix cores (the probe library built beside the attention library)")
    ap.add_argument("--counters-from", metavar="FOLDER",
                    help="only summarize a rocprofv3 --pmc --kernel-trace run of this script "
                         "(MFMA busy, LDS bank conflicts, shader clock) for the attention kernel")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "ring_attention_03_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Job:
    """One workload with its inputs resident on the device and a run() for one step."""

    def __init__(self, name, fused=True):
        import torch

        from ring_attention_03_amd import (ChunkedPrefill, RingAttention, RingLayout, ZigzagLayout,
                                           ZigzagRing)
        from ring_attention_03_amd.workloads import WORKLOADS, make_qkv

        self.w = w = WORKLOADS[name]
        self.name = name
        self.fused = fused
        q, k, v = make_qkv(w)
        self.cpu_inputs = (q, k, v)
        dev = torch.device("cuda:0")
        self.layout = RingLayout(w.seqlens, w.n_chunks)
        self.rank = 0 if w.rank is None else w.rank
        # a ring workload without a rank is the whole ring: every device's share, one after another
        self.sweep = w.mode == "ring" and w.rank is None and w.n_chunks > 1
        lay = self.layout
        if w.n_chunks == 1:
            self.q = q.to(dev)
            self.k, self.v = k.to(dev), v.to(dev)
            self.cu = lay.cu
        elif w.mode == "zigzag":
            zz = ZigzagLayout(w.seqlens, w.n_chunks)
            self.q = zz.gather(q, self.rank).to(dev).contiguous()
            self.chunks = [(zz.gather(k, j).to(dev).contiguous(), zz.gather(v, j).to(dev).contiguous())
                           for j in range(w.n_chunks)]
            self.zigzag = (zz, ZigzagRing(zz, self.rank))
        elif w.mode == "chunked":
            self.q = lay.gather(q, self.rank).to(dev).contiguous()
            self.k = lay.gather_prefix(k, self.rank).to(dev).contiguous()
            self.v = lay.gather_prefix(v, self.rank).to(dev).contiguous()
        elif self.sweep:
            self.chunks = [(lay.gather(k, j).to(dev).contiguous(), lay.gather(v, j).to(dev).contiguous())
                           for j in range(w.n_chunks)]
            self.q_ranks = [lay.gather(q, r).to(dev).contiguous() for r in range(w.n_chunks)]
            self.q = self.q_ranks[-1]
        else:
            self.q = lay.gather(q, self.rank).to(dev).contiguous()
            self.chunks = [(lay.gather(k, j).to(dev).contiguous(), lay.gather(v, j).to(dev).contiguous())
                           for j in range(w.n_chunks)]
            self.ring = RingAttention(lay, self.rank)
        tq, hq, d = self.q.shape
        self.o = torch.empty(tq, hq, d, device=dev)
        self.lse = torch.empty(hq, tq, device=dev)
        self.o_p = self.lse_p = None
        if w.n_chunks > 1 and w.mode == "ring" and not fused:
            self.o_p, self.lse_p = torch.empty_like(self.o), torch.empty_like(self.lse)
        if self.sweep:
            self.pairs = sum(lay.visible_pairs(r) for r in range(w.n_chunks))
        else:
            self.pairs = (self.zigzag[0] if w.mode == "zigzag" else lay).visible_pairs(self.rank)
        self.flops = 4 * w.head_dim * w.num_q_heads * self.pairs
        # every launch's arguments are marshalled once: the timed loop only enqueues
        if w.n_chunks == 1:
            from ring_attention_03_amd import attn_prefill_causal

            self.prefill = lambda: attn_prefill_causal(self.q, self.k, self.v, self.o, self.lse,
                                                       cu_seqlens=self.cu)
        elif w.mode == "chunked":
            self.prefill = ChunkedPrefill(lay, self.rank).prepare(self.q, self.k, self.v, self.o,
                                                                  self.lse)
        elif w.mode == "zigzag":
            self.prepared = self.zigzag[1].prepare(self.q, self.chunks, self.o, self.lse)
        elif self.sweep:
            self.outs = [(torch.empty(x.shape[0], hq, d, device=dev), torch.empty(hq, x.shape[0], device=dev))
                         for x in self.q_ranks]
            self.prepared_all = [RingAttention(lay, r).prepare(self.q_ranks[r], self.chunks, *self.outs[r],
                                                               fused=fused)
                                 for r in range(w.n_chunks)]
        else:
            self.prepared = self.ring.prepare(self.q, self.chunks, self.o, self.lse, self.o_p,
                                              self.lse_p, fused=fused)

    def run(self, events=None, event_pool=None):
        if self.w.n_chunks == 1 or self.w.mode == "chunked":
            if events is None:
                self.prefill()
            else:
                s, e = event_pool.pop(), event_pool.pop()
                s.record()
                self.prefill()
                e.record()
                events.append(("step", s, e))
            return 1
        if self.sweep:
            return sum(p.run(events=events, event_pool=event_pool) for p in self.prepared_all)
        return self.prepared.run(events=events, event_pool=event_pool)

    def launches_per_step(self):
        if self.sweep:
            return 2 * self.w.n_chunks * self.w.n_chunks
        return 1 if self.w.n_chunks == 1 or self.w.mode == "chunked" else 2 * self.w.n_chunks

    def config(self):
        w = self.w
        return {"workload": self.name, "description": w.note, "mode": w.mode, "seq_lens": list(w.seqlens),
                "ring_chunks": w.n_chunks,
                "rank": "all (one after another)" if self.sweep else self.rank, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                "head_dim": w.head_dim, "causal": True, "local_q_rows": int(self.q.shape[0]),
                "algorithmic_tflop": self.flops / 1e12,
                "merge": "in the step kernel" if self.fused else "separate merge kernel"}


def warm_up(job, warmup, min_seconds=0.0):
    """Run `warmup` untimed steps, then more until about `min_seconds` have passed.

    Returns the number of steps run.  After the host-side setup of a workload
    the GPU has idled, and its clock takes tens of milliseconds of load to
    settle (a 32K ring step ran 8% slow over its first 20 ms), so a workload
    with short steps needs more than a few steps of warmup.
    """
    import torch

    t0 = time.perf_counter()
    for _ in range(warmup):
        job.run()
    torch.cuda.synchronize()
    done = warmup
    elapsed = time.perf_counter() - t0
    if warmup > 0 and elapsed < min_seconds:
        more = int(math.ceil((min_seconds - elapsed) / (elapsed / warmup)))
        for _ in range(more):
            job.run()
        torch.cuda.synchronize()
        done += more
    return done


def time_job(job, steps, warmup, min_warmup_seconds=0.0):
    """Median-free whole-job timing: warmup, then exactly `steps` steps between synchronizations.

    The wall-clock region behind the throughput holds only the launches.  The
    per-kernel durations come from a second pass of the same `steps` steps,
    right after it, with HIP events recorded around every launch on the
    launch stream: each event is a packet of its own in the stream, which adds
    a few microseconds between launches, so it is kept out of the first region.
    `min_warmup_seconds` extends the warmup (see `warm_up`); the headline run
    uses exactly the requested warmup steps.
    """
    import torch

    job.warmup_steps_run = warm_up(job, warmup, min_warmup_seconds)
    t0 = time.perf_counter()
    for _ in range(steps):
        job.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # timing events are created before the event-timed pass (two per launch at most)
    pool = [torch.cuda.Event(enable_timing=True) for _ in range(2 * job.launches_per_step() * steps)]
    events = []
    torch.cuda.synchronize()
    for _ in range(steps):
        job.run(events=events, event_pool=pool)
    torch.cuda.synchronize()
    per_kind = {}
    for kind, s, e in events:
        per_kind.setdefault(kind, []).append(s.elapsed_time(e))
    return wall, per_kind


def time_cold(job, reps, flush_mib=1024):
    """Median time of one step with the caches cold: before each step a buffer
    larger than L2 and the last-level (MALL) cache together is overwritten, as
    K/V chunks on a real ring arrive fresh from a neighbour.  Each step is
    bracketed by events on the launch stream; the flush is outside them."""
    import torch

    flush = torch.empty(flush_mib * (1 << 20) // 4, device="cuda:0")
    times = []
    for i in range(reps):
        flush.fill_(float(i))
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        job.run()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    del flush
    times.sort()
    return times[len(times) // 2]


def summarize(job, steps, wall, per_kind):
    ms = wall * 1e3 / steps
    tflops = job.flops / (ms * 1e-3) / 1e12
    step_ms = per_kind.get("step", [])
    merge_ms = per_kind.get("merge", [])
    out = {"ms_per_step": ms, "tflops": tflops, "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
           "step_launches_per_step": len(step_ms) / steps,
           "step_kernel_ms_avg": (sum(step_ms) / len(step_ms)) if step_ms else None,
           "merge_kernel_ms_avg": (sum(merge_ms) / len(merge_ms)) if merge_ms else None}
    if step_ms:
        # all algorithmic flops are done by the attention launches
        out["attention_kernel_tflops"] = job.flops * steps / (sum(step_ms) * 1e-3) / 1e12
    return out


def traffic_entry(job):
    """HBM bytes per attention launch from committed counter runs, if they match this kernel build."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash() or rec.get("workload") != job.name:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(job, nrows):
    """The fp64 oracle timed on host cores for a seeded sample of the device's rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import causal_attention_ref, ring_ref
    from ring_attention_03_amd.workloads import sample_rows

    w = job.w
    q, k, v = job.cpu_inputs
    local_rows = int(job.q.shape[0])
    rows = sample_rows(local_rows, nrows, w.seed)[:nrows]
    t0 = time.perf_counter()
    if w.n_chunks == 1:
        causal_attention_ref(q, k, v, w.seqlens, rows=rows)
    else:
        ring_ref(q, k, v, w.seqlens, w.n_chunks, job.rank, rows=rows)
    sec = time.perf_counter() - t0
    # work of the sampled rows: each local row sees its global position + 1 keys
    cl = job.layout.chunk_lens
    cu = np.cumsum([0] + cl)
    pairs = 0
    for r in rows:
        b = int(np.searchsorted(cu, r, side="right") - 1)
        pairs += job.rank * cl[b] + (r - cu[b]) + 1
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {local_rows} local query rows (first/last 8 + seeded random), "
                      f"all {w.num_q_heads} heads, full ring; fp64 numpy; {sec:.1f} s, "
                      f"{flops / 1e9:.1f} GFLOP algorithmic; host {cpu}, os.cpu_count()={os.cpu_count()}"}


COPY_KERNEL = "neg_kernel"  # torch's elementwise negation: reads n words, writes n words


def calibrate_copy(mib):
    """A plain streaming kernel of known size (y = -x over `mib` MiB) for counter scaling."""
    import torch

    n = mib * (1 << 20) // 4
    x = torch.ones(n, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_each_way": n * 4, "launches": 3}), flush=True)


def _counter_per_dispatch(folder, counter, name_part):
    """Mean over matching dispatches of one counter (summed over its instances) in a --pmc run."""
    import csv
    import glob

    per_dispatch = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    for path in files:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    key = (path, r["Dispatch_Id"])
                    per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    if not per_dispatch:
        raise SystemExit(f"no {counter} values for kernels matching {name_part!r} under {folder}")
    vals = list(per_dispatch.values())
    return sum(vals) / len(vals), len(vals)


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload, copy_mib):
    """HBM bytes per attention launch, each counter scaled by its reading for a copy of known size.

    FETCH_SIZE and WRITE_SIZE count KiB moved between L2 and memory per
    dispatch.  The copy kernel moves exactly copy_mib MiB each way, so
    factor = bytes moved / (counter * 1024) corrects the counter's unit and
    coverage.  The result is averaged over all attention launches of the run,
    like the event-timed launch duration it sits beside.
    """
    copy_bytes = copy_mib * (1 << 20)
    cf, _ = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", COPY_KERNEL)
    cw, _ = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", COPY_KERNEL)
    f_kib, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", DOMINANT_KERNEL)
    w_kib, nw = _counter_per_dispatch(write_dir, "WRITE_SIZE", DOMINANT_KERNEL)
    ff, wf = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    rec = {"kernel": DOMINANT_KERNEL, "kernel_source_sha": kernel_source_hash(), "workload": workload,
           "bytes_per_launch": f_kib * 1024 * ff + w_kib * 1024 * wf,
           "fetch_bytes_per_launch": f_kib * 1024 * ff, "write_bytes_per_launch": w_kib * 1024 * wf,
           "fetch_kib_raw": f_kib, "write_kib_raw": w_kib, "launches": [nf, nw],
           "copy_mib": copy_mib, "fetch_factor": ff, "write_factor": wf}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)


# MI355X: 256 compute units of 4 SIMDs in 8 accelerator complex dies (XCDs)
N_CU, N_XCD, SIMD_PER_CU = 256, 8, 4


def _counters_present(folder, name_part):
    """Names of the counters recorded for kernels matching ``name_part`` in a --pmc run."""
    import csv
    import glob

    names = set()
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if name_part in r["Kernel_Name"]:
                    names.add(r["Counter_Name"])
    return names


def summarize_counters(folder):
    """Derived figures of the attention kernel from one rocprofv3 --pmc --kernel-trace run.

    Counter values are summed over their hardware instances per dispatch, then
    averaged over the kernel's dispatches.  GRBM_GUI_ACTIVE counts busy clocks
    of every XCD, so one XCD's share over the traced duration gives the
    shader clock; SQ_VALU_MFMA_BUSY_CYCLES counts per SIMD, so dividing by
    that clock count times the SIMD count gives the matrix cores' busy
    fraction at the clock the kernel actually ran.  The figures of whichever
    further counters the run holds are added: LDS (SQ_INSTS_LDS,
    SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE) or vector ALU
    (SQ_ACTIVE_INST_VALU in quad-cycles per wave, SQ_VALU_MFMA_COEXEC_CYCLES:
    cycles with the matrix core busy and a vector instruction issued).
    """
    import csv
    import glob

    present = _counters_present(folder, DOMINANT_KERNEL)
    need = ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA"]
    missing = [n for n in need if n not in present]
    if missing:
        raise SystemExit(f"counters {missing} missing for {DOMINANT_KERNEL} under {folder}")
    vals = {n: _counter_per_dispatch(folder, n, DOMINANT_KERNEL)[0] for n in sorted(present)}
    durs = []
    for path in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if DOMINANT_KERNEL in r["Kernel_Name"]:
                    durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    if not durs:
        raise SystemExit(f"no kernel trace of {DOMINANT_KERNEL} under {folder}")
    dur = sum(durs) / len(durs)
    clocks = vals["GRBM_GUI_ACTIVE"] / N_XCD
    simds = N_CU * SIMD_PER_CU
    mfma = vals["SQ_INSTS_MFMA"]
    rec = {"kernel": DOMINANT_KERNEL, "kernel_source_sha": kernel_source_hash(), "dispatches": len(durs),
           "avg_duration_us": dur * 1e6, "shader_clock_ghz": clocks / dur / 1e9,
           "mfma_busy_pct": 100.0 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (clocks * simds),
           "mfma_instructions": mfma}
    if "SQ_INSTS_VALU" in vals:
        rec["valu_per_mfma"] = vals["SQ_INSTS_VALU"] / mfma
    if "SQ_INSTS_VALU_TRANS_F32" in vals:
        rec["trans_per_mfma"] = vals["SQ_INSTS_VALU_TRANS_F32"] / mfma
    if "SQ_INSTS_LDS" in vals:
        rec["lds_per_mfma"] = vals["SQ_INSTS_LDS"] / mfma
    if "SQ_LDS_IDX_ACTIVE" in vals:
        rec["lds_active_pct"] = 100.0 * vals["SQ_LDS_IDX_ACTIVE"] / (clocks * N_CU)
        if "SQ_LDS_BANK_CONFLICT" in vals:
            rec["lds_bank_conflict_pct"] = 100.0 * vals["SQ_LDS_BANK_CONFLICT"] / max(vals["SQ_LDS_IDX_ACTIVE"], 1.0)
    if "SQ_ACTIVE_INST_VALU" in vals:
        rec["valu_active_pct"] = 100.0 * 4 * vals["SQ_ACTIVE_INST_VALU"] / (clocks * simds)
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in vals:
        rec["mfma_coexec_pct_of_busy"] = 100.0 * vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / vals["SQ_VALU_MFMA_BUSY_CYCLES"]
    if "SQ_WAVES" in vals:
        rec["waves"] = vals["SQ_WAVES"]
    rec["raw"] = vals
    print(json.dumps(rec, indent=1), flush=True)


def gemm_ceiling():
    """Sustained bf16 GEMM rate of the vendor library on N(0,1) data.

    The published dense peak assumes the top shader clock; with random
    operands the matrix cores draw enough power that the board lowers its
    clock, so a large library GEMM measures the rate that is reachable in
    practice.  The GPU is kept busy for a few seconds first so the clock
    has settled.
    """
    import torch

    n = 8192
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 3.0:
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    reps = 50
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
    print(json.dumps({"gemm": f"bf16 {n}x{n}x{n}, N(0,1) operands, torch.matmul (vendor BLAS)",
                      "ms": ms, "tflops": tf, "pct_bf16_peak": 100.0 * tf / PEAK_BF16_TFLOPS}), flush=True)


def mfma_ceiling():
    """Sustained rate of back-to-back 32x32x16 bf16 MFMAs on constant and on random operands.

    Two workgroups of 4 waves per CU (two waves per SIMD, all resident at
    once, so there is no tail of late workgroups), each wave doing 16 MFMAs
    per iteration on four independent accumulators; each case first runs for
    3 s so the clock settles under its own load.
    """
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "ring_attention_03_amd", "libattnprobe.so"))
    lib.attn_probe_mfma.restype = ctypes.c_int
    lib.attn_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 4096
    out = torch.empty(blocks * 256, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for name, random in (("constant_operands", 0), ("random_operands", 1)):
        def launch():
            st = lib.attn_probe_mfma(ctypes.c_void_p(out.data_ptr()), blocks, random, iters, stream)
            if st != 0:
                raise RuntimeError(f"attn_probe_mfma failed with HIP error {st}")
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 3.0:
            launch()
            torch.cuda.synchronize()
        reps = 20
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            launch()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        flops = blocks * 4 * iters * 16 * 2.0 * 32 * 32 * 16
        res[name] = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}
    res["pct_bf16_peak"] = {k: 100.0 * v["tflops"] / PEAK_BF16_TFLOPS for k, v in res.items()}
    print(json.dumps({"mfma": "v_mfma_f32_32x32x16_bf16, 2 waves per SIMD, 16 per iteration, 4 accumulators",
                      **res}), flush=True)


# probe modes of attn_probe_valu: (name, MFMAs per iteration, vector instructions per iteration)
VALU_PROBES = [
    ("v_fma_f32", 0, 32), ("v_exp_f32", 0, 32), ("v_add_f32", 0, 32), ("v_cvt_pk_bf16_f32", 0, 32),
    ("v_dot2c_f32_bf16", 0, 32), ("v_max3_f32", 0, 32),
    ("mfma_32x32x16_bf16", 16, 0), ("mfma_16x16x32_bf16", 16, 0),
    ("block_mix: 8 mfma + 16 fma + 16 exp + 16 add + 8 cvt", 8, 56),
    ("block_mix_without_exp: 8 mfma + 16 fma + 16 add + 8 cvt", 8, 40),
    ("block_mix_without_mfma: 16 fma + 16 exp + 16 add + 8 cvt", 0, 56),
    ("mfma_with_fma: 8 mfma + 32 fma", 8, 32),
    ("mfma_with_exp: 8 mfma + 16 exp", 8, 16),
    ("mfma_with_fma64: 8 mfma + 64 fma", 8, 64),
    None,  # (probe 14 retired)
    ("block_mix_poly_exp: 8 mfma + 16 fma + 16 cubic exp2 + 16 add + 8 cvt", 8, 168),
    ("block_mix_16x16x32: 16 mfma 16x16x32 + 16 fma + 16 exp + 16 add + 8 cvt", 8, 56),
    ("mfma_agpr_with_fma: 8 mfma (AGPR accumulators) + 32 fma", 8, 32),
    ("block_mix_agpr: 8 mfma (AGPR accumulators) + 16 fma + 16 exp + 16 add + 8 cvt", 8, 56),
    ("mfma16_with_fma: 16 mfma 16x16x32 + 32 fma", 8, 32),
    ("mfma_ab_agpr_with_fma: 8 mfma (A, B, C in AGPRs) + 32 fma", 8, 32),
    ("block_mix_ab_agpr: 8 mfma (A, B, C in AGPRs) + 16 fma + 16 exp + 16 add + 8 cvt", 8, 56),
    ("block_mix_a_agpr: 8 mfma (A, C in AGPRs) + 16 fma + 16 exp + 16 add + 8 cvt", 8, 56),
    ("block_mix_lds: the block mix with A operands from 4 ds_read_b128 + 8 ds_read_b64_tr_b16", 8, 56),
    ("block_mix_lds_unused: the same LDS reads issued, MFMAs on register operands", 8, 56),
    ("block_mix_lds_b128: the value operands by 4 ds_read_b128 (same bytes, 8 reads per block)", 8, 56),
    ("block_mix_lds_2tiles: two query sub-tiles per wave share each read (per-block figures)", 16, 112),
    ("v_mul_f32", 0, 32), ("v_fmamk_f32 (literal multiplier)", 0, 32), ("v_fmac_f32", 0, 32),
    ("block_mix_literal_scale: the block mix with its FMAs as v_fmamk_f32", 8, 56),
    ("block_mix_lds_literal_scale: the LDS-fed block mix with its FMAs as v_fmamk_f32", 8, 56),
    ("block_mix_lds_2tiles_random: probe 26 on random bf16 operands (per-block figures)", 16, 112),
]
MIX_2TILE, MIX_2TILE_RANDOM = 26, 32  # the kernel's inner loop: both query sub-tiles, LDS-fed


def mix_ceiling():
    """Sustained matrix-core rate of the attention kernel's inner-loop mix.

    Probes 26 and 32 of the probe library: per iteration a wave does what one
    kernel step does for its two 32-row query sub-tiles - 16 MFMAs 32x32x16
    with their key and value operands read from LDS as the kernel reads them,
    32 exponentials with their FMAs, 32 adds and 16 bf16 packs - on constant
    operands (26) or random ones (32, bf16 uniform in (-2, 2)).  One workgroup
    per CU with w waves per SIMD (2 is the kernel's occupancy).  Each case runs
    for 3 s first, so the clock settles under its own load, then 5 launches of
    about 0.2 s are timed.  The MFMA flops per second of that loop are what the
    kernel would reach if it did nothing but its inner loop: no tile copies,
    barriers, masks, keep checks, prologues, epilogues or launch ends.
    """
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "ring_attention_03_amd", "libattnprobe.so"))
    lib.attn_probe_valu.restype = ctypes.c_int
    lib.attn_probe_valu.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.empty(cus * 4 * 256, device="cuda:0")
    cyc, rt, st0 = (torch.empty(cus * 16, dtype=torch.int64, device="cuda:0") for _ in range(3))
    for mode, operands in ((MIX_2TILE, "constant"), (MIX_2TILE_RANDOM, "random")):
        for w in (2, 4):
            iters = 240_000 // w

            def launch():
                rc = lib.attn_probe_valu(*(ctypes.c_void_p(t.data_ptr()) for t in (sink, cyc, rt, st0)),
                                         mode, cus, w, iters, stream)
                if rc != 0:
                    raise RuntimeError(f"attn_probe_valu mode {mode} failed with HIP error {rc}")
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 3.0:
                launch()
                torch.cuda.synchronize()
            reps = 5
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                launch()
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e) / reps
            n = cus * 4 * w
            ticks, real = cyc[:n].double(), rt[:n].double()
            simd_per_iter = float(ticks.view(cus, 4 * w).max(dim=1).values.median()) / (iters * w)
            flops = n * iters * 16 * 2.0 * 32 * 32 * 16
            tf = flops / (ms * 1e-3) / 1e12
            print(json.dumps({"mix": "attention inner loop: 16 MFMA 32x32x16 + 32 exp + 32 fma + 32 add + "
                                     "16 cvt per wave-iteration, LDS-fed", "operands": operands,
                              "waves_per_simd": w, "ms": round(ms, 3), "tflops": round(tf, 1),
                              "pct_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
                              "clock_ghz": round(float((ticks / (real * 1e-8)).median()) / 1e9, 3),
                              "mfma_busy": round(32.0 * 16 / simd_per_iter, 3)}), flush=True)



def valu_rates():
    """Issue rates of the softmax's instruction mix, in shader clocks per SIMD.

    Each probe runs one instruction mix in a loop on every SIMD with w = 1, 2
    or 4 waves per SIMD (one workgroup of 4*w waves per CU).  Every wave reads
    the shader-clock counter (s_memtime) and the 100 MHz real-time counter
    around its loop and records its start; the waves of a workgroup start
    together (the start spread is reported).  Waves sharing a SIMD do not
    progress evenly - the oldest issues first - so a SIMD's time is its
    slowest wave's: SIMD clocks per loop iteration = the longest loop of a
    workgroup / (iterations * w), the median over workgroups.  Operands are
    nearly constant, so the clock stays high: these are issue rates, not
    power-limited rates.
    """
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "ring_attention_03_amd", "libattnprobe.so"))
    lib.attn_probe_valu.restype = ctypes.c_int
    lib.attn_probe_valu.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.empty(cus * 4 * 256, device="cuda:0")
    cyc, rt, st0 = (torch.empty(cus * 16, dtype=torch.int64, device="cuda:0") for _ in range(3))
    rows = []
    only = os.environ.get("VALU_PROBES")  # optional comma list of probe numbers
    for mode, probe in enumerate(VALU_PROBES):
        if probe is None or (only and str(mode) not in only.split(",")):
            continue
        name, n_mfma, n_valu = probe
        for w in (1, 2, 4):
            iters = 2000

            def launch():
                rc = lib.attn_probe_valu(*(ctypes.c_void_p(t.data_ptr()) for t in (sink, cyc, rt, st0)),
                                         mode, cus, w, iters, stream)
                if rc != 0:
                    raise RuntimeError(f"attn_probe_valu mode {mode} failed with HIP error {rc}")
            for _ in range(3):
                launch()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            launch()
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e)
            n = cus * 4 * w
            ticks, real, start = cyc[:n].double(), rt[:n].double(), st0[:n].double()
            simd_per_iter = float(ticks.view(cus, 4 * w).max(dim=1).values.median()) / (iters * w)
            clock = float((ticks / (real * 1e-8)).median()) / 1e9
            spread = float((start.max() - start.min()) / real.median())
            row = {"probe": name, "waves_per_simd": w, "simd_clocks_per_iteration": round(simd_per_iter, 2),
                   "clock_ghz": round(clock, 3), "launch_ms": round(ms, 4),
                   "start_spread_of_loop": round(spread, 4)}
            if n_mfma == 0:
                row["simd_clocks_per_vector_instruction"] = round(simd_per_iter / n_valu, 3)
            elif n_valu == 0:
                row["simd_clocks_per_mfma"] = round(simd_per_iter / n_mfma, 3)
            else:
                row["mfma_busy"] = round(32.0 * n_mfma / simd_per_iter, 3)
            rows.append(row)
            print(json.dumps(row), flush=True)
    return rows


def summarize_trace(folder, workload, warmup, steps):
    """Attention-kernel durations of a rocprofv3 --kernel-trace run of this script.

    Dispatches are taken in launch order.  A run launches warmup steps, then
    the timed steps, then the same steps again with events around every
    launch (cold passes are left out with --no-cold); the first
    warmup * launches-per-step dispatches are the warmup and are listed apart.
    """
    import csv
    import glob

    from ring_attention_03_amd import RingLayout
    from ring_attention_03_amd.workloads import WORKLOADS

    w = WORKLOADS[workload]
    if w.mode != "ring" or w.rank is None:
        raise SystemExit("--trace-from summarizes a single-rank ring workload")
    lay = RingLayout(w.seqlens, w.n_chunks)
    per_step = sum(1 for j in range(w.n_chunks) if j <= w.rank)  # chunks with visible keys
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if DOMINANT_KERNEL in r["Kernel_Name"]:
                    rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    if len(rows) < per_step * (warmup + 2 * steps):
        raise SystemExit(f"{len(rows)} dispatches, expected {per_step * (warmup + 2 * steps)}")
    durs = [(e - s) * 1e-3 for s, e in rows]  # microseconds
    warm, timed = durs[: per_step * warmup], durs[per_step * warmup:]
    flops = 4 * w.head_dim * w.num_q_heads * lay.visible_pairs(w.rank) / per_step
    avg = sum(timed) / len(timed)
    rec = {"kernel": DOMINANT_KERNEL, "workload": workload, "kernel_source_sha": kernel_source_hash(),
           "launches_per_step": per_step, "warmup_dispatches": len(warm),
           "warmup_avg_us": sum(warm) / len(warm) if warm else None,
           "timed_dispatches": len(timed), "timed_avg_us": avg, "timed_min_us": min(timed),
           "timed_max_us": max(timed), "kernel_ms_per_step": avg * per_step * 1e-3,
           "flop_per_launch": flops, "achieved_tflops": flops / (avg * 1e-6) / 1e12}
    print(json.dumps(rec, indent=1), flush=True)


def main():
    args = parse_args()
    if args.trace_from:
        summarize_trace(args.trace_from, args.workload, args.warmup, args.steps)
        return
    if args.counters_from:
        summarize_counters(args.counters_from)
        return
    if args.traffic_from:
        write_traffic(*args.traffic_from, workload=args.workload, copy_mib=args.calibrate_copy or 2048)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported "
              "(this library runs one device's share of the ring; it has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gemm_ceiling:
        gemm_ceiling()
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.valu_rates:
        valu_rates()
        return
    if args.mix_ceiling:
        mix_ceiling()
        return
    from ring_attention_03_amd import load_library

    load_library()
    log = lambda m: print(m, file=sys.stderr, flush=True)  # noqa: E731

    log(f"bench: preparing {args.workload}")
    job = Job(args.workload, fused=not args.unfused)
    wall, per_kind = time_job(job, args.steps, args.warmup)
    main_res = summarize(job, args.steps, wall, per_kind)
    # the same step with L2 and MALL flushed before it (median of 11)
    if not args.no_cold:
        main_res["cold_ms_per_step_median"] = time_cold(job, 11)
    log(f"bench: {args.workload}: {main_res['ms_per_step']:.3f} ms/step, {main_res['tflops']:.1f} TFLOP/s "
        f"({main_res['pct_bf16_peak']:.1f}% of bf16 peak)")

    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != args.workload]:
        log(f"bench: preparing {name}")
        ej = Job(name, fused=not args.unfused)
        ew, epk = time_job(ej, args.extra_steps, args.extra_warmup, min_warmup_seconds=0.3)
        extra[name] = summarize(ej, args.extra_steps, ew, epk)
        extra[name]["algorithmic_tflop"] = ej.flops / 1e12
        extra[name]["warmup_steps"] = ej.warmup_steps_run
        log(f"bench: {name}: {extra[name]['ms_per_step']:.3f} ms/step, {extra[name]['tflops']:.1f} TFLOP/s")
        del ej
        torch.cuda.empty_cache()

    achieved = main_res.get("attention_kernel_tflops")
    traffic = traffic_entry(job)
    roofline = {"bound": "mfma", "kernel": DOMINANT_KERNEL, "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": (achieved / PEAK_BF16_TFLOPS) if achieved else None,
                "traffic": traffic,
                "avg_launch_ms": main_res["step_kernel_ms_avg"],
                "flop_per_launch": job.flops / main_res["step_launches_per_step"]}

    base = None
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on a row sample (cpu_baseline)")
        base = cpu_baseline(job, args.cpu_rows)

    line = {"metric": METRIC, "value": main_res["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded iid N(0,1) Q/K, V per workload recipe; no model weights)",
            "config": job.config(), "pct_bf16_peak": main_res["pct_bf16_peak"],
            "roofline": roofline, "cpu_baseline": base,
            "detail": {args.workload: main_res, **extra},
            "kernel_source_sha": kernel_source_hash()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
