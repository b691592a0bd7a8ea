"""The oracle's ring result over many rows, split across worker processes.

Test infrastructure.  Each worker is a fresh interpreter (``spawn``, so nothing
of the test process - and nothing of its GPU state - is inherited); it rebuilds
the workload's seeded inputs once, then runs ``oracle.ring_ref`` on blocks of
rows with its BLAS held to one thread.  Rows are independent, so the blocks
simply concatenate.  Pool size: at most 16 workers, the CPU share of one GPU on
the test hosts.
"""

import multiprocessing as mp
import os

import numpy as np

_state = {}


def _init(name):
    from ring_attention_03_amd.workloads import WORKLOADS, make_qkv

    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    _state["w"] = w
    _state["qkv"] = tuple(x.float().numpy().astype(np.float64) for x in (q, k, v))


def _block(rows):
    from threadpoolctl import threadpool_limits

    from oracle import ring_ref

    w = _state["w"]
    q, k, v = _state["qkv"]
    with threadpool_limits(1):
        return ring_ref(q, k, v, w.seqlens, w.n_chunks, w.rank, rows=rows)


def ring_ref_rows(name, rows, block=64, workers=None):
    """(O [R, Hq, d], LSE [Hq, R]) of workload `name`'s ring share for `rows`."""
    rows = np.asarray(rows)
    n = workers or min(16, os.cpu_count() or 1)
    blocks = [rows[i:i + block] for i in range(0, len(rows), block)]
    with mp.get_context("spawn").Pool(n, initializer=_init, initargs=(name,)) as pool:
        parts = pool.map(_block, blocks)
    return np.concatenate([p[0] for p in parts], axis=0), np.concatenate([p[1] for p in parts], axis=1)
