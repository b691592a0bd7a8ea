"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on a GPU.

Tolerances are the ones the work is specified to: max abs error <= 1e-2 on O
and <= 1e-3 on LSE for bf16 inputs with fp32 accumulation; the fp32-input
path is held to 1e-4 on both.  Inputs come from the seeded recipe in
``ring_attention_03_amd.workloads``; expected values come only from the
oracle.  Small cases are compared on every element; the long-context
workloads at full size are compared on a seeded sample of rows (the first
and last 8 rows of the local chunk plus random ones) - rows are independent,
so every sampled row is an exact check.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import attention_ref, causal_attention_ref, chunk_layout_ref, merge_ref, ring_ref
from ring_attention_03_amd import (AttnError, ChunkedPrefill, RingAttention, RingLayout,
                                   ZigzagLayout, ZigzagRing, attn_prefill_causal, attn_ring_merge,
                                   attn_ring_step, attn_ring_step_merge)
from ring_attention_03_amd.workloads import WORKLOADS, make_qkv, sample_rows

pytestmark = pytest.mark.gpu

O_TOL_BF16, LSE_TOL_BF16 = 1e-2, 1e-3
TOL_F32 = 1e-4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def run_ring(q, k, v, seqlens, n, rank, scale=0.0, fused=True):
    """Run device ``rank``'s ring on the GPU from full packed CPU tensors; returns CPU (O, LSE)."""
    lay = RingLayout(tuple(seqlens), n)
    dev = "cuda"
    q_local = lay.gather(q, rank).to(dev).contiguous()
    chunks = [(lay.gather(k, j).to(dev).contiguous(), lay.gather(v, j).to(dev).contiguous())
              for j in range(n)]
    tq, hq, d = q_local.shape
    o = torch.empty(tq, hq, d, device=dev)
    lse = torch.empty(hq, tq, device=dev)
    o_p, lse_p = torch.empty_like(o), torch.empty_like(lse)
    RingAttention(lay, rank, scale).run(q_local, chunks, o, lse, o_p, lse_p, fused=fused)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def assert_close(o, lse, o_ref, lse_ref, o_tol, lse_tol, what=""):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite O"
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: -inf pattern of LSE"
    fin = np.isfinite(lse_ref)
    err_o = float(np.abs(o - o_ref).max()) if o.size else 0.0
    err_l = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    log(f"{what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= o_tol, f"{what}: O error {err_o}"
    assert err_l <= lse_tol, f"{what}: LSE error {err_l}"


# ---------------------------------------------------------------------------- the tiny fp32 ring
def test_tiny_ring_fp32_every_rank():
    w = WORKLOADS["tiny_ring_512"]
    q, k, v = make_qkv(w)
    full_o, full_lse = causal_attention_ref(q, k, v)
    for r in range(w.n_chunks):
        log(f"tiny fp32 ring rank {r}")
        o, lse = run_ring(q, k, v, w.seqlens, w.n_chunks, r)
        o_ref, lse_ref = ring_ref(q, k, v, w.seqlens, w.n_chunks, r)
        assert_close(o, lse, o_ref, lse_ref, TOL_F32, TOL_F32, f"fp32 rank {r}")
        rows = np.arange(r * 128, (r + 1) * 128)  # and the ring equals unchunked attention
        assert_close(o, lse, full_o[rows], full_lse[:, rows], TOL_F32, TOL_F32, "vs unchunked")


def test_fp32_ring_ragged_tiles_every_rank():
    # the fp32 kernel over many row tiles with ragged tails: chunks of 125 rows,
    # GQA 8:1, a varlen pair of sequences
    w = WORKLOADS["tiny_ring_512"].scaled(seqlens=(1000, 500), n_chunks=4, num_q_heads=16,
                                          num_kv_heads=2, seed=24)
    q, k, v = make_qkv(w)
    for r in range(w.n_chunks):
        log(f"fp32 ring {w.seqlens} N=4 16/2 rank {r}")
        o, lse = run_ring(q, k, v, w.seqlens, w.n_chunks, r, fused=(r % 2 == 0))
        o_ref, lse_ref = ring_ref(q, k, v, w.seqlens, w.n_chunks, r)
        assert_close(o, lse, o_ref, lse_ref, TOL_F32, TOL_F32, f"fp32 ring rank {r}")


# ---------------------------------------------------------------------------- bf16 rings, reduced size
RING_CASES = [
    # (seqlens, N, Hq, Hkv, v_dist) -- shapes of the long workloads, scaled down
    ((2048,), 4, 16, 2, "normal"),       # GQA 8:1, chunks of 512
    ((1000,), 8, 8, 2, "uniform"),       # GQA 4:1, chunks of 125 (ragged tiles)
    ((768,), 3, 4, 4, "normal"),         # MHA, chunks of 256
    ((1024, 512, 256, 128), 4, 8, 1, "normal"),  # varlen 8:1 (the head all-to-all share)
    ((640, 64, 192), 2, 16, 2, "normal"),        # varlen with a short sequence
    ((768,), 4, 12, 2, "uniform"),       # GQA 6:1: two heads per workgroup
    ((512,), 2, 12, 4, "normal"),        # GQA 3:1: one head per workgroup, kv head = head / 3
    # 16 head groups: each XCD's workgroups take a contiguous range of them
    ((640,), 2, 64, 8, "normal"),        # GQA 8:1 at the long workloads' 64/8 heads
    ((512,), 2, 32, 16, "uniform"),      # GQA 2:1, two heads per workgroup
    ((384,), 2, 16, 16, "normal"),       # MHA, one head per workgroup
]


@pytest.mark.parametrize("seqlens,n,hq,hkv,vd", RING_CASES)
def test_bf16_ring_every_rank(seqlens, n, hq, hkv, vd):
    w = WORKLOADS["ring_64k_rank7"].scaled(seqlens=seqlens, n_chunks=n, num_q_heads=hq,
                                           num_kv_heads=hkv, v_dist=vd, seed=11)
    q, k, v = make_qkv(w)
    for r in range(n):
        log(f"bf16 ring {seqlens} N={n} Hq={hq} Hkv={hkv} rank {r}")
        o, lse = run_ring(q, k, v, seqlens, n, r)
        o_ref, lse_ref = ring_ref(q, k, v, seqlens, n, r)
        assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, f"rank {r}")


def run_chunked(q, k, v, seqlens, n, index):
    """Chunked prefill of chunk ``index`` on the GPU from full packed CPU tensors; CPU (O, LSE)."""
    lay = RingLayout(tuple(seqlens), n)
    dev = "cuda"
    q_chunk = lay.gather(q, index).to(dev).contiguous()
    kp = lay.gather_prefix(k, index).to(dev).contiguous()
    vp = lay.gather_prefix(v, index).to(dev).contiguous()
    tq, hq, d = q_chunk.shape
    o = torch.full((tq, hq, d), float("nan"), device=dev)  # every row must be written
    lse = torch.full((hq, tq), float("nan"), device=dev)
    ChunkedPrefill(lay, index).run(q_chunk, kp, vp, o, lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


CHUNKED_CASES = [
    # (seqlens, N, Hq, Hkv, dtype): chunked prefill of every chunk index
    ((3072,), 6, 16, 2, "bf16"),                 # chunks of 512: 1..6 chunks of prefix
    ((1000, 600, 200), 4, 8, 1, "bf16"),         # varlen, ragged chunks (250, 150, 50)
    ((384,), 3, 4, 1, "fp32"),                   # the fp32 path
]


@pytest.mark.parametrize("seqlens,n,hq,hkv,dtype", CHUNKED_CASES)
def test_chunked_prefill_every_chunk(seqlens, n, hq, hkv, dtype):
    # each chunk's queries against its whole prefix in one call equal full causal
    # attention for those rows (the oracle's definition on the whole prompt)
    w = WORKLOADS["chunked_prefill_12k"].scaled(seqlens=seqlens, n_chunks=n, num_q_heads=hq,
                                                num_kv_heads=hkv, dtype=dtype, seed=23)
    q, k, v = make_qkv(w)
    tol = (O_TOL_BF16, LSE_TOL_BF16) if dtype == "bf16" else (TOL_F32, TOL_F32)
    for i in range(n):
        log(f"chunked prefill {seqlens} N={n} chunk {i} {dtype}")
        o, lse = run_chunked(q, k, v, seqlens, n, i)
        rows, _, _ = chunk_layout_ref(seqlens, n, i)
        o_ref, lse_ref = causal_attention_ref(q, k, v, seqlens, rows=rows)
        assert_close(o, lse, o_ref, lse_ref, *tol, f"chunk {i}")


def run_zigzag(q, k, v, seqlens, n, rank):
    """Device ``rank``'s zigzag ring on the GPU from full packed CPU tensors; CPU (O, LSE)."""
    zz = ZigzagLayout(tuple(seqlens), n)
    dev = "cuda"
    q_local = zz.gather(q, rank).to(dev).contiguous()
    pairs = [(zz.gather(k, j).to(dev).contiguous(), zz.gather(v, j).to(dev).contiguous())
             for j in range(n)]
    tq, hq, d = q_local.shape
    o = torch.full((tq, hq, d), float("nan"), device=dev)  # every row must be written
    lse = torch.full((hq, tq), float("nan"), device=dev)
    ZigzagRing(zz, rank).run(q_local, pairs, o, lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def zigzag_rows(seqlens, n, rank):
    """Global packed rows of device ``rank`` in its packed order (per sequence: early, late chunk)."""
    lo, _, _ = chunk_layout_ref(seqlens, 2 * n, rank)
    hi, _, _ = chunk_layout_ref(seqlens, 2 * n, 2 * n - 1 - rank)
    c = [s // (2 * n) for s in seqlens]
    rows, a = [], 0
    for cb in c:
        rows += list(lo[a:a + cb]) + list(hi[a:a + cb])
        a += cb
    return rows


ZIGZAG_CASES = [
    # (seqlens, N devices, Hq, Hkv, dtype)
    ((2048,), 4, 16, 2, "bf16"),                 # 8 chunks of 256
    ((1000, 600), 2, 8, 1, "bf16"),              # varlen, ragged chunks (250, 150)
    ((256,), 2, 4, 1, "fp32"),                   # the fp32 path
]


@pytest.mark.parametrize("seqlens,n,hq,hkv,dtype", ZIGZAG_CASES)
def test_zigzag_ring_every_rank(seqlens, n, hq, hkv, dtype):
    # each device's two chunks after its zigzag ring equal full causal attention
    # for those rows, and every device does the same causal work
    w = WORKLOADS["ring_64k_zigzag_rank7"].scaled(seqlens=seqlens, n_chunks=n, num_q_heads=hq,
                                                  num_kv_heads=hkv, dtype=dtype, seed=24)
    q, k, v = make_qkv(w)
    tol = (O_TOL_BF16, LSE_TOL_BF16) if dtype == "bf16" else (TOL_F32, TOL_F32)
    pairs = [ZigzagLayout(seqlens, n).visible_pairs(r) for r in range(n)]
    assert len(set(pairs)) == 1
    for r in range(n):
        log(f"zigzag ring {seqlens} N={n} rank {r} {dtype}")
        o, lse = run_zigzag(q, k, v, seqlens, n, r)
        o_ref, lse_ref = causal_attention_ref(q, k, v, seqlens, rows=zigzag_rows(seqlens, n, r))
        assert_close(o, lse, o_ref, lse_ref, *tol, f"zigzag rank {r}")


def _prefill(q, k, v, seqlens=None):
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    t, hq, d = q.shape
    o = torch.empty(t, hq, d, device=dev)
    lse = torch.empty(hq, t, device=dev)
    cu = None if seqlens is None else [0, *np.cumsum(seqlens).tolist()]
    attn_prefill_causal(qd, kd, vd, o, lse, cu_seqlens=cu)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("seqlens,hq,hkv,dtype", [
    ((1500,), 16, 2, "bf16"), ((300, 1, 77, 640), 8, 1, "bf16"), ((200,), 4, 1, "fp32"),
    ((65, 130), 6, 3, "fp32")])
def test_prefill_matches_oracle(seqlens, hq, hkv, dtype):
    w = WORKLOADS["prefill_100k"].scaled(seqlens=seqlens, num_q_heads=hq, num_kv_heads=hkv,
                                         dtype=dtype, seed=12)
    q, k, v = make_qkv(w)
    log(f"prefill {seqlens} {hq}/{hkv} {dtype}")
    o, lse = _prefill(q, k, v, seqlens)
    o_ref, lse_ref = causal_attention_ref(q, k, v, seqlens)
    tol = (O_TOL_BF16, LSE_TOL_BF16) if dtype == "bf16" else (TOL_F32, TOL_F32)
    assert_close(o, lse, o_ref, lse_ref, *tol, f"prefill {seqlens}")


def test_prefill_with_the_most_sequences_a_call_takes():
    # 64 packed sequences (the per-call maximum) of ragged lengths 1..97
    seqlens = tuple(1 + (37 * i) % 97 for i in range(64))
    w = WORKLOADS["prefill_100k"].scaled(seqlens=seqlens, num_q_heads=8, num_kv_heads=1, seed=23)
    q, k, v = make_qkv(w)
    log(f"prefill of {len(seqlens)} sequences, {sum(seqlens)} rows")
    o, lse = _prefill(q, k, v, seqlens)
    o_ref, lse_ref = causal_attention_ref(q, k, v, seqlens)
    assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "64 sequences")


def test_prefill_equals_ring_of_16():
    w = WORKLOADS["ring_100k_n16"].scaled(seqlens=(1024,), seed=13)
    q, k, v = make_qkv(w)
    o1, l1 = _prefill(q, k, v)
    for r in (0, 7, 15):
        o, lse = run_ring(q, k, v, w.seqlens, 16, r)
        rows = slice(r * 64, (r + 1) * 64)
        assert float((o - o1[rows]).abs().max()) < O_TOL_BF16
        assert float((lse - l1[:, rows]).abs().max()) < LSE_TOL_BF16


# ---------------------------------------------------------------------------- closed forms, edges
def test_zero_query_gives_prefix_mean():
    t = 300
    q = torch.zeros(t, 8, 64, dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(14)
    k = torch.randn(t, 1, 64, generator=g).to(torch.bfloat16)
    v = torch.randn(t, 1, 64, generator=g).to(torch.bfloat16)
    o, lse = _prefill(q, k, v)
    vv = v.double()[:, 0]
    mean = torch.cumsum(vv, 0) / torch.arange(1, t + 1, dtype=torch.float64)[:, None]
    # bf16 P is exactly 1.0 here, so only fp32 summation error remains
    assert float((o.double() - mean[:, None, :]).abs().max()) < 1e-4
    assert float((lse.double() - torch.log(torch.arange(1, t + 1).double())).abs().max()) < 1e-5


def test_uniform_v_and_large_scores():
    t = 700
    g = torch.Generator().manual_seed(15)
    q = (torch.randn(t, 8, 64, generator=g) * 30).to(torch.bfloat16)  # scores far past exp overflow
    k = torch.randn(t, 2, 64, generator=g).to(torch.bfloat16)
    row = torch.randn(1, 1, 64, generator=g).to(torch.bfloat16)
    v = row.expand(t, 2, 64).contiguous()
    o, lse = _prefill(q, k, v)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # O = v up to the bf16 rounding of the non-dominant weights (relative 2^-8)
    # and fp32 sums
    assert float((o - row.float()).abs().max()) < 4e-3 * float(row.float().abs().max())
    o_ref, lse_ref = causal_attention_ref(q, k, v)
    assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "scores x30, uniform V")


def _peaked_qkv(t, hq, hkv, vdist, seed):
    """Q x 30: scores far past exp overflow, so nearly every row is dominated by one key."""
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(t, hq, 64, generator=g) * 30).to(torch.bfloat16)
    k = torch.randn(t, hkv, 64, generator=g).to(torch.bfloat16)
    if vdist == "normal":
        v = torch.randn(t, hkv, 64, generator=g)
    else:
        v = 2 * torch.rand(t, hkv, 64, generator=g) - 1
    return q, k, v.to(torch.bfloat16)


@pytest.mark.parametrize("vdist", ["normal", "uniform"])
@pytest.mark.parametrize("seed", [15, 31, 47, 63])
def test_large_scores_prefill(vdist, seed):
    # One key dominates almost every row.  Its weight must enter O exactly (1.0),
    # not rounded to bf16 with relative error up to 2^-8, which would move O by
    # up to 2^-8 * |v| (~1e-2 for N(0,1) values).
    q, k, v = _peaked_qkv(700, 8, 2, vdist, seed)
    log(f"scores x30 prefill, V {vdist}, seed {seed}")
    o, lse = _prefill(q, k, v)
    o_ref, lse_ref = causal_attention_ref(q, k, v)
    assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, f"x30 prefill V {vdist} seed {seed}")


@pytest.mark.parametrize("vdist", ["normal", "uniform"])
def test_large_scores_ring_every_rank(vdist):
    # the same peaked rows through ring steps with the merge fused into the steps
    seqlens, n = (2048,), 4
    q, k, v = _peaked_qkv(2048, 16, 2, vdist, 41)
    for r in range(n):
        log(f"scores x30 ring N={n} rank {r}, V {vdist}")
        o, lse = run_ring(q, k, v, seqlens, n, r)
        o_ref, lse_ref = ring_ref(q, k, v, seqlens, n, r)
        assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, f"x30 ring rank {r} V {vdist}")


def test_very_negative_scores_keep_their_softmax():
    # Every score is about -1000 (log2 units): exponentials against any fixed
    # reference underflow, so the kernel must take each row's true maximum.
    g = torch.Generator().manual_seed(21)
    t = 600
    u = torch.randn(64, generator=g)
    u = u / u.norm()
    k = (u + 0.02 * torch.randn(t, 1, 64, generator=g))  # every key close to u
    q = -(1000.0 * 8.0 / 1.4427) * u + 0.5 * torch.randn(t, 8, 64, generator=g)
    v = torch.randn(t, 1, 64, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o, lse = _prefill(q, k, v)
    o_ref, lse_ref = causal_attention_ref(q, k, v)
    assert float(lse_ref.max()) < -400  # the scores really are that negative
    assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "very negative scores")


def test_growing_scores_rescale_every_block():
    # Scores grow along the keys (key i scores about 150*i/t against every
    # query), so each 32-key block exceeds the running reference by far more
    # than 2^8 and every block takes the rescale path; the softmax of each row
    # is dominated by its own latest keys.
    g = torch.Generator().manual_seed(22)
    t = 512
    u = torch.randn(64, generator=g)
    u = u / u.norm()
    ramp = torch.arange(t, dtype=torch.float32)[:, None, None] / t
    k = 40.0 * ramp * u + 0.05 * torch.randn(t, 2, 64, generator=g)
    q = 30.0 * u + 0.5 * torch.randn(t, 8, 64, generator=g)
    v = torch.randn(t, 2, 64, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o, lse = _prefill(q, k, v)
    o_ref, lse_ref = causal_attention_ref(q, k, v)
    assert float(lse_ref[:, -1].min()) > 100  # the last rows' scores really are that large
    assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "scores growing along the keys")


def test_fully_masked_step_skips_or_writes_identity():
    g = torch.Generator().manual_seed(16)
    q = torch.randn(100, 8, 64, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(50, 1, 64, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(50, 1, 64, generator=g).to(torch.bfloat16).cuda()
    o = torch.full((100, 8, 64), 7.0, device="cuda")
    lse = torch.full((8, 100), 7.0, device="cuda")
    launched = attn_ring_step(q, k, v, o, lse, q_pos0=[0], k_pos0=[100])
    torch.cuda.synchronize()
    assert launched is False and bool((o == 7).all())  # nothing enqueued
    attn_ring_step(q, k, v, o, lse, q_pos0=[0], k_pos0=[100], report_skip=False)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_partial_visibility_and_empty_sequences():
    # sequence 0: queries at 40.., keys at 60..: early rows see nothing, later ones some keys;
    # sequence 1 has no query rows; sequence 2 has no keys.
    g = torch.Generator().manual_seed(17)
    cu_q, cu_k = [0, 150, 150, 230], [0, 90, 190, 190]
    qp0, kp0 = [40, 0, 5], [60, 3, 0]
    q = torch.randn(230, 8, 64, generator=g).to(torch.bfloat16)
    k = torch.randn(190, 2, 64, generator=g).to(torch.bfloat16)
    v = torch.randn(190, 2, 64, generator=g).to(torch.bfloat16)
    o = torch.empty(230, 8, 64, device="cuda")
    lse = torch.empty(8, 230, device="cuda")
    assert attn_ring_step(q.cuda(), k.cuda(), v.cuda(), o, lse, cu_q=cu_q, cu_k=cu_k,
                          q_pos0=qp0, k_pos0=kp0)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_ref(q, k, v, cu_q=cu_q, cu_k=cu_k, q_pos0=qp0, k_pos0=kp0)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "partial")


def test_non_causal_block_and_explicit_scale():
    g = torch.Generator().manual_seed(18)
    q = torch.randn(130, 16, 64, generator=g).to(torch.bfloat16)
    k = torch.randn(333, 2, 64, generator=g).to(torch.bfloat16)
    v = torch.randn(333, 2, 64, generator=g).to(torch.bfloat16)
    o = torch.empty(130, 16, 64, device="cuda")
    lse = torch.empty(16, 130, device="cuda")
    attn_ring_step(q.cuda(), k.cuda(), v.cuda(), o, lse, causal=False, scale=0.09)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_ref(q, k, v, causal=False, scale=0.09)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "non-causal")


def test_merge_kernel_matches_oracle():
    g = torch.Generator().manual_seed(19)
    t, h = 333, 8
    oa, ob = torch.randn(t, h, 64, generator=g), torch.randn(t, h, 64, generator=g)
    la, lb = torch.randn(h, t, generator=g) * 5, torch.randn(h, t, generator=g) * 5
    la[0, :10] = -math.inf
    lb[1, :10] = -math.inf
    la[2, :5] = -math.inf
    lb[2, :5] = -math.inf
    oa[:10, 0] = 0
    ob[:10, 1] = 0
    oa[:5, 2] = 0
    ob[:5, 2] = 0
    o_acc, l_acc = oa.cuda(), la.cuda()
    attn_ring_merge(o_acc, l_acc, ob.cuda(), lb.cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = merge_ref(oa, la, ob, lb)
    assert_close(o_acc.cpu(), l_acc.cpu(), o_ref, l_ref, 1e-5, 1e-5, "merge")


@pytest.mark.parametrize("seqlens,n,hq,hkv,vd", [RING_CASES[0], RING_CASES[3]])
def test_fused_merge_ring_matches_unfused_ring(seqlens, n, hq, hkv, vd):
    # the merge folded into the step epilogue computes the same log-sum-exp
    # combination as the separate merge kernel: only rounding may differ
    w = WORKLOADS["ring_64k_rank7"].scaled(seqlens=seqlens, n_chunks=n, num_q_heads=hq,
                                           num_kv_heads=hkv, v_dist=vd, seed=21)
    q, k, v = make_qkv(w)
    for r in range(n):
        log(f"fused vs unfused ring {seqlens} N={n} rank {r}")
        o_f, lse_f = run_ring(q, k, v, seqlens, n, r, fused=True)
        o_u, lse_u = run_ring(q, k, v, seqlens, n, r, fused=False)
        assert torch.equal(torch.isneginf(lse_f), torch.isneginf(lse_u))
        fin = torch.isfinite(lse_u)
        assert float((o_f - o_u).abs().max()) <= 1e-5
        assert float((lse_f[fin] - lse_u[fin]).abs().max()) <= 1e-5
        o_ref, lse_ref = ring_ref(q, k, v, seqlens, n, r)
        assert_close(o_f, lse_f, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, f"fused rank {r}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_step_merge_folds_a_block_into_the_state(dtype):
    # running state from one key block (positions 0..89), then a second block
    # (positions 90..199) folded in by the fused step; queries at 40..229, so
    # the first 50 rows see no key of the second block and must stay untouched
    g = torch.Generator().manual_seed(22)
    tq, hq, hkv = 190, 8, 2
    q = torch.randn(tq, hq, 64, generator=g).to(dtype)
    k = torch.randn(200, hkv, 64, generator=g).to(dtype)
    v = torch.randn(200, hkv, 64, generator=g).to(dtype)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty(tq, hq, 64, device="cuda")
    lse = torch.empty(hq, tq, device="cuda")
    assert attn_ring_step(qd, kd[:90], vd[:90], o, lse, q_pos0=[40], k_pos0=[0])
    torch.cuda.synchronize()
    o_before, lse_before = o.clone(), lse.clone()
    assert attn_ring_step_merge(qd, kd[90:].contiguous(), vd[90:].contiguous(), o, lse,
                                q_pos0=[40], k_pos0=[90])
    torch.cuda.synchronize()
    assert torch.equal(o[:50], o_before[:50]) and torch.equal(lse[:, :50], lse_before[:, :50])
    oa, la = attention_ref(q, k[:90], v[:90], q_pos0=[40], k_pos0=[0])
    ob, lb = attention_ref(q, k[90:], v[90:], q_pos0=[40], k_pos0=[90])
    o_ref, lse_ref = merge_ref(oa, la, ob, lb)
    full_o, full_lse = attention_ref(q, k, v, q_pos0=[40], k_pos0=[0])  # and that is full attention
    assert np.abs(o_ref - full_o).max() < 1e-12 and np.abs(lse_ref - full_lse).max() < 1e-12
    tol = (O_TOL_BF16, LSE_TOL_BF16) if dtype == torch.bfloat16 else (TOL_F32, TOL_F32)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, *tol, f"step merge {dtype}")
    # a block wholly in the future of every row enqueues nothing and changes nothing
    o_before, lse_before = o.clone(), lse.clone()
    assert not attn_ring_step_merge(qd, kd, vd, o, lse, q_pos0=[40], k_pos0=[400])
    torch.cuda.synchronize()
    assert torch.equal(o, o_before) and torch.equal(lse, lse_before)


def test_deterministic():
    # Ten runs of a full-tile ring share are bitwise identical: an 8192-row query
    # chunk against its 8192-key diagonal chunk and one full chunk, merged in the
    # step epilogue, 64 query / 8 kv heads (every LDS buffer of the pipeline and
    # every head of a workgroup in use).
    w = WORKLOADS["ring_64k_rank7"].scaled(seqlens=(16384,), n_chunks=2, seed=20)
    q, k, v = make_qkv(w)
    lay = RingLayout(w.seqlens, 2)
    q_local = lay.gather(q, 1).cuda().contiguous()
    chunks = [(lay.gather(k, j).cuda().contiguous(), lay.gather(v, j).cuda().contiguous()) for j in range(2)]
    first = None
    for rep_i in range(10):
        o = torch.full((8192, 64, 64), float("nan"), device="cuda")
        lse = torch.full((64, 8192), float("nan"), device="cuda")
        RingAttention(lay, 1).run(q_local, chunks, o, lse, None, None, fused=True)
        torch.cuda.synchronize()
        if first is None:
            first = (o.clone(), lse.clone())
            assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        else:
            assert torch.equal(first[0], o) and torch.equal(first[1], lse), f"repeat {rep_i} differs"
    log("10 repeats bitwise identical")


def test_invalid_arguments_raise_before_launch():
    q = torch.zeros(64, 6, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(64, 4, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(64, 6, 64, device="cuda")
    lse = torch.empty(6, 64, device="cuda")
    with pytest.raises(AttnError):
        attn_ring_step(q, k, k, o, lse)  # 6 query heads over 4 kv heads
    with pytest.raises(TypeError):
        attn_ring_step(q, k.float(), k.float(), o, lse)
    with pytest.raises(ValueError):
        attn_ring_step(q.cpu(), k, k, o, lse)
    q2 = torch.zeros(64, 8, 32, dtype=torch.bfloat16, device="cuda")
    k2 = torch.zeros(64, 1, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnError) as e:
        attn_ring_step(q2, k2, k2, torch.empty(64, 8, 32, device="cuda"),
                       torch.empty(8, 64, device="cuda"))
    assert e.value.status == 2


# ---------------------------------------------------------------------------- full-size workloads
FULL = [("ring_32k_rank3", 24), ("ring_64k_rank7", 24), ("varlen_ulysses_rank7", 24)]


@pytest.mark.parametrize("name,nsample", FULL)
def test_full_size_ring_sampled_rows(name, nsample):
    w = WORKLOADS[name]
    log(f"full-size {name}: generating inputs")
    q, k, v = make_qkv(w)
    o, lse = run_ring(q, k, v, w.seqlens, w.n_chunks, w.rank)
    rows = sample_rows(o.shape[0], nsample, w.seed)
    log(f"full-size {name}: oracle on {len(rows)} rows")
    o_ref, lse_ref = ring_ref(q, k, v, w.seqlens, w.n_chunks, w.rank, rows=rows)
    assert_close(o[rows], lse[:, rows], o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, name)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("name", ["ring_32k_rank3", "ring_64k_rank7", "varlen_ulysses_rank7"])
def test_full_size_ring_every_row(name):
    """A full-size ring share (C2, C3, C5) against the oracle on every local row and head."""
    from oracle_pool import ring_ref_rows

    w = WORKLOADS[name]
    log(f"full-size {name}, every row: generating inputs")
    q, k, v = make_qkv(w)
    o, lse = run_ring(q, k, v, w.seqlens, w.n_chunks, w.rank)
    log(f"full-size {name}: oracle on all {o.shape[0]} rows (worker pool)")
    o_ref, lse_ref = ring_ref_rows(name, np.arange(o.shape[0]))
    assert_close(o, lse, o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, f"{name} every row")


def test_full_size_chunked_prefill_sampled_rows():
    w = WORKLOADS["chunked_prefill_12k"]
    log("full-size chunked_prefill_12k: generating inputs")
    q, k, v = make_qkv(w)
    o, lse = run_chunked(q, k, v, w.seqlens, w.n_chunks, w.rank)
    local = sample_rows(o.shape[0], 24, w.seed)
    rows, _, _ = chunk_layout_ref(w.seqlens, w.n_chunks, w.rank)
    log(f"full-size chunked_prefill_12k: oracle on {len(local)} rows")
    o_ref, lse_ref = causal_attention_ref(q, k, v, w.seqlens, rows=[rows[r] for r in local])
    assert_close(o[local], lse[:, local], o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "chunked 12k")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("rank", [0, 7])
def test_full_size_zigzag_sampled_rows(rank):
    w = WORKLOADS["ring_64k_zigzag_rank7"]
    log(f"full-size zigzag rank {rank}: generating inputs")
    q, k, v = make_qkv(w)
    o, lse = run_zigzag(q, k, v, w.seqlens, w.n_chunks, rank)
    local = sample_rows(o.shape[0], 24, w.seed + rank)
    rows = zigzag_rows(w.seqlens, w.n_chunks, rank)
    log(f"full-size zigzag rank {rank}: oracle on {len(local)} rows")
    o_ref, lse_ref = causal_attention_ref(q, k, v, w.seqlens, rows=[rows[r] for r in local])
    assert_close(o[local], lse[:, local], o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "zigzag 64k")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_full_size_prefill_100k_and_ring16_sampled_rows():
    w = WORKLOADS["prefill_100k"]
    log("prefill_100k: generating inputs")
    q, k, v = make_qkv(w)
    o, lse = _prefill(q, k, v)
    rows = sample_rows(o.shape[0], 24, w.seed)
    o_ref, lse_ref = causal_attention_ref(q, k, v, rows=rows)
    assert_close(o[rows], lse[:, rows], o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, "prefill 100k")
    # The same sequence as a ring of 16 chunks of 6400: every rank against the
    # oracle's ring on sampled rows (each chunk's first and last 8 rows plus
    # seeded ones), and every row of every rank against the prefill.
    n = WORKLOADS["ring_100k_n16"].n_chunks
    qf, kf, vf = (x.float().numpy().astype(np.float64) for x in (q, k, v))  # upcast once (exact)
    for r in range(n):
        orr, lr = run_ring(q, k, v, w.seqlens, n, r)
        lr_rows = sample_rows(6400, 12, w.seed + 100 + r)
        o_ref, lse_ref = ring_ref(qf, kf, vf, w.seqlens, n, r, rows=lr_rows)
        assert_close(orr[lr_rows], lr[:, lr_rows], o_ref, lse_ref, O_TOL_BF16, LSE_TOL_BF16, f"ring16 rank {r}")
        sl = slice(r * 6400, (r + 1) * 6400)
        do = float((orr - o[sl]).abs().max())
        dl = float((lr - lse[:, sl]).abs().max())
        log(f"ring16 rank {r}: max|dO| vs prefill {do:.2e}, max|dLSE| {dl:.2e}")
        assert do < O_TOL_BF16 and dl < LSE_TOL_BF16
