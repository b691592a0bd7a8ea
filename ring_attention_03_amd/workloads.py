"""Seeded synthetic inputs for the ring-attention workloads.

This module only draws random numbers and describes shapes: it holds none of
the attention arithmetic, so both the oracle-side tests and the device path
can take their inputs from it.  It imports neither the native library nor the
oracle.

The workloads mirror the evaluation of Moreh's "Optimizing Long-Context
Prefill on Multiple Older-Generation GPU Nodes" (section "Evaluation": long
single prompts of 32K, 64K and 100K tokens on a GQA model) at the attention
shape of one device's share: 64 query heads sharing 8 key/value heads with
head_dim 64, or the 8:1 share left after a head all-to-all.  No model weights
or datasets are involved: Q/K/V are iid draws from a seeded CPU generator.

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; draw the whole packed
Q [T, Hq, d], then K [T, Hkv, d], then V [T, Hkv, d] in float32 - ``randn``
for N(0,1), ``2*rand-1`` for U(-1,1) - then cast to the workload dtype with
round-to-nearest-even.  Chunks and local rows are slices of these tensors.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple            # lengths of the packed sequences (whole prompts)
    n_chunks: int             # ring size N: every sequence is cut into N equal chunks
    rank: int | None          # the device whose share is timed (None: every rank)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                # "bf16" or "fp32"
    v_dist: str = "normal"    # "normal" = N(0,1), "uniform" = U(-1,1)
    seed: int = 0
    # "ring": the rank's query chunk against every key/value chunk in ring order;
    # "chunked": chunked prefill - the rank's query chunk against its whole
    # prefix (chunks 0..rank) in one call;
    # "zigzag": load-balanced ring - sequences cut into 2N chunks, device r
    # holds chunks r and 2N-1-r (n_chunks is the device count N)
    mode: str = "ring"
    note: str = field(default="", compare=False)

    def __post_init__(self):
        if self.mode not in ("ring", "chunked", "zigzag"):
            raise ValueError(f"workload {self.name}: unknown mode {self.mode!r}")

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    def scaled(self, **changes) -> "Workload":
        """A copy with some fields changed (used for reduced-size parity cases)."""
        return replace(self, **changes)


WORKLOADS = {
    "tiny_ring_512": Workload(
        "tiny_ring_512", (512,), 4, None, 4, 1, 64, "fp32", "normal", 1, "ring",
        "S=512 in 4 ring chunks of 128, GQA 4:1, fp32; every rank"),
    "ring_32k_rank3": Workload(
        "ring_32k_rank3", (32768,), 8, 3, 64, 8, 64, "bf16", "normal", 2, "ring",
        "S=32768 in 8 chunks of 4096, rank 3 against all 8 chunks"),
    "ring_64k_rank7": Workload(
        "ring_64k_rank7", (65536,), 8, 7, 64, 8, 64, "bf16", "uniform", 3, "ring",
        "S=65536 in 8 chunks of 8192, last rank (heaviest causal share)"),
    "prefill_100k": Workload(
        "prefill_100k", (102400,), 1, 0, 64, 8, 64, "bf16", "normal", 4, "ring",
        "S=102400 full causal prefill in one call"),
    "ring_100k_n16": Workload(
        "ring_100k_n16", (102400,), 16, None, 64, 8, 64, "bf16", "normal", 4, "ring",
        "S=102400 in 16 ring chunks of 6400, every rank"),
    "ring_100k_n16_rank15": Workload(
        "ring_100k_n16_rank15", (102400,), 16, 15, 64, 8, 64, "bf16", "normal", 4, "ring",
        "S=102400 in 16 ring chunks of 6400, last rank (heaviest causal share)"),
    "ring_64k_zigzag_rank7": Workload(
        "ring_64k_zigzag_rank7", (65536,), 8, 7, 64, 8, 64, "bf16", "uniform", 3, "zigzag",
        "S=65536 on 8 devices, load-balanced: 16 chunks of 4096, rank 7 holds chunks 7 and 8"),
    "chunked_prefill_12k": Workload(
        "chunked_prefill_12k", (98304,), 8, 7, 64, 8, 64, "bf16", "normal", 6, "chunked",
        "chunked prefill: the 8th 12288-token chunk of a 98304-token prompt against its prefix"),
    "varlen_ulysses_rank7": Workload(
        "varlen_ulysses_rank7", (131072, 65536, 32768, 16384), 8, 7, 8, 1, 64, "bf16",
        "normal", 5, "ring",
        "4 packed requests after a head all-to-all (8 q / 1 kv head), N=8, rank 7"),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def make_qkv(w: Workload):
    """Full packed (Q, K, V) on the CPU for workload ``w`` (see the module recipe)."""
    g = torch.Generator(device="cpu").manual_seed(int(w.seed))
    t = w.total_tokens
    q = torch.randn(t, w.num_q_heads, w.head_dim, generator=g, dtype=torch.float32)
    k = torch.randn(t, w.num_kv_heads, w.head_dim, generator=g, dtype=torch.float32)
    if w.v_dist == "uniform":
        v = 2.0 * torch.rand(t, w.num_kv_heads, w.head_dim, generator=g, dtype=torch.float32) - 1.0
    else:
        v = torch.randn(t, w.num_kv_heads, w.head_dim, generator=g, dtype=torch.float32)
    dt = torch_dtype(w.dtype)
    return q.to(dt), k.to(dt), v.to(dt)


def sample_rows(n_rows: int, count: int, seed: int, edge: int = 8):
    """Sorted row indices in [0, n_rows): the first and last ``edge`` rows plus seeded random ones."""
    g = torch.Generator(device="cpu").manual_seed(int(seed) + 7919)
    edge_rows = set(range(min(edge, n_rows))) | set(range(max(0, n_rows - edge), n_rows))
    extra = torch.randperm(n_rows, generator=g)[:count].tolist()
    return sorted(edge_rows | set(extra))
