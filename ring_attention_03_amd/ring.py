"""Host-side ring schedule for one device's share of a ring-attention prefill.

Context parallelism cuts each prompt along the sequence into N contiguous
chunks, one per device; with Ring Attention every device keeps its query
chunk and runs attention on each key/value chunk as it arrives from its ring
neighbour (Moreh, "Optimizing Long-Context Prefill on Multiple
Older-Generation GPU Nodes", section "Introduction to Context Parallelism":
the context-parallelism paragraph and the Ring Attention bullet).  At step t
device r holds the chunk that started on device (r - t) mod N.

On one GPU the ring is simulated: all key/value chunks are already resident
in HBM and the "arrival" of chunk j is simply its turn in the loop.  This
module only does index arithmetic and calls the library; every step of the
computation runs in the HIP kernels.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _native


@dataclass(frozen=True)
class RingLayout:
    """Packed sequences, each cut into ``n_chunks`` equal contiguous chunks."""

    seqlens: tuple
    n_chunks: int

    def __post_init__(self):
        for n in self.seqlens:
            if n % self.n_chunks:
                raise ValueError(f"sequence length {n} does not split into {self.n_chunks} chunks")

    @property
    def chunk_lens(self):
        return [n // self.n_chunks for n in self.seqlens]

    @property
    def cu(self):
        """Prefix offsets of one chunk in packed form (the same for every chunk)."""
        out = [0]
        for c in self.chunk_lens:
            out.append(out[-1] + c)
        return out

    def pos0(self, chunk: int):
        """Global position of each sequence's first token in chunk ``chunk``."""
        return [chunk * c for c in self.chunk_lens]

    def ranges(self, chunk: int):
        """Row ranges (start, stop) of chunk ``chunk`` inside the full packed tensor."""
        out, start = [], 0
        for n, c in zip(self.seqlens, self.chunk_lens):
            out.append((start + chunk * c, start + (chunk + 1) * c))
            start += n
        return out

    def gather(self, x: torch.Tensor, chunk: int) -> torch.Tensor:
        """Chunk ``chunk`` of packed tensor ``x`` in packed form (a view for one sequence)."""
        parts = [x[a:b] for a, b in self.ranges(chunk)]
        return parts[0] if len(parts) == 1 else torch.cat(parts, dim=0)

    def prefix_cu(self, chunk: int):
        """Prefix offsets of chunks 0..chunk of every sequence, packed (a chunked-prefill key set)."""
        out = [0]
        for c in self.chunk_lens:
            out.append(out[-1] + (chunk + 1) * c)
        return out

    def gather_prefix(self, x: torch.Tensor, chunk: int) -> torch.Tensor:
        """Chunks 0..chunk of every sequence of packed ``x``, packed (a view for one sequence)."""
        parts, start = [], 0
        for n, c in zip(self.seqlens, self.chunk_lens):
            parts.append(x[start:start + (chunk + 1) * c])
            start += n
        return parts[0] if len(parts) == 1 else torch.cat(parts, dim=0)

    def visible_pairs(self, rank: int) -> int:
        """Causal (query, key) pairs whose query is in chunk ``rank``."""
        total = 0
        for c in self.chunk_lens:
            lo, hi = rank * c, (rank + 1) * c
            total += (hi * (hi + 1) - lo * (lo + 1)) // 2
        return total


def ring_chunk(rank: int, step: int, n_chunks: int) -> int:
    """Key/value chunk that device ``rank`` holds at ring step ``step``."""
    return (rank - step) % n_chunks


class RingAttention:
    """Runs device ``rank``'s ring: N steps of attention merged by LSE into (o, lse).

    ``q_local`` is the device's packed query chunk; ``kv_chunks[j]`` is the
    packed (k, v) of chunk j, already in device memory.  The first step that
    has visible keys writes straight into the running state (merging into the
    identity would give the same result); every later active step is folded
    in by log-sum-exp.  By default the fold happens in the step kernel's
    epilogue (``attn_ring_step_merge``); with ``o_part``/``lse_part`` given and
    ``fused=False`` each step writes the partial buffers and
    ``attn_ring_merge`` folds them in.  Fully masked steps launch nothing.

    ``prepare`` marshals every call of the ring once; the returned
    ``PreparedRing`` can run the same ring on the same buffers many times with
    no per-launch argument work (the schedule is static).
    """

    def __init__(self, layout: RingLayout, rank: int, scale: float = 0.0):
        if not 0 <= rank < layout.n_chunks:
            raise ValueError("rank outside the ring")
        self.layout = layout
        self.rank = rank
        self.scale = scale

    def prepare(self, q_local, kv_chunks, o_acc, lse_acc, o_part=None, lse_part=None, stream=None,
                fused=True) -> "PreparedRing":
        if not fused and (o_part is None or lse_part is None):
            raise ValueError("the unfused ring needs o_part and lse_part")
        lay, r = self.layout, self.rank
        cu = lay.cu
        q_pos0 = lay.pos0(r)
        steps = []
        for t in range(lay.n_chunks):
            j = ring_chunk(r, t, lay.n_chunks)
            k_j, v_j = kv_chunks[j]
            kw = dict(cu_q=cu, cu_k=cu, q_pos0=q_pos0, k_pos0=lay.pos0(j), scale=self.scale,
                      causal=True, stream=stream)
            write = _native.prepare_ring_step(q_local, k_j, v_j, o_acc, lse_acc, report_skip=True, **kw)
            if fused:
                fold, merge = _native.prepare_ring_step_merge(q_local, k_j, v_j, o_acc, lse_acc, **kw), None
            else:
                fold = _native.prepare_ring_step(q_local, k_j, v_j, o_part, lse_part, report_skip=True, **kw)
                merge = _native.prepare_ring_merge(o_acc, lse_acc, o_part, lse_part, stream=stream)
            steps.append((write, fold, merge))
        k_0, v_0 = kv_chunks[ring_chunk(r, 0, lay.n_chunks)]
        identity = _native.prepare_ring_step(q_local, k_0, v_0, o_acc, lse_acc, cu_q=cu, cu_k=cu,
                                             q_pos0=q_pos0, k_pos0=lay.pos0(r), scale=self.scale,
                                             causal=True, report_skip=False, stream=stream)
        return PreparedRing(steps, identity, stream)

    def run(self, q_local, kv_chunks, o_acc, lse_acc, o_part=None, lse_part=None, stream=None,
            events=None, fused=True) -> int:
        """Run the ring once; returns the number of steps that launched work.

        ``events``, if a list, receives ``(kind, start, end)`` timing events
        (kind "step" or "merge") recorded on the launch stream around every
        launch, for per-kernel timing.
        """
        ring = self.prepare(q_local, kv_chunks, o_acc, lse_acc, o_part, lse_part, stream, fused)
        return ring.run(events=events)


class ZigzagLayout:
    """Load-balanced causal ring: every sequence is cut into 2N equal chunks and
    device r holds chunks r and 2N-1-r (an early and a late one), so every
    device does the same causal work, where contiguous chunks give device N-1
    N times the work of device 0.  The kernels take arbitrary per-sequence
    positions and key ranges, so only the host schedule differs from the
    contiguous ring.  A device's local rows (and the key/value pair it holds)
    are packed per sequence as [early chunk; late chunk].
    """

    def __init__(self, seqlens, n_devices: int):
        self.seqlens = tuple(seqlens)
        self.n = n_devices
        self.chunks = RingLayout(self.seqlens, 2 * n_devices)

    @property
    def chunk_lens(self):
        return self.chunks.chunk_lens

    def pair(self, dev: int):
        return dev, 2 * self.n - 1 - dev

    def cu(self):
        """Packed offsets of the 2B segments (early, late per sequence) of a local pair."""
        out = [0]
        for c in self.chunk_lens:
            out += [out[-1] + c, out[-1] + 2 * c]
        return out

    def positions(self, dev: int):
        """Global position of each segment's first token on device ``dev``."""
        lo, hi = self.pair(dev)
        out = []
        for c in self.chunk_lens:
            out += [lo * c, hi * c]
        return out

    def gather(self, x: torch.Tensor, dev: int) -> torch.Tensor:
        """Device ``dev``'s rows of packed ``x``: per sequence its early then late chunk."""
        lo, hi = self.pair(dev)
        parts = []
        for (a, b), (c, d) in zip(self.chunks.ranges(lo), self.chunks.ranges(hi)):
            parts += [x[a:b], x[c:d]]
        return torch.cat(parts, dim=0)

    def visible_pairs(self, dev: int) -> int:
        lo, hi = self.pair(dev)
        return self.chunks.visible_pairs(lo) + self.chunks.visible_pairs(hi)


class ZigzagRing:
    """Device ``rank``'s share of a zigzag ring (see ZigzagLayout).

    At step t the device holds device j = (rank - t) mod N's key/value pair
    (X = chunk j, Y = chunk 2N-1-j) and its own query pair (A = chunk rank,
    B = chunk 2N-1-rank).  A sees X in full when j < rank, causally when
    j = rank, and never sees Y; B sees all of X always, and Y (causally, on
    the diagonal when j = rank) when j >= rank.  Each step is one launch over
    the 2B packed query segments, each with one key range:

    * A: the rows of X, or none when j > rank;
    * B: X and Y together when j >= rank - they are adjacent rows of the held
      pair - with positions counted back from Y's first key, so X's keys sit
      just before Y's.  Every one of them is then earlier than every query
      of B, which is exactly B's full view of X, and Y keeps its true
      positions for the causal mask.  When j < rank, B takes X alone.

    The first launch (j = rank) writes the running state; every later one
    merges into it.
    """

    def __init__(self, layout: ZigzagLayout, rank: int, scale: float = 0.0):
        if not 0 <= rank < layout.n:
            raise ValueError("rank outside the ring")
        self.layout, self.rank, self.scale = layout, rank, scale

    def step_keys(self, j: int):
        """Per query segment (A, B per sequence): the key range and its first position at the
        step that holds device j's pair, as (k_row0, k_len, k_pos0) lists."""
        lay, r = self.layout, self.rank
        cu = lay.cu()
        kpos = lay.positions(j)
        k_row0, k_len, k_pos0 = [], [], []
        for b, c in enumerate(lay.chunk_lens):
            x0, px, py = cu[2 * b], kpos[2 * b], kpos[2 * b + 1]
            k_row0 += [x0, x0]
            if j >= r:
                k_len += [c if j == r else 0, 2 * c]
                k_pos0 += [px, py - c]
            else:
                k_len += [c, c]
                k_pos0 += [px, px]
        return k_row0, k_len, k_pos0

    def prepare(self, q_local, kv_pairs, o, lse, stream=None) -> "PreparedCalls":
        lay, r = self.layout, self.rank
        cu = lay.cu()
        q_pos0 = lay.positions(r)
        calls = []
        for t in range(lay.n):
            j = (r - t) % lay.n
            k_j, v_j = kv_pairs[j]
            k_row0, k_len, k_pos0 = self.step_keys(j)
            args = dict(cu_q=cu, q_pos0=q_pos0, k_row0=k_row0, k_len=k_len, k_pos0=k_pos0,
                        scale=self.scale, causal=True, stream=stream)
            if t == 0:
                calls.append(_native.prepare_ring_step(q_local, k_j, v_j, o, lse, report_skip=False,
                                                       **args))
            else:
                calls.append(_native.prepare_ring_step_merge(q_local, k_j, v_j, o, lse, **args))
        return PreparedCalls(calls, stream)

    def run(self, q_local, kv_pairs, o, lse, stream=None, events=None) -> int:
        return self.prepare(q_local, kv_pairs, o, lse, stream).run(events=events)


class PreparedCalls:
    """A fixed sequence of prepared launches; ``run`` enqueues them in order and
    returns how many launched (a fully masked merge launches nothing)."""

    def __init__(self, calls, stream):
        self.calls, self.stream = calls, stream

    def run(self, events=None, event_pool=None) -> int:
        timed = _EventTimer(events, self.stream, event_pool)
        active = 0
        for call in self.calls:
            with timed("step") as mark:
                launched = call()
                mark(launched)
            active += bool(launched)
        return active


class ChunkedPrefill:
    """Chunked prefill of chunk ``index`` of every sequence: its queries attend
    causally to the whole prefix (chunks 0..index) in one launch - full key
    blocks plus a diagonal block, the same step kernel as the ring.  The result
    is final (it equals full causal attention for those rows), so no merge is
    needed.  SGLang's pipeline-parallel prefill runs prompts in such chunks
    (chunked prefill size 12K in the pages' PP evaluation).
    """

    def __init__(self, layout: RingLayout, index: int, scale: float = 0.0):
        if not 0 <= index < layout.n_chunks:
            raise ValueError("chunk index outside the prompt")
        self.layout, self.index, self.scale = layout, index, scale

    def prepare(self, q_chunk, k_prefix, v_prefix, o, lse, stream=None):
        lay = self.layout
        return _native.prepare_ring_step(
            q_chunk, k_prefix, v_prefix, o, lse, cu_q=lay.cu, cu_k=lay.prefix_cu(self.index),
            q_pos0=lay.pos0(self.index), k_pos0=[0] * len(lay.seqlens), scale=self.scale,
            causal=True, report_skip=False, stream=stream)

    def run(self, q_chunk, k_prefix, v_prefix, o, lse, stream=None) -> None:
        self.prepare(q_chunk, k_prefix, v_prefix, o, lse, stream)()


class PreparedRing:
    """The calls of one ring, marshalled; ``run`` enqueues the whole ring."""

    def __init__(self, steps, identity, stream):
        self.steps, self.identity, self.stream = steps, identity, stream

    def run(self, events=None, event_pool=None) -> int:
        """Enqueue the ring; returns the number of steps that launched work.

        ``events``/``event_pool`` as in ``RingAttention.run``; with a pool
        (a list of timing-enabled events) the events are taken from it
        instead of created per launch.
        """
        timed = _EventTimer(events, self.stream, event_pool)
        wrote_state = False
        active = 0
        for write, fold, merge in self.steps:
            with timed("step") as mark:
                launched = fold() if wrote_state else write()
                mark(launched)
            if not launched:
                continue
            active += 1
            if wrote_state and merge is not None:
                with timed("merge") as mark:
                    merge()
                    mark(True)
            wrote_state = True
        if not wrote_state:  # every chunk was in the future: the state is the identity
            self.identity()
        return active


class _EventTimer:
    """Context manager factory recording HIP events around launches (no-op without a list)."""

    def __init__(self, sink, stream, pool=None):
        self.sink = sink
        self.stream = stream
        self.pool = pool

    def event(self):
        if self.pool:
            return self.pool.pop()
        return torch.cuda.Event(enable_timing=True)

    def __call__(self, kind):
        return _EventSpan(self, kind)


class _EventSpan:
    def __init__(self, timer, kind):
        self.timer, self.kind = timer, kind
        self.keep = False
        self.start = None

    def __enter__(self):
        if self.timer.sink is not None:
            self.start = self.timer.event()
            self.start.record(self.timer.stream)
        return self._mark

    def _mark(self, launched):
        self.keep = bool(launched)

    def __exit__(self, *exc):
        if self.timer.sink is not None and self.keep and exc[0] is None:
            end = self.timer.event()
            end.record(self.timer.stream)
            self.timer.sink.append((self.kind, self.start, end))
        return False
