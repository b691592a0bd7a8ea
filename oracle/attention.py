"""Plain fp64 definition of causal GQA attention, its LSE merge and the ring.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

Source of each function
-----------------------
Moreh, "Optimizing Long-Context Prefill on Multiple Older-Generation GPU
Nodes", section "Introduction to Context Parallelism":

* ``attention_ref``: the attention each device runs on its partial query and
  key/value blocks (Ring Attention bullet).  The pages print no formula, so
  this is the textbook definition of scaled dot-product attention with a
  causal mask, evaluated in fp64 with an explicit, whole-row softmax:

      s[p, k]  = scale * <q[p, h], k[k, g]>          g = h // (Hq / Hkv)
      V(p)     = keys k of p's sequence with position(k) <= position(p)
      LSE[h,p] = m + ln( sum_{k in V(p)} exp(s[p,k] - m) ),  m = max_{V(p)} s
      O[p, h]  = sum_{k in V(p)} exp(s[p,k] - LSE[h,p]) * v[k, g]

  A row whose visible set is empty (a key block that lies wholly in the
  row's future) gives O = 0 and LSE = -inf, the identity of the merge.
* ``merge_ref``: combining the partial results of two disjoint key blocks.
  Softmax over a disjoint union of key sets splits exactly this way, which is
  what lets the partial results add up to full attention.
* ``ring_ref``: the ring itself - each device keeps its query block while the
  key/value blocks travel around the ring of neighbours; at step t device r
  holds the block that started on device (r - t) mod N.
* ``chunk_layout_ref``: the context-parallel split along the sequence
  dimension (the paragraph introducing context parallelism), read as
  contiguous, equal chunks of every sequence.

Readings where the pages are silent (each one is listed with its reason in
the design notes): scale defaults to 1/sqrt(head_dim); query head h uses
key/value head h // (Hq/Hkv) (consecutive groups); causality is decided by
global token positions; LSE is a natural log laid out [Hq, T].

Layouts: q is [Tq, Hq, d]; k and v are [Tk, Hkv, d]; several sequences may be
packed along the token axis, described by prefix offsets ``cu_q`` / ``cu_k``
and the global position of each sequence's first row ``q_pos0`` / ``k_pos0``.
Inputs of any float dtype are upcast to float64 before use, so the oracle sees
exactly the values the device is given.
"""

from __future__ import annotations

import math

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Return ``x`` as a float64 numpy array (accepts numpy arrays or CPU torch tensors)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32 so bf16 is upcast exactly
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def _offsets(cu, total: int) -> np.ndarray:
    if cu is None:
        return np.array([0, total], dtype=np.int64)
    return np.asarray(cu, dtype=np.int64)


def attention_ref(q, k, v, *, cu_q=None, cu_k=None, q_pos0=None, k_pos0=None,
                  scale: float | None = None, causal: bool = True, rows=None):
    """Causal (or unmasked) GQA attention of packed query rows against packed key rows.

    Returns ``(O, LSE)`` in float64: ``O`` is [R, Hq, d] and ``LSE`` is [Hq, R]
    where R is ``Tq`` or ``len(rows)`` when a subset of query rows is asked for
    (each row depends only on its own query and the keys, so a subset is exact).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    assert v.shape == k.shape and dk == d, "k and v must both be [Tk, Hkv, d]"
    assert hq % hkv == 0, "query heads must be a multiple of key/value heads"
    group = hq // hkv
    cq, ck = _offsets(cu_q, tq), _offsets(cu_k, tk)
    nseq = len(cq) - 1
    assert len(ck) == nseq + 1 and cq[-1] == tq and ck[-1] == tk
    qp0 = np.zeros(nseq, np.int64) if q_pos0 is None else np.asarray(q_pos0, np.int64)
    kp0 = np.zeros(nseq, np.int64) if k_pos0 is None else np.asarray(k_pos0, np.int64)
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)

    rows = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), hq, d), dtype=np.float64)
    lse = np.full((hq, len(rows)), -np.inf, dtype=np.float64)

    for b in range(nseq):
        # which requested rows belong to sequence b, and where they go in the output
        sel = np.nonzero((rows >= cq[b]) & (rows < cq[b + 1]))[0]
        if len(sel) == 0 or ck[b + 1] == ck[b]:
            continue
        local = rows[sel] - cq[b]
        qpos = qp0[b] + local                      # global positions of these query rows
        kpos = kp0[b] + np.arange(ck[b + 1] - ck[b])  # global positions of the keys
        if causal:
            visible = kpos[None, :] <= qpos[:, None]
        else:
            visible = np.ones((len(sel), len(kpos)), dtype=bool)
        has_any = visible.any(axis=1)
        for h in range(hq):
            g = h // group
            qh = q[cq[b] + local, h, :]                # [n, d]
            kg = k[ck[b]:ck[b + 1], g, :]              # [Lk, d]
            vg = v[ck[b]:ck[b + 1], g, :]              # [Lk, d]
            s = scale * (qh @ kg.T)                    # [n, Lk]
            s = np.where(visible, s, -np.inf)
            m = np.where(has_any, s.max(axis=1), 0.0)  # any finite shift works for empty rows
            with np.errstate(divide="ignore"):
                row_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
            row_lse = np.where(has_any, row_lse, -np.inf)
            p = np.where(visible, np.exp(s - np.where(has_any, row_lse, 0.0)[:, None]), 0.0)
            out[sel, h, :] = p @ vg
            lse[h, sel] = row_lse
    return out, lse


def merge_ref(o_a, lse_a, o_b, lse_b):
    """Combine the partial results of two disjoint key sets.

    With M = max(La, Lb):  L = M + ln(e^(La-M) + e^(Lb-M)),
    O = e^(La-L) * Oa + e^(Lb-L) * Ob.  (0, -inf) is the identity; two empty
    partials merge to (0, -inf).  O is [T, Hq, d], LSE is [Hq, T].
    """
    o_a, o_b = _as_f64(o_a), _as_f64(o_b)
    la, lb = _as_f64(lse_a), _as_f64(lse_b)
    mx = np.maximum(la, lb)
    empty = np.isneginf(mx)
    mx_safe = np.where(empty, 0.0, mx)
    with np.errstate(divide="ignore"):
        lse = mx_safe + np.log(np.exp(la - mx_safe) + np.exp(lb - mx_safe))
    lse = np.where(empty, -np.inf, lse)
    lse_safe = np.where(empty, 0.0, lse)
    wa = np.where(empty, 0.0, np.exp(la - lse_safe))  # [Hq, T]
    wb = np.where(empty, 0.0, np.exp(lb - lse_safe))
    out = wa.T[:, :, None] * o_a + wb.T[:, :, None] * o_b
    return out, lse


def chunk_layout_ref(seqlens, n_chunks: int, chunk: int):
    """Rows of chunk ``chunk`` when every sequence is cut into ``n_chunks`` equal contiguous parts.

    Returns ``(rows, cu, pos0)``: the packed global row indices of the chunk
    (sequences packed back to back in the order given), the prefix offsets of
    the chunk's packed form, and each sequence's first global position in it.
    """
    rows, cu, pos0 = [], [0], []
    start = 0
    for n in seqlens:
        assert n % n_chunks == 0, "each sequence must split into equal chunks"
        c = n // n_chunks
        rows.append(np.arange(start + chunk * c, start + (chunk + 1) * c))
        cu.append(cu[-1] + c)
        pos0.append(chunk * c)
        start += n
    return np.concatenate(rows), np.array(cu), np.array(pos0)


def causal_attention_ref(q, k, v, seqlens=None, *, scale=None, rows=None):
    """Full causal attention over whole packed sequences (no chunking): the ring's target."""
    q = _as_f64(q)
    seqlens = [q.shape[0]] if seqlens is None else list(seqlens)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    return attention_ref(q, k, v, cu_q=cu, cu_k=cu, scale=scale, causal=True, rows=rows)


def ring_ref(q, k, v, seqlens, n_chunks: int, rank: int, *, scale=None, rows=None,
             steps=None):
    """Result of device ``rank`` after the ring, from full packed q/k/v.

    Device ``rank`` keeps query chunk ``rank``; at ring step t it holds the
    key/value chunk that started on device (rank - t) mod N, runs attention
    on it and folds the partial result into its running (O, LSE) with
    ``merge_ref``, starting from the identity (0, -inf).  ``steps`` may list
    the step indices to run (default: all N, in order) so that tests can
    drop, repeat or reorder steps.  ``rows`` picks a subset of the device's
    local rows.  Returns (O [R, Hq, d], LSE [Hq, R]) over local rows.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    qrows, cu_q, q_pos0 = chunk_layout_ref(seqlens, n_chunks, rank)
    q_local = q[qrows]
    nrows = len(qrows) if rows is None else len(rows)
    o = np.zeros((nrows, q.shape[1], q.shape[2]))
    lse = np.full((q.shape[1], nrows), -np.inf)
    for t in (range(n_chunks) if steps is None else steps):
        j = (rank - t) % n_chunks
        krows, cu_k, k_pos0 = chunk_layout_ref(seqlens, n_chunks, j)
        o_p, lse_p = attention_ref(q_local, k[krows], v[krows], cu_q=cu_q, cu_k=cu_k,
                                   q_pos0=q_pos0, k_pos0=k_pos0, scale=scale,
                                   causal=True, rows=rows)
        o, lse = merge_ref(o, lse, o_p, lse_p)
    return o, lse


def visible_pairs_ref(seqlens, n_chunks: int = 1, rank: int | None = None) -> int:
    """Number of (query, key) token pairs with key position <= query position.

    With ``rank`` given, counts only the pairs whose query lies in that
    device's chunk.  Used to count algorithmic work: 4 * d * Hq flops per pair
    (2d for the score dot product, 2d for the weighted sum of values).
    """
    total = 0
    for n in seqlens:
        if rank is None:
            total += n * (n + 1) // 2
        else:
            c = n // n_chunks
            lo, hi = rank * c, (rank + 1) * c  # query positions lo..hi-1 see keys 0..p
            total += (hi * (hi + 1) - lo * (lo + 1)) // 2
    return total
