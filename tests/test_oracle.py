"""Pins of the fp64 oracle against things other than itself (CPU only).

Every check here is fixed by mathematics or by an independent routine, not by
the oracle's own formula: a hand-worked example, torch's CPU scaled
dot-product attention, a pure-Python brute force, closed forms and exact
invariants of softmax.  A dropped term, a wrong sign, a transposed operand or
a wrong head/position index in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention_ref, causal_attention_ref, chunk_layout_ref, merge_ref,
                    ring_ref, visible_pairs_ref)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ----------------------------------------------------------------------------- hand example
def test_golden_hand_example():
    with open(os.path.join(GOLDEN, "causal_3x2_hand.json")) as f:
        g = json.load(f)
    q = np.array(g["q"])
    k = np.zeros((3, 1, 2))
    k[:, 0, 0] = np.log(np.array(g["k_log_arg"], dtype=float))
    v = np.array(g["v"])
    o, lse = causal_attention_ref(q, k, v, scale=g["scale"])
    np.testing.assert_allclose(o, np.array(g["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], np.log(np.array(g["lse_exp_arg"], dtype=float)),
                               rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- library routine
def _torch_reference(q, k, v, scale):
    """torch CPU fp64 SDPA with K/V heads repeated per group, plus logsumexp of the masked scores."""
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, T, d]
    group = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    t = q.shape[0]
    mask = torch.ones(t, t, dtype=torch.bool).tril()
    scores = torch.matmul(qt, kt.transpose(1, 2)) * scale
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.numpy()


@pytest.mark.parametrize("hq,hkv,t,d", [(4, 1, 37, 16), (6, 2, 50, 8), (3, 3, 21, 64)])
def test_matches_torch_sdpa(hq, hkv, t, d):
    q, k, v = rand((t, hq, d), 1), rand((t, hkv, d), 2), rand((t, hkv, d), 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = causal_attention_ref(q, k, v)
    o_t, lse_t = _torch_reference(q, k, v, scale)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-12)


def test_explicit_scale_is_used():
    q, k, v = rand((9, 2, 4), 4), rand((9, 1, 4), 5), rand((9, 1, 4), 6)
    o, lse = causal_attention_ref(q, k, v, scale=0.37)
    o_t, lse_t = _torch_reference(q, k, v, 0.37)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- brute force
def _brute(q, k, v, cu_q, cu_k, qp0, kp0, scale, causal):
    tq, hq, d = len(q), len(q[0]), len(q[0][0])
    hkv = len(k[0])
    o = [[[0.0] * d for _ in range(hq)] for _ in range(tq)]
    lse = [[-math.inf] * tq for _ in range(hq)]
    for b in range(len(cu_q) - 1):
        for i in range(cu_q[b], cu_q[b + 1]):
            pq = qp0[b] + i - cu_q[b]
            for h in range(hq):
                g = (h * hkv) // hq
                scores = []
                for j in range(cu_k[b], cu_k[b + 1]):
                    pk = kp0[b] + j - cu_k[b]
                    if causal and pk > pq:
                        continue
                    s = scale * sum(q[i][h][x] * k[j][g][x] for x in range(d))
                    scores.append((s, j))
                if not scores:
                    continue
                total = sum(math.exp(s) for s, _ in scores)
                lse[h][i] = math.log(total)
                for s, j in scores:
                    w = math.exp(s) / total
                    for x in range(d):
                        o[i][h][x] += w * v[j][g][x]
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_brute_force_varlen_positions(causal):
    cu_q, cu_k = [0, 3, 8, 9], [0, 4, 6, 11]
    qp0, kp0 = [5, 2, 0], [3, 4, 0]
    hq, hkv, d = 4, 2, 3
    q, k, v = rand((9, hq, d), 7), rand((11, hkv, d), 8), rand((11, hkv, d), 9)
    o, lse = attention_ref(q, k, v, cu_q=cu_q, cu_k=cu_k, q_pos0=qp0, k_pos0=kp0,
                           scale=0.6, causal=causal)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), cu_q, cu_k, qp0, kp0, 0.6, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)
    if causal:  # sequence 1: query positions 2..6 against key positions 4..5 - rows 0,1 see nothing
        assert np.isneginf(lse[:, 3]).all() and np.isneginf(lse[:, 4]).all()
        assert (o[3:5] == 0).all()


def test_row_subset_is_exact():
    q, k, v = rand((40, 4, 8), 10), rand((40, 2, 8), 11), rand((40, 2, 8), 12)
    o, lse = causal_attention_ref(q, k, v, seqlens=[15, 25])
    rows = [0, 3, 14, 15, 16, 39]
    o_s, lse_s = causal_attention_ref(q, k, v, seqlens=[15, 25], rows=rows)
    np.testing.assert_array_equal(o_s, o[rows])
    np.testing.assert_array_equal(lse_s, lse[:, rows])


# ----------------------------------------------------------------------------- closed forms
def test_zero_query_gives_prefix_mean():
    t, d = 12, 5
    q = np.zeros((t, 2, d))
    k, v = rand((t, 1, d), 13), rand((t, 1, d), 14)
    o, lse = causal_attention_ref(q, k, v)
    for p in range(t):
        np.testing.assert_allclose(o[p, :, :], np.broadcast_to(v[: p + 1, 0].mean(0), (2, d)),
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, p], math.log(p + 1), rtol=0, atol=1e-13)


def test_first_row_and_uniform_v():
    t, d = 10, 6
    q, k = rand((t, 3, d), 15), rand((t, 1, d), 16)
    v = np.broadcast_to(rand((1, 1, d), 17), (t, 1, d)).copy()
    o, lse = causal_attention_ref(q, k, v, scale=0.5)
    np.testing.assert_allclose(o, np.broadcast_to(v[0, 0], o.shape), rtol=0, atol=1e-13)
    for h in range(3):
        np.testing.assert_allclose(lse[h, 0], 0.5 * q[0, h] @ k[0, 0], rtol=0, atol=1e-13)


def test_probabilities_sum_to_one_and_match_softmax():
    # One-hot V (d = T) turns each output row into the row of attention weights.
    t = 11
    q, k = rand((t, 2, t), 18), rand((t, 1, t), 19)
    v = np.eye(t).reshape(t, 1, t)
    o, lse = causal_attention_ref(q, k, v, scale=0.3)
    np.testing.assert_allclose(o.sum(-1), 1.0, rtol=0, atol=1e-12)
    for p in range(t):
        for h in range(2):
            s = 0.3 * (k[: p + 1, 0] @ q[p, h])
            w = np.exp(s - s.max())
            w /= w.sum()
            np.testing.assert_allclose(o[p, h, : p + 1], w, rtol=0, atol=1e-13)
            assert (o[p, h, p + 1:] == 0).all()  # no weight on future keys


def test_shift_invariance():
    # Append a coordinate so every score of query row p grows by c_p: O unchanged, LSE + c_p.
    t, d = 9, 4
    q, k, v = rand((t, 2, d), 20), rand((t, 1, d), 21), rand((t, 1, d), 22)
    c = rand((t, 2), 23) * 3
    q2 = np.concatenate([q, c[:, :, None]], axis=2)
    k2 = np.concatenate([k, np.ones((t, 1, 1))], axis=2)
    v2 = np.concatenate([v, np.zeros((t, 1, 1))], axis=2)
    o, lse = causal_attention_ref(q, k, v, scale=1.0)
    o2, lse2 = causal_attention_ref(q2, k2, v2, scale=1.0)
    np.testing.assert_allclose(o2[:, :, :d], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + c.T, rtol=0, atol=1e-12)


def test_large_scores_stay_finite():
    t, d = 64, 64
    q, k, v = rand((t, 4, d), 24, 30.0), rand((t, 1, d), 25), rand((t, 1, d), 26)
    o, lse = causal_attention_ref(q, k, v)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    o_t, lse_t = _torch_reference(q, k, v, 1.0 / 8.0)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, lse_t, rtol=1e-13, atol=1e-9)


# ----------------------------------------------------------------------------- merge and ring
def test_merge_identity_commutative_associative():
    t, h, d = 7, 3, 4
    parts = []
    for s in range(3):
        o = rand((t, h, d), 30 + s)
        lse = rand((h, t), 40 + s)
        lse[0, s] = -np.inf
        o[s, 0] = 0.0
        parts.append((o, lse))
    zero = (np.zeros((t, h, d)), np.full((h, t), -np.inf))
    o, lse = merge_ref(*zero, *parts[0])
    np.testing.assert_array_equal(o, parts[0][0])
    np.testing.assert_array_equal(lse, parts[0][1])
    ab = merge_ref(*parts[0], *parts[1])
    ba = merge_ref(*parts[1], *parts[0])
    np.testing.assert_allclose(ab[0], ba[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], rtol=0, atol=1e-14)
    left = merge_ref(*ab, *parts[2])
    right = merge_ref(*parts[0], *merge_ref(*parts[1], *parts[2]))
    np.testing.assert_allclose(left[0], right[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], rtol=0, atol=1e-13)
    both_empty = merge_ref(*zero, *zero)
    assert (both_empty[0] == 0).all() and np.isneginf(both_empty[1]).all()


def test_merge_closed_forms():
    # Two copies of the same partial are the same keys twice: the weights stay
    # the same (O unchanged) and the normaliser doubles (LSE + ln 2).  Partials
    # whose LSEs differ by ln 3 weigh 3:1.  Huge LSEs must not overflow.
    o, lse = rand((5, 2, 4), 60), rand((2, 5), 61)
    m_o, m_l = merge_ref(o, lse, o, lse)
    np.testing.assert_allclose(m_o, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(m_l, lse + math.log(2.0), rtol=0, atol=1e-14)
    o2 = rand((5, 2, 4), 62)
    big = np.full((2, 5), 800.0)
    m_o, m_l = merge_ref(o, big + math.log(3.0), o2, big)
    # (LSEs of 800 carry ~800 * 2^-53 = 1e-13 of rounding into the weights' exponents)
    np.testing.assert_allclose(m_o, 0.75 * o + 0.25 * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m_l, big + math.log(4.0), rtol=0, atol=1e-12)


def test_merge_of_disjoint_key_sets_is_full_softmax():
    # Split the keys of a non-causal problem into two sets: the merge must equal the whole.
    q, k, v = rand((6, 2, 5), 50), rand((10, 1, 5), 51), rand((10, 1, 5), 52)
    full = attention_ref(q, k, v, causal=False)
    a = attention_ref(q, k[:4], v[:4], causal=False)
    b = attention_ref(q, k[4:], v[4:], causal=False)
    m = merge_ref(*a, *b)
    np.testing.assert_allclose(m[0], full[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(m[1], full[1], rtol=0, atol=1e-13)


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_ring_equals_unchunked_every_rank(n):
    seqlens = [64, 32]
    q, k, v = rand((96, 4, 8), 60), rand((96, 2, 8), 61), rand((96, 2, 8), 62)
    full_o, full_lse = causal_attention_ref(q, k, v, seqlens)
    got_o = np.zeros_like(full_o)
    got_lse = np.zeros_like(full_lse)
    for r in range(n):
        rows, _, _ = chunk_layout_ref(seqlens, n, r)
        o, lse = ring_ref(q, k, v, seqlens, n, r)
        got_o[rows] = o
        got_lse[:, rows] = lse
    np.testing.assert_allclose(got_o, full_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got_lse, full_lse, rtol=0, atol=1e-12)


def test_ring_split_and_resume():
    seqlens, n, r = [48], 4, 3
    q, k, v = rand((48, 2, 4), 63), rand((48, 1, 4), 64), rand((48, 1, 4), 65)
    whole = ring_ref(q, k, v, seqlens, n, r)
    first = ring_ref(q, k, v, seqlens, n, r, steps=[0, 1])
    second = ring_ref(q, k, v, seqlens, n, r, steps=[2, 3])
    resumed = merge_ref(*first, *second)
    np.testing.assert_allclose(resumed[0], whole[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(resumed[1], whole[1], rtol=0, atol=1e-13)


def test_ring_mutations_are_caught():
    seqlens, n, r = [64], 4, 3
    q, k, v = rand((64, 2, 4), 66), rand((64, 1, 4), 67), rand((64, 1, 4), 68)
    rows, _, _ = chunk_layout_ref(seqlens, n, r)
    target = causal_attention_ref(q, k, v, seqlens, rows=rows)

    def err(steps):
        o, lse = ring_ref(q, k, v, seqlens, n, r, steps=steps)
        return max(np.abs(o - target[0]).max(), np.abs(lse - target[1]).max())

    assert err([0, 1, 2, 3]) < 1e-12
    assert err([3, 1, 0, 2]) < 1e-12      # order changes only rounding
    assert err([0, 1, 3]) > 1e-2          # a dropped step is visible
    assert err([0, 1, 1, 2, 3]) > 1e-2    # so is a repeated one


def test_gqa_equals_repeated_heads():
    q, k, v = rand((20, 8, 4), 70), rand((20, 2, 4), 71), rand((20, 2, 4), 72)
    gqa = causal_attention_ref(q, k, v)
    mha = causal_attention_ref(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    np.testing.assert_array_equal(gqa[0], mha[0])
    np.testing.assert_array_equal(gqa[1], mha[1])


def test_varlen_packed_equals_separate_and_isolated():
    seqlens = [7, 12, 5]
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    q, k, v = rand((24, 2, 4), 73), rand((24, 1, 4), 74), rand((24, 1, 4), 75)
    packed = causal_attention_ref(q, k, v, seqlens)
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        sep = causal_attention_ref(q[sl], k[sl], v[sl])
        np.testing.assert_array_equal(packed[0][sl], sep[0])
        np.testing.assert_array_equal(packed[1][:, sl], sep[1])
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 5.0
    v2[cu[1]:cu[2]] -= 3.0
    moved = causal_attention_ref(q, k2, v2, seqlens)
    for b in (0, 2):
        sl = slice(cu[b], cu[b + 1])
        np.testing.assert_array_equal(moved[0][sl], packed[0][sl])
        np.testing.assert_array_equal(moved[1][:, sl], packed[1][:, sl])
    assert not np.array_equal(moved[0][cu[1]:cu[2]], packed[0][cu[1]:cu[2]])


def test_chunk_layout_and_pair_count():
    rows, cu, pos0 = chunk_layout_ref([8, 4], 4, 2)
    assert rows.tolist() == [4, 5, 10]
    assert cu.tolist() == [0, 2, 3] and pos0.tolist() == [4, 2]
    for seqlens, n in [([12], 3), ([8, 16], 4), ([6], 1)]:
        brute_total = sum(p + 1 for s in seqlens for p in range(s))
        assert visible_pairs_ref(seqlens) == brute_total
        assert sum(visible_pairs_ref(seqlens, n, r) for r in range(n)) == brute_total
    # closed forms for the long workloads: rank r of N chunks of c sees r*c*c + c*(c+1)/2
    # pairs (65536/8 rank 7: 7*8192^2 + 8192*8193/2); a whole prompt S sees S*(S+1)/2
    assert visible_pairs_ref([65536], 8, 7) == 503_320_576
    assert visible_pairs_ref([32768], 8, 3) == 58_722_304
    assert visible_pairs_ref([102400]) == 5_242_931_200
    assert 7 * 8192 ** 2 + 8192 * 8193 // 2 == 503_320_576 and 102400 * 102401 // 2 == 5_242_931_200
