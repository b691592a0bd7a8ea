"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, and rejects invalid arguments on the host before any HIP call.

The invalid-argument cases pass placeholder (never dereferenced) pointers, so
they only run on hosts without a visible GPU; ``test_gpu_parity.py`` repeats
the error paths with real device buffers.
"""

import ctypes
import math
import os
import re

import pytest
import torch

from ring_attention_03_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnring.h")

no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="placeholder pointers must never reach a real GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_native.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _native.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.attn_abi_version() == _native.ABI_VERSION == 3
    assert lib.attn_last_error() is not None


def test_problem_struct_layout_matches_header():
    # 4 pointers after an int32 (padded), 7 int32/float fields (padded), 2 pointers: checks
    # ctypes mirrors the C struct
    assert ctypes.sizeof(_native.AttnProblem) == 8 + 4 * 8 + 7 * 4 + 4 + 2 * 8
    assert _native.AttnProblem.total_q.offset == 40
    assert _native.AttnProblem.k_row0.offset == 72 and _native.AttnProblem.k_len.offset == 80


FAKE = 1 << 32  # 16-byte aligned placeholder address, never dereferenced on the host
# (multiples of FAKE are 4 GiB apart, so placeholder buffers never overlap)


def _prob(**kw):
    base = dict(num_seqs=1, total_q=128, total_k=128, num_q_heads=8, num_kv_heads=1, head_dim=64,
                scale=0.0, causal=1)
    base.update(kw)
    arrays = {}
    p = _native.AttnProblem()
    for key, val in base.items():
        if key in ("cu_q", "cu_k", "q_pos0", "k_pos0", "k_row0", "k_len"):
            arr = (ctypes.c_int32 * len(val))(*val)
            arrays[key] = arr
            setattr(p, key, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
        else:
            setattr(p, key, val)
    return p, arrays


def _step(p, dtype=0, ptrs=None, launched=True):
    lib = _native.load_library()
    q, k, v, o, lse = ptrs or (FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5)
    flag = ctypes.c_int32(-1)
    st = lib.attn_ring_step(ctypes.byref(p), dtype, q, k, v, o, lse,
                            ctypes.byref(flag) if launched else None, None)
    return st, flag.value, lib.attn_last_error().decode()


@no_gpu_only
@pytest.mark.parametrize("kw,expect,needle", [
    (dict(num_seqs=0), 1, "num_seqs"),
    (dict(num_seqs=65), 1, "num_seqs"),
    (dict(num_q_heads=6, num_kv_heads=4), 1, "multiple"),
    (dict(num_kv_heads=0), 1, "head counts"),
    (dict(head_dim=128), 2, "head_dim"),
    (dict(head_dim=0), 1, "head_dim"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(scale=math.inf), 1, "scale"),
    (dict(causal=2), 1, "causal"),
    (dict(total_q=-1), 1, "negative"),
    (dict(num_seqs=2), 1, "cu_q is NULL"),
    (dict(num_seqs=2, cu_q=[0, 100, 90], cu_k=[0, 64, 128]), 1, "non-decreasing"),
    (dict(num_seqs=2, cu_q=[1, 64, 128], cu_k=[0, 64, 128]), 1, "cu_q[0]"),
    (dict(num_seqs=2, cu_q=[0, 64, 127], cu_k=[0, 64, 128]), 1, "total"),
    (dict(q_pos0=[-3]), 1, "negative"),
    (dict(k_pos0=[2**31 - 10]), 1, "overflow"),
    # bf16 keys of one sequence: 2**21 rows x 8 heads x 64 x 2 B = 2 GiB
    (dict(total_k=2**21, num_q_heads=8, num_kv_heads=8, causal=0), 2, "2 GiB"),
    # explicit key ranges
    (dict(k_row0=[0]), 1, "together"),
    (dict(k_len=[10]), 1, "together"),
    (dict(k_row0=[0], k_len=[10], cu_k=[0, 128]), 1, "not both"),
    (dict(k_row0=[-1], k_len=[10]), 1, ">= 0"),
    (dict(k_row0=[100], k_len=[29]), 1, "past total_k"),
    (dict(num_seqs=2, cu_q=[0, 64, 128], k_row0=[0, 0], k_len=[128, 129]), 1, "past total_k"),
    (dict(k_row0=[0], k_len=[10], k_pos0=[2**31 - 5]), 1, "overflow"),
])
def test_invalid_problem_is_rejected_before_launch(kw, expect, needle):
    p, keep = _prob(**kw)
    st, launched, msg = _step(p)
    assert st == expect, msg
    assert needle in msg
    assert launched == 0
    del keep


@no_gpu_only
def test_explicit_key_ranges_may_overlap_and_prefill_refuses_them():
    # two query sequences attending to the same 64 keys (overlapping ranges) is valid:
    # with every key in the future of every query nothing is enqueued (no GPU needed)
    p, keep = _prob(num_seqs=2, cu_q=[0, 64, 128], k_row0=[0, 0], k_len=[64, 64],
                    q_pos0=[0, 64], k_pos0=[500, 500])
    st, launched, msg = _step(p)
    assert st == 0 and launched == 0, msg
    lib = _native.load_library()
    p, keep = _prob(k_row0=[0], k_len=[128])
    assert lib.attn_prefill_causal(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4,
                                   FAKE * 5, None) == 1
    assert "k_row0" in lib.attn_last_error().decode()
    del keep


@no_gpu_only
def test_step_merge_validates_like_the_step():
    lib = _native.load_library()

    def call(p, ptrs=(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5)):
        flag = ctypes.c_int32(-1)
        st = lib.attn_ring_step_merge(ctypes.byref(p), 0, *ptrs, ctypes.byref(flag), None)
        return st, flag.value, lib.attn_last_error().decode()

    p, keep = _prob(num_kv_heads=3)
    st, launched, msg = call(p)
    assert st == 1 and launched == 0 and "multiple" in msg
    p, keep = _prob(head_dim=128)
    assert call(p)[0] == 2
    p, keep = _prob()
    st, _, msg = call(p, ptrs=(FAKE, FAKE * 100, FAKE * 200, FAKE + 64, FAKE * 300))
    assert st == 1 and "overlap" in msg
    # a block wholly in the future: valid, nothing to merge, nothing enqueued
    p, keep = _prob(q_pos0=[0], k_pos0=[1000])
    st, launched, _ = call(p)
    assert st == 0 and launched == 0
    del keep


@no_gpu_only
def test_invalid_pointers_are_rejected():
    p, keep = _prob()
    assert _step(p, ptrs=(None, FAKE, FAKE * 2, FAKE * 3, FAKE * 4))[0] == 1
    assert _step(p, ptrs=(FAKE + 2, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5))[0] == 1  # misaligned q
    assert _step(p, ptrs=(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 4 + 1))[0] == 1  # misaligned lse
    # o overlapping q
    st, _, msg = _step(p, ptrs=(FAKE, FAKE * 100, FAKE * 200, FAKE + 64, FAKE * 300))
    assert st == 1 and "overlap" in msg
    assert _step(p, dtype=7)[0] == 1
    del keep


@no_gpu_only
def test_fully_masked_step_enqueues_nothing():
    # keys at positions 200.. are all in the future of query positions 0..127
    p, keep = _prob(q_pos0=[0], k_pos0=[200])
    st, launched, msg = _step(p)
    assert st == 0, msg
    assert launched == 0
    # no local rows: nothing to do either
    p2, keep2 = _prob(total_q=0)
    assert _step(p2)[:2] == (0, 0)
    del keep, keep2


@no_gpu_only
def test_prefill_and_merge_validation():
    lib = _native.load_library()
    p, keep = _prob(causal=0)
    assert lib.attn_prefill_causal(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4,
                                   FAKE * 5, None) == 1
    p, keep = _prob(total_k=64)
    assert lib.attn_prefill_causal(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4,
                                   FAKE * 5, None) == 1
    p, keep = _prob(num_seqs=2, cu_q=[0, 64, 128], cu_k=[0, 60, 128])
    assert lib.attn_prefill_causal(ctypes.byref(p), 0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4,
                                   FAKE * 5, None) == 1
    assert lib.attn_ring_merge(16, 4, 64, FAKE, FAKE * 2, FAKE, FAKE * 3, None) == 1  # aliasing
    assert "overlap" in lib.attn_last_error().decode()
    assert lib.attn_ring_merge(16, 4, 32, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None) == 2
    assert lib.attn_ring_merge(-1, 4, 64, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None) == 1
    assert lib.attn_ring_merge(0, 4, 64, None, None, None, None, None) == 0  # nothing to do
    del keep


def test_probe_library_is_built_apart_from_the_abi():
    # the matrix-core probe used by bench.py lives in its own library, so the
    # attention library exports exactly the declared ABI
    import os

    probe = os.path.join(os.path.dirname(_native.__file__), "libattnprobe.so")
    lib = ctypes.CDLL(probe)
    assert hasattr(lib, "attn_probe_mfma")
    assert not hasattr(_native.load_library(), "attn_probe_mfma")
