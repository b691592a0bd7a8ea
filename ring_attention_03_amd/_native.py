"""ctypes binding of ``libattnring.so`` (argument marshalling only).

Every computation happens in the HIP library; this module turns torch
tensors into device pointers and sizes, calls the C ABI declared in
``include/attnring.h`` and raises on a non-OK status.  There is no fallback:
if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

# the in-tree build; ATTNRING_LIB may name another build of the same ABI (the
# tests point it at an AddressSanitizer build of the host code)
LIB_PATH = os.environ.get("ATTNRING_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libattnring.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP = 0, 1, 2, 3
ATTN_DTYPE_BF16, ATTN_DTYPE_FP32 = 0, 1
MAX_SEQS = 64
ABI_VERSION = 3
EXPORTED = ("attn_ring_step", "attn_ring_step_merge", "attn_ring_merge", "attn_prefill_causal",
            "attn_last_error", "attn_abi_version")


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"attnring status {status}: {message}")
        self.status = status


class AttnProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("cu_q", ctypes.POINTER(ctypes.c_int32)),
        ("cu_k", ctypes.POINTER(ctypes.c_int32)),
        ("q_pos0", ctypes.POINTER(ctypes.c_int32)),
        ("k_pos0", ctypes.POINTER(ctypes.c_int32)),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("k_row0", ctypes.POINTER(ctypes.c_int32)),
        ("k_len", ctypes.POINTER(ctypes.c_int32)),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m ring_attention_03_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.attn_ring_step.argtypes = [ctypes.POINTER(AttnProblem), ctypes.c_int, vp, vp, vp, vp, vp,
                                   ctypes.POINTER(ctypes.c_int32), vp]
    lib.attn_ring_step.restype = ctypes.c_int
    lib.attn_ring_step_merge.argtypes = [ctypes.POINTER(AttnProblem), ctypes.c_int, vp, vp, vp, vp,
                                         vp, ctypes.POINTER(ctypes.c_int32), vp]
    lib.attn_ring_step_merge.restype = ctypes.c_int
    lib.attn_prefill_causal.argtypes = [ctypes.POINTER(AttnProblem), ctypes.c_int, vp, vp, vp, vp,
                                        vp, vp]
    lib.attn_prefill_causal.restype = ctypes.c_int
    lib.attn_ring_merge.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.attn_ring_merge.restype = ctypes.c_int
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = ctypes.c_int32
    if lib.attn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.attn_abi_version()}, expected {ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status, _lib.attn_last_error().decode())


def _int_array(values, n):
    if values is None:
        return None
    vals = [int(x) for x in values]
    if len(vals) != n:
        raise ValueError(f"expected {n} entries, got {len(vals)}")
    return (ctypes.c_int32 * n)(*vals)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float32:
        return ATTN_DTYPE_FP32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _require_device(*tensors):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def make_problem(q, k, *, cu_q=None, cu_k=None, q_pos0=None, k_pos0=None, scale=0.0,
                 causal=True, num_seqs=None, k_row0=None, k_len=None):
    """Build the C ``attn_problem`` for q [Tq, Hq, d] and k [Tk, Hkv, d]; returns (struct, keepalive)."""
    if num_seqs is None:
        num_seqs = 1 if cu_q is None else len(cu_q) - 1
    arrays = (_int_array(cu_q, num_seqs + 1), _int_array(cu_k, num_seqs + 1),
              _int_array(q_pos0, num_seqs), _int_array(k_pos0, num_seqs),
              _int_array(k_row0, num_seqs), _int_array(k_len, num_seqs))
    as_ptr = [ctypes.cast(a, ctypes.POINTER(ctypes.c_int32)) if a is not None else None
              for a in arrays]
    prob = AttnProblem(num_seqs, as_ptr[0], as_ptr[1], as_ptr[2], as_ptr[3], q.shape[0],
                       k.shape[0], q.shape[1], k.shape[1], q.shape[2], float(scale),
                       1 if causal else 0, as_ptr[4], as_ptr[5])
    return prob, arrays


class PreparedCall:
    """One library call with every argument already marshalled (ctypes structs,
    pointers, stream); calling it only crosses into the library.  The tensors
    it was prepared from must stay alive and unmoved while it is used."""

    __slots__ = ("fn", "args", "launched", "keep")

    def __init__(self, fn, args, launched, keep):
        self.fn, self.args, self.launched, self.keep = fn, args, launched, keep

    def __call__(self) -> bool:
        _check(self.fn(*self.args))
        return bool(self.launched.value) if self.launched is not None else True


def _prepare_step(name, q, k, v, o, lse, *, cu_q, cu_k, q_pos0, k_pos0, scale, causal, report,
                  stream, k_row0=None, k_len=None):
    lib = load_library()
    _require_device(q, k, v, o, lse)
    _check_inputs(q, k, v)
    _check_out_shapes(q, o, lse)
    prob, keep = make_problem(q, k, cu_q=cu_q, cu_k=cu_k, q_pos0=q_pos0, k_pos0=k_pos0,
                              scale=scale, causal=causal, k_row0=k_row0, k_len=k_len)
    launched = ctypes.c_int32(0) if report else None
    args = (ctypes.byref(prob), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
            ctypes.byref(launched) if report else None, _stream(stream))
    return PreparedCall(getattr(lib, name), args, launched, (prob, keep))


def prepare_ring_step(q, k, v, o_part, lse_part, *, cu_q=None, cu_k=None, q_pos0=None,
                      k_pos0=None, scale=0.0, causal=True, report_skip=True, stream=None,
                      k_row0=None, k_len=None):
    """``attn_ring_step`` with its arguments marshalled once (see ``attn_ring_step``)."""
    return _prepare_step("attn_ring_step", q, k, v, o_part, lse_part, cu_q=cu_q, cu_k=cu_k,
                         q_pos0=q_pos0, k_pos0=k_pos0, scale=scale, causal=causal,
                         report=report_skip, stream=stream, k_row0=k_row0, k_len=k_len)


def prepare_ring_step_merge(q, k, v, o_acc, lse_acc, *, cu_q=None, cu_k=None, q_pos0=None,
                            k_pos0=None, scale=0.0, causal=True, stream=None, k_row0=None,
                            k_len=None):
    """``attn_ring_step_merge`` with its arguments marshalled once."""
    return _prepare_step("attn_ring_step_merge", q, k, v, o_acc, lse_acc, cu_q=cu_q, cu_k=cu_k,
                         q_pos0=q_pos0, k_pos0=k_pos0, scale=scale, causal=causal, report=True,
                         stream=stream, k_row0=k_row0, k_len=k_len)


def prepare_ring_merge(o_acc, lse_acc, o_part, lse_part, *, stream=None):
    """``attn_ring_merge`` with its arguments marshalled once."""
    lib = load_library()
    _require_device(o_acc, lse_acc, o_part, lse_part)
    for t in (o_acc, lse_acc, o_part, lse_part):
        if t.dtype != torch.float32:
            raise TypeError("merge buffers must be float32")
    if o_part.shape != o_acc.shape or lse_part.shape != lse_acc.shape:
        raise ValueError("partial and running state shapes differ")
    tq, hq, d = o_acc.shape
    if tuple(lse_acc.shape) != (hq, tq):
        raise ValueError(f"lse must be [Hq, T] = {(hq, tq)}, got {tuple(lse_acc.shape)}")
    args = (tq, hq, d, _ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), _stream(stream))
    return PreparedCall(lib.attn_ring_merge, args, None, None)


def attn_ring_step(q, k, v, o_part, lse_part, *, cu_q=None, cu_k=None, q_pos0=None, k_pos0=None,
                   scale=0.0, causal=True, report_skip=True, stream=None) -> bool:
    """One ring step (see ``attn_ring_step`` in attnring.h).  Returns whether outputs were written.

    With ``report_skip`` a fully masked block enqueues nothing and returns
    False (the caller must skip the merge); without it the identity is written.
    """
    return prepare_ring_step(q, k, v, o_part, lse_part, cu_q=cu_q, cu_k=cu_k, q_pos0=q_pos0,
                             k_pos0=k_pos0, scale=scale, causal=causal, report_skip=report_skip,
                             stream=stream)()


def attn_ring_step_merge(q, k, v, o_acc, lse_acc, *, cu_q=None, cu_k=None, q_pos0=None,
                         k_pos0=None, scale=0.0, causal=True, stream=None) -> bool:
    """One ring step folded into the running state (see ``attn_ring_step_merge`` in attnring.h).

    Returns whether a kernel was enqueued (False: no key of this block is
    visible, and the state is unchanged).
    """
    return prepare_ring_step_merge(q, k, v, o_acc, lse_acc, cu_q=cu_q, cu_k=cu_k, q_pos0=q_pos0,
                                   k_pos0=k_pos0, scale=scale, causal=causal, stream=stream)()


def attn_prefill_causal(q, k, v, o, lse, *, cu_seqlens=None, scale=0.0, stream=None) -> None:
    """Full causal attention of every packed sequence in one call (see attnring.h)."""
    lib = load_library()
    _require_device(q, k, v, o, lse)
    _check_inputs(q, k, v)
    _check_out_shapes(q, o, lse)
    prob, keep = make_problem(q, k, cu_q=cu_seqlens, cu_k=cu_seqlens, scale=scale, causal=True)
    _check(lib.attn_prefill_causal(ctypes.byref(prob), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(o), _ptr(lse), _stream(stream)))
    del keep


def attn_ring_merge(o_acc, lse_acc, o_part, lse_part, *, stream=None) -> None:
    """Fold (o_part, lse_part) into (o_acc, lse_acc) in place (see attnring.h)."""
    prepare_ring_merge(o_acc, lse_acc, o_part, lse_part, stream=stream)()


def _check_inputs(q, k, v):
    if q.dim() != 3 or k.dim() != 3 or tuple(k.shape) != tuple(v.shape):
        raise ValueError("q must be [Tq, Hq, d]; k and v the same [Tk, Hkv, d]")
    if k.shape[2] != q.shape[2]:
        raise ValueError("q and k head_dim differ")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")


def _check_out_shapes(q, o, lse):
    tq, hq, d = q.shape
    if tuple(o.shape) != (tq, hq, d) or o.dtype != torch.float32:
        raise ValueError(f"o must be float32 {(tq, hq, d)}, got {o.dtype} {tuple(o.shape)}")
    if tuple(lse.shape) != (hq, tq) or lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32 {(hq, tq)}, got {lse.dtype} {tuple(lse.shape)}")
