"""MI355X-native blockwise causal GQA ring attention (one device's share).

The HIP library ``libattnring.so`` (C ABI in ``include/attnring.h``) holds
every kernel; this package is its thin Python binding plus the host-side
ring schedule.  Importing the package does not load the library; the first
call does, and raises if it has not been built.
"""

from ._native import (  # noqa: F401
    AttnError,
    attn_prefill_causal,
    attn_ring_merge,
    attn_ring_step,
    attn_ring_step_merge,
    load_library,
)
from .ring import (ChunkedPrefill, RingAttention, RingLayout, ZigzagLayout, ZigzagRing,  # noqa: F401
                   ring_chunk)

__all__ = ["attn_ring_step", "attn_ring_step_merge", "attn_ring_merge", "attn_prefill_causal",
           "load_library", "AttnError", "RingAttention", "RingLayout", "ChunkedPrefill",
           "ZigzagLayout", "ZigzagRing", "ring_chunk"]
