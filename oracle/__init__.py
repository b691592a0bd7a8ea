"""CPU fp64 oracle for blockwise causal GQA ring attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (``ring_attention_03_amd``) never imports it, and this package
imports nothing from the product path: the two share no code.

What it computes follows the problem statement of Moreh's post "Optimizing
Long-Context Prefill on Multiple Older-Generation GPU Nodes", section
"Introduction to Context Parallelism":

* context parallelism splits the prompt along the sequence; only attention
  couples tokens (the paragraph that introduces context parallelism);
* Ring Attention has every device run attention on its partial query, key and
  value while trading key/value blocks with its neighbours (the "Ring
  Attention" bullet), so the partial results must add up to ordinary causal
  attention over the whole sequence;
* grouped-query attention shares one key/value head among several query
  heads (the paragraph on the trade-offs of the two approaches).

The pages give no formula; the formula used is the textbook definition of
scaled dot-product causal softmax attention, written out plainly in fp64
(see ``attention.py``).  Every function here is pinned by the ``-m "not gpu"``
tests in ``tests/test_oracle.py`` against closed forms, a library routine
(torch's CPU scaled-dot-product attention) and a brute-force loop.
"""

from .attention import (  # noqa: F401
    attention_ref,
    causal_attention_ref,
    chunk_layout_ref,
    merge_ref,
    ring_ref,
    visible_pairs_ref,
)
