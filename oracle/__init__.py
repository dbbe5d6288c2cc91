"""CPU fp64 oracle for fused causal attention, paged decode, the paged cache
append and the residual-add + RMSNorm fusion.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this package:
only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code with the HIP library or its Python
binding, and imports nothing from them.

Every function is the plain definition of the operation, written out so that it
can be checked against the source pages by eye:

* "Fast attention kernels and operator fusion" (the-ai.news), section
  "FlashAttention-style attention and paged attention": attention builds a
  T x T score matrix per head; a paged KV cache stores keys and values in
  fixed-size blocks and a block table maps logical positions to physical
  blocks, through which the kernel must translate every position.
* "Hugging Face attention profiling guide" (aiexpert.news), second paragraph:
  the naive forward is Q @ K^T, a scaling, a causal masked_fill, a softmax and
  a final product with V.

All functions are pinned by ``tests/test_oracle.py`` (brute force, closed
forms, invariants and a library special case); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    prefill,
    decode_paged,
    gather_paged_kv,
    kv_append,
    add_rmsnorm,
)
