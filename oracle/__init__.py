"""CPU oracle for paged attention and its cache companions.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
load this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its binding.

What it is: a plain, slow, float64 numpy statement of what the path computes,
written from the pages' description of PagedAttention:

* ``codecs``  — bfloat16 and OCP FP8 E4M3FN storage decoded from their bit
  fields; the FP8 encoder used by the quantising cache write.
* ``paged``   — gather a sequence's K/V through its block table into
  contiguous arrays, softmax(q·Kᵀ·scale)·V per query head (GQA groups are
  contiguous), the causal chunked-prefill variant, the slot-mapped cache
  write, the block copy used by copy-on-write, the block swap to and from
  host memory, and the log-sum-exp merge of per-partition softmax states.
* ``block_manager`` — the reference block manager: free list, reference
  counts, fork / append / free with copy-on-write, swap of sequence sets to
  host blocks, and automatic prefix caching (chained FNV-1a block hashes,
  lookup, touch, commit, eviction).

Every function is pinned by ``tests/test_oracle_*.py`` against something
other than itself: torch's library casts and attention, brute-force loops,
closed forms, the worked block-table examples and figures on the pages,
published hash test vectors, and brute-force token memories for the block
manager, plus the paging invariants (relabelling physical blocks or sharing
prefix blocks leaves the outputs unchanged).  No function here is "parity unpinned".
"""
from . import block_manager, codecs, paged  # noqa: F401
