"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the paged decode path
computes, written from the pages' statement of the problem:

* spindle ("Paging"): a pool of fixed-size blocks and a per-sequence block
  table; reference counts give copy-on-write forking.
* spindle ("Why write the forward pass"): batched decoding must equal decoding
  each sequence alone (no attention leaking across sequences).
* spindle ("Two bugs worth recording"): the cache never works out a length
  itself; the position of a write and the number of tokens a read covers are
  both passed in by the caller.
* the mlsystems topic listing (flash-decoding entry): KV-length-parallel
  decode whose partial results are merged afterwards.

Paging and the split-KV merge are exact rewrites of plain softmax attention,
so the oracle is that plain definition: gather each sequence's blocks into
contiguous K/V, then run naive softmax attention in float64.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``paged_kv_cache_200_amd``) and imports nothing from it.

Modules
-------
paged_attention  numpy/float64: gather, decode, partitioned decode, LSE merge,
                 append, block copy.
brute            the same definitions as pure-Python loops (tiny inputs only).
block_pool       a plain-Python model of the block pool: FIFO free list,
                 tables, reference counts, fork and copy-on-write.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, the pages' worked copy-on-write example, invariants, a library routine
(PyTorch scaled-dot-product attention in float64) and brute force.
"""

from . import block_pool, brute, paged_attention  # noqa: F401
from .paged_attention import (  # noqa: F401
    combine_partitions,
    contiguous_decode,
    copy_blocks,
    decode_partitions,
    gather_sequence,
    kv_append,
    paged_decode,
    widen,
)
