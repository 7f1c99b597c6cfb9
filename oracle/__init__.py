"""CPU oracle for the PagedAttention decode hot path (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may use it.  It shares no code with the HIP library: no
kernels, headers, helpers, tables or constants.

What it computes, and where the pages define it:

* ``attention.decode`` -- single-query decode attention read through a
  per-sequence block table.  The PagedAttention pages (foundry "PagedAttention"
  ops page, sections *Concept* and *How it works*) say the KV cache of each
  sequence is cut into fixed-size blocks stored anywhere in a shared pool, that
  a block table maps logical positions to physical blocks, and that reading KV
  through the table leaves the attention math unchanged.  The math itself is
  the textbook softmax(q K^T * scale) V, evaluated here in fp64 on a contiguous
  gather of each sequence's blocks.
* ``prefill.prefill`` -- causal attention of a chunk of new queries per
  sequence (a prompt, or its next piece) read through the block table: query
  ``i`` of ``n`` sits at position ``ctx - n + i`` and sees keys ``0 .. that``
  (foundry page, *Concept* and *How it works*; textbook causal softmax).
* ``attention.partials`` / ``attention.merge`` -- the same result computed per
  context partition and merged (online-softmax normaliser merge,
  Milakov & Gimelshein 2018); exact in real arithmetic.
* ``kvcache.write_kv`` -- the new token's key and value stored into the
  sequence's current block ("How it works").
* ``kvcache.copy_blocks`` -- whole-block duplication for copy-on-write
  (foundry page, *How it works* and *At a glance*).
* ``kvcache.ContiguousModel`` -- each sequence's logical KV kept as one
  contiguous run (the slab the method replaces), to check pools bitwise
  through the tables.
* ``block_manager.BlockManagerModel`` -- free pool, reference counts, on-demand
  table extension, sharing, copy-on-write and release (foundry page,
  *Concept*, *How it works*, *At a glance*; aiacademy lesson "Paged
  Attention", the virtual-memory analogy table); also its swap space and
  prefix cache (foundry page, *How it works* and *Trade-offs*; aimodelwiki
  "PagedAttention" glossary entry, prefix-caching paragraph).
* ``waste.simulate`` -- a serving loop over one pool of KV slots, contiguous
  slabs against paged blocks, counting live and held slots per step (foundry
  page, *Concept* and *At a glance*; aiacademy lesson, its toy memory map).

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
something other than itself: brute-force loops on tiny inputs, PyTorch's
scaled-dot-product attention in fp64 on contiguous data, closed forms,
hand-worked golden fixtures under ``tests/golden/`` and invariants the pages
state (placement independence, sharing, tail blocks).
"""

from . import attention, block_manager, kvcache, numerics, prefill, waste  # noqa: F401
