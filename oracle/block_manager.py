"""Host block manager model: free pool, reference counts, block tables.

Test infrastructure only (see the package docstring).

Plain-Python restatement of the bookkeeping the pages describe:

* foundry "PagedAttention" ops page, *Concept*: memory is handed out one
  fixed-size block at a time on demand; freed blocks go back to a shared pool.
* same page, *How it works*: the new token goes into the sequence's current
  block; when that block is full a fresh block is taken from the global free
  pool and the block table is extended, so allocation follows the actual
  length.  Sequences with identical content point their tables at the same
  physical blocks and copy on write when they diverge.  An empty free pool is
  the point where a scheduler would preempt (here: an error, state unchanged).
* same page, *At a glance*: shared blocks are tracked by reference count and a
  block is copied only when a sequence writes to it.
* aiacademy lesson "Paged Attention": a new block is allocated only when decode
  fills the last one, every block is released when the request completes, and
  any free block fits any request.

Readings where the pages are silent (the same contract the C library states):

* the free pool is a stack; it starts as ``free_order`` with ``free_order[0]``
  handed out first, and released blocks are pushed on top (reused first);
* releasing a sequence walks its table in logical order;
* on copy-on-write the writing sequence receives the new private block and the
  other sharers keep the original (its count drops by one);
* a block whose count is 1 is written in place, without a copy;
* every failing call leaves the whole state unchanged;
* a batch append checks every sequence id before taking any block (an
  unknown id is a state error even when the pool is also short).

Swap (foundry page, *How it works* and *Trade-offs*: when the pool runs dry a
scheduler preempts, and a preempted sequence's blocks can be swapped out to
CPU memory and brought back).  Readings: the host swap space is a second
stack of its own blocks; swapping out gives every logical block of the
sequence its own host block, in logical order, and drops one reference to
the device block (which returns to the free pool only if no other sequence
shares it); swapping in takes a device block per host block, in logical
order, and returns the host blocks; a swapped-out sequence can only be
swapped in, inspected or released.

Prefix caching (aimodelwiki "PagedAttention" glossary entry, prefix-caching
paragraph: requests sharing a prompt prefix reuse its KV blocks; foundry ops
page, At a glance: shared blocks are tracked by reference count).  Readings:
when enabled, a sequence created from its prompt tokens registers each of
its full blocks under the exact key (prefix node of the previous block, the
block's tokens); node ids are never reused.  A new prompt shares the longest
run of its full blocks found that way.  A cached block whose count falls to
0 is kept at the tail of an LRU list instead of the free stack; a block is
taken from the free stack first, else by evicting the LRU head (its cache
entry goes).  A cached block is immutable: forcing a private copy of it
copies even when its count is 1.
"""

import copy
from collections import OrderedDict


class PoolExhausted(Exception):
    """No free block left for a required allocation (state unchanged)."""


class StateError(Exception):
    """Unknown or duplicate sequence id, or another invalid request."""


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise StateError("pool dimensions must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise StateError("free_order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(reversed(order))  # top of stack = end of list
        self.refcount = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        self.host_free = []   # host swap blocks, top of stack = end of list
        self.swapped = set()  # sequences whose table names host blocks
        self.prefix_cache = False
        self.cache = {}          # (parent node, tokens tuple) -> (block, node)
        self.block_key = {}      # cached block -> its key
        self.lru = OrderedDict()  # cached blocks with count 0, least recent first
        self.next_node = 1

    # -- helpers ---------------------------------------------------------
    def _available(self):
        return len(self.free) + len(self.lru)

    def _take(self):
        if self.free:
            blk = self.free.pop()
        elif self.lru:
            blk, _ = self.lru.popitem(last=False)  # evict the least recently released
            del self.cache[self.block_key.pop(blk)]
        else:
            raise PoolExhausted()
        self.refcount[blk] = 1
        return blk

    def _release(self, blk):
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            if blk in self.block_key:
                self.lru[blk] = None
            else:
                self.free.append(blk)

    def _need(self, seq):
        if seq not in self.tables:
            raise StateError(f"unknown sequence {seq}")
        if seq in self.swapped:
            raise StateError(f"sequence {seq} is swapped out")

    def _atomic(self, fn):
        saved = (list(self.free), list(self.refcount), copy.deepcopy(self.tables), dict(self.lens),
                 list(self.host_free), set(self.swapped), dict(self.cache), dict(self.block_key),
                 OrderedDict(self.lru), self.next_node)
        try:
            return fn()
        except Exception:
            (self.free, self.refcount, self.tables, self.lens, self.host_free, self.swapped, self.cache,
             self.block_key, self.lru, self.next_node) = saved
            raise

    # -- operations -------------------------------------------------------
    def create(self, seq, num_tokens):
        """New sequence holding ``num_tokens`` tokens in ceil(n / bs) blocks."""
        if seq in self.tables:
            raise StateError(f"sequence {seq} exists")
        if num_tokens < 0:
            raise StateError("negative length")

        def run():
            nb = -(-num_tokens // self.block_size)
            self.tables[seq] = [self._take() for _ in range(nb)]
            self.lens[seq] = num_tokens

        self._atomic(run)

    def fork(self, parent, child):
        """``child`` shares every block of ``parent``; counts go up by one."""
        self._need(parent)
        if child in self.tables:
            raise StateError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.refcount[blk] += 1

    def append(self, seq):
        """Reserve the slot for one new token; returns ``(slot, pair)``.

        ``pair`` is ``(src, dst)`` when the current block was shared and had to
        be copied first, else ``None``.
        """
        self._need(seq)

        def run():
            pos = self.lens[seq]
            table = self.tables[seq]
            lb, off = divmod(pos, self.block_size)
            pair = None
            if off == 0:
                table.append(self._take())
            elif self.refcount[table[lb]] > 1:
                src = table[lb]
                dst = self._take()
                self._release(src)
                table[lb] = dst
                pair = (src, dst)
            self.lens[seq] = pos + 1
            return table[lb] * self.block_size + off, pair

        return self._atomic(run)

    def append_batch(self, seqs):
        """``append`` for each sequence in order; all-or-nothing.

        Every sequence id is checked before any block is taken, so a batch
        naming an unknown sequence fails as a state error even when the pool
        would also run short.
        """
        for s in seqs:
            self._need(s)
        return self._atomic(lambda: [self.append(s) for s in seqs])

    def cow(self, seq, logical_block):
        """Give ``seq`` a private copy of one logical block if it is shared."""
        self._need(seq)
        table = self.tables[seq]
        if not 0 <= logical_block < len(table):
            raise StateError("logical block out of range")
        src = table[logical_block]
        if self.refcount[src] == 1 and src not in self.block_key:
            return None

        def run():
            dst = self._take()
            self._release(src)
            table[logical_block] = dst
            return (src, dst)

        return self._atomic(run)

    def release(self, seq):
        """Return every block of ``seq`` to its pool (device: count drops by
        one each; host swap blocks of a swapped-out sequence: freed)."""
        if seq in self.swapped:
            self.swapped.remove(seq)
            self.host_free.extend(self.tables.pop(seq))
            del self.lens[seq]
            return
        self._need(seq)
        for blk in self.tables.pop(seq):
            self._release(blk)
        del self.lens[seq]

    # -- prefix cache ---------------------------------------------------------
    def enable_prefix_cache(self):
        self.prefix_cache = True

    def create_cached(self, seq, tokens):
        """New sequence holding ``tokens``; shares the longest cached run of
        its full blocks.  Returns the number of tokens found cached."""
        if not self.prefix_cache:
            raise StateError("prefix caching is not enabled")
        if seq in self.tables:
            raise StateError(f"sequence {seq} exists")
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        need = -(-len(tokens) // bs)
        full = len(tokens) // bs
        hits, parent = [], 0
        for i in range(full):
            hit = self.cache.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            if hit is None:
                break
            hits.append(hit[0])
            parent = hit[1]
        idle = sum(1 for b in hits if self.refcount[b] == 0)
        if need - len(hits) + idle > self._available():
            raise PoolExhausted()
        table = []
        for b in hits:
            if self.refcount[b] == 0:
                del self.lru[b]
            self.refcount[b] += 1
            table.append(b)
        for i in range(len(hits), need):
            b = self._take()
            table.append(b)
            if i < full:
                key = (parent, tuple(tokens[i * bs:(i + 1) * bs]))
                node = self.next_node
                self.next_node += 1
                self.cache[key] = (b, node)
                self.block_key[b] = key
                parent = node
        self.tables[seq] = table
        self.lens[seq] = len(tokens)
        return len(hits) * bs

    def is_cached(self, blk):
        return blk in self.block_key

    def lru_order(self):
        return list(self.lru)

    # -- swap ---------------------------------------------------------------
    def set_swap_space(self, num_host_blocks, host_free_order=None):
        """A host swap space of ``num_host_blocks`` blocks (replaces the old
        one; not while a sequence is swapped out)."""
        if self.swapped:
            raise StateError("sequences are swapped out")
        order = list(range(num_host_blocks)) if host_free_order is None else [int(h) for h in host_free_order]
        if sorted(order) != list(range(num_host_blocks)):
            raise StateError("host_free_order must be a permutation")
        self.host_free = list(reversed(order))

    def swap_out(self, seq):
        """Move ``seq`` to host blocks; returns the (device, host) copies to do."""
        self._need(seq)
        table = self.tables[seq]
        if len(table) > len(self.host_free):
            raise PoolExhausted()
        pairs = []
        for lb, blk in enumerate(table):
            h = self.host_free.pop()
            pairs.append((blk, h))
            table[lb] = h
            self._release(blk)
        self.swapped.add(seq)
        return pairs

    def swap_in(self, seq):
        """Bring ``seq`` back to device blocks; returns the (host, device) copies."""
        if seq not in self.tables:
            raise StateError(f"unknown sequence {seq}")
        if seq not in self.swapped:
            raise StateError(f"sequence {seq} is not swapped out")
        table = self.tables[seq]
        if len(table) > self._available():
            raise PoolExhausted()
        pairs = []
        for lb, h in enumerate(table):
            blk = self._take()
            pairs.append((h, blk))
            table[lb] = blk
            self.host_free.append(h)
        self.swapped.remove(seq)
        return pairs

    def is_swapped(self, seq):
        if seq not in self.tables:
            raise StateError(f"unknown sequence {seq}")
        return seq in self.swapped

    def slots(self, seq, start, count):
        """Slots of logical positions ``start .. start+count-1`` of ``seq``."""
        self._need(seq)
        if start < 0 or count < 0 or start + count > self.lens[seq]:
            raise StateError("positions outside the sequence")
        table = self.tables[seq]
        out = []
        for pos in range(start, start + count):
            lb, off = divmod(pos, self.block_size)
            out.append(table[lb] * self.block_size + off)
        return out

    # -- inspection -------------------------------------------------------
    def num_free(self):
        return len(self.free)

    def table(self, seq):
        """Block ids of ``seq`` (host swap blocks while it is swapped out)."""
        if seq not in self.tables:
            raise StateError(f"unknown sequence {seq}")
        return list(self.tables[seq])

    def length(self, seq):
        if seq not in self.tables:
            raise StateError(f"unknown sequence {seq}")
        return self.lens[seq]
