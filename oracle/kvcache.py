"""KV-slot write, block copy and a contiguous reference model (oracle side).

Test infrastructure only (see the package docstring).

These operations move bytes and never do arithmetic on the stored values, so
the oracle works on the raw element arrays (float32, or uint16 bf16 patterns)
and every comparison with the device is bitwise.

Sources:

* foundry "PagedAttention" ops page, *How it works*: at each decode step the
  new token's key and value go into the sequence's current block; blocks may be
  shared between sequences and are copied only when a sharer writes to one
  (copy-on-write, also *At a glance*).
* aiacademy lesson "Paged Attention", the virtual-memory analogy table: token
  positions are contiguous while physical blocks are scattered.

Readings where the pages are silent:

* a slot is ``physical_block * block_size + offset_in_block`` (int64); a
  negative slot means "no token" and is skipped;
* block copies move the whole block (every KV head, every slot) and follow
  snapshot semantics: all sources are read as they were before the call.
"""

import numpy as np

from .attention import gather_sequence


def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, block_size):
    """Return copies of the pools with token ``i``'s K/V stored at its slot.

    k_cache, v_cache ``[NB][Hkv][bs][d]``; k_new, v_new ``[T][Hkv][d]``;
    slot_mapping ``int64 [T]``.  Token ``i`` with ``slot >= 0`` lands in
    block ``slot // bs`` at offset ``slot % bs`` for every KV head.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb = kc.shape[0]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), int(block_size))
        if blk >= nb:
            raise IndexError("slot outside the pool")
        kc[blk, :, off, :] = k_new[i]
        vc[blk, :, off, :] = v_new[i]
    return kc, vc


def copy_blocks(k_cache, v_cache, pairs):
    """Return copies of the pools with ``block[dst] = block[src]`` per pair.

    ``pairs`` is ``int64 [n][2]`` of (src, dst).  Sources are read from a
    snapshot taken before any copy, so the result does not depend on order.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ks = np.array(k_cache, copy=True)
    vs = np.array(v_cache, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        kc[dst] = ks[src]
        vc[dst] = vs[src]
    return kc, vc


def logical_view(cache, table_row, ctx, block_size):
    """A sequence's stored rows in logical order, ``[Hkv][ctx][d]`` (raw dtype)."""
    return gather_sequence(cache, table_row, ctx, block_size)


class ContiguousModel:
    """Every sequence's logical K/V as one growing contiguous run.

    This is the per-request slab that paging replaces (foundry page, *Concept*)
    used as ground truth: after any sequence of writes, copies and table
    changes, gathering the pools through the block tables must reproduce these
    runs bitwise, whichever physical blocks were chosen.
    """

    def __init__(self):
        self.k = {}
        self.v = {}

    def create(self, seq, k_rows, v_rows):
        """k_rows, v_rows ``[Hkv][n][d]``."""
        self.k[seq] = np.array(k_rows, copy=True)
        self.v[seq] = np.array(v_rows, copy=True)

    def fork(self, parent, child):
        self.k[child] = self.k[parent].copy()
        self.v[child] = self.v[parent].copy()

    def append(self, seq, k_tok, v_tok):
        """k_tok, v_tok ``[Hkv][d]``: one new token at the end of ``seq``."""
        self.k[seq] = np.concatenate([self.k[seq], k_tok[:, None, :]], axis=1)
        self.v[seq] = np.concatenate([self.v[seq], v_tok[:, None, :]], axis=1)

    def free(self, seq):
        del self.k[seq]
        del self.v[seq]

    def length(self, seq):
        return self.k[seq].shape[1]
