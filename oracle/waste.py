"""KV-cache memory waste: contiguous per-request slabs against paged blocks.

Test infrastructure only (see the package docstring).  A step-by-step
simulation of a serving loop over one KV pool of ``capacity`` token slots,
written as plainly as the rules below allow.

What the pages fix:

* foundry "PagedAttention" ops page, Concept: a naive engine reserves one
  contiguous slab per request sized to its maximum length, so a request that
  stops early strands the rest; paging hands memory out one block at a time,
  so at most one partly filled block per sequence is wasted, and freed
  blocks return to a shared pool.  At a glance: the slab strands memory
  inside (unfilled reserved slots) and outside (gaps too small to reuse).
* aiacademy "Paged Attention" lesson: the slab is sized for the longest
  output the request might produce; a new block is taken only when decode
  fills the last one, and every block is freed when the request completes;
  the toy memory map of twelve slots.
* aimodelwiki "PagedAttention" glossary entry: waste is the headline
  measurement (paged well below contiguous).

Readings where the pages leave a step open (each is in the design notes):

* requests arrive together, in order; each has a prompt of ``p`` tokens, a
  generated length ``o`` and a slab size ``r >= p + o`` (the longest it
  might have produced);
* one step = admission, then the state is recorded, then every running
  request stores the KV of one new token, then finished requests leave;
* admission is first come, first served: the head of the queue is admitted
  while it fits, and nothing behind it jumps the queue.  A slab takes the
  lowest-addressed free gap of at least ``r`` slots (first fit; freed slabs
  merge with free neighbours).  A paged request takes ``ceil(p / bs)``
  blocks from the block manager;
* when a paged request needs a block and none is free, the most recently
  admitted running request is preempted (its blocks freed, its progress
  lost) and goes back to the front of the queue, until a block is free or
  the request itself was preempted;
* a request that can never fit alone is an error.

Recorded per step (after admission, before the step's new tokens): live
slots (tokens stored), held slots (the slab sizes, or blocks x bs), running
requests; plus preemptions and the steps where the queue head was refused
although the free slots added up to its slab (external fragmentation).
Waste = 1 - live / held over the whole run.
"""

from .block_manager import BlockManagerModel, PoolExhausted

CONTIGUOUS = "contiguous"
PAGED = "paged"


class Stats(dict):
    """Integer counters of one run."""

    KEYS = ("steps", "live_slot_steps", "held_slot_steps", "running_steps", "max_running", "preemptions",
            "frag_blocked_steps", "decode_tokens")

    def waste(self):
        return 1.0 - self["live_slot_steps"] / self["held_slot_steps"] if self["held_slot_steps"] else 0.0


def _first_fit(gaps, r):
    """Lowest-addressed gap (start, length) with length >= r, or None."""
    for i, (start, length) in enumerate(gaps):
        if length >= r:
            return i
    return None


def _free_slab(gaps, start, r):
    """Return [start, start + r) to the sorted gap list, merging neighbours."""
    gaps.append((start, r))
    gaps.sort()
    merged = []
    for s, n in gaps:
        if merged and merged[-1][0] + merged[-1][1] == s:
            merged[-1] = (merged[-1][0], merged[-1][1] + n)
        else:
            merged.append((s, n))
    gaps[:] = merged


def simulate(mode, capacity, block_size, prompt_lens, output_lens, reserve_lens):
    """Run the serving loop to completion; returns ``Stats``."""
    n = len(prompt_lens)
    p = [int(x) for x in prompt_lens]
    o = [int(x) for x in output_lens]
    r = [int(x) for x in reserve_lens]
    if mode not in (CONTIGUOUS, PAGED):
        raise ValueError(mode)
    if len(o) != n or len(r) != n or block_size < 1 or capacity < 0:
        raise ValueError("bad arguments")
    num_blocks = capacity // block_size
    for i in range(n):
        if p[i] < 1 or o[i] < 1 or r[i] < p[i] + o[i]:
            raise ValueError(f"request {i}: need p >= 1, o >= 1, r >= p + o")
        if mode == CONTIGUOUS and r[i] > capacity:
            raise ValueError(f"request {i}: slab of {r[i]} exceeds the pool")
        if mode == PAGED and -(-(p[i] + o[i]) // block_size) > num_blocks:
            raise ValueError(f"request {i}: {p[i] + o[i]} tokens exceed the pool")

    st = Stats({k: 0 for k in Stats.KEYS})
    waiting = list(range(n))
    running = []          # admission order
    length = {}           # request -> tokens stored
    slab = {}             # request -> slab start (contiguous)
    gaps = [(0, capacity)] if capacity else []
    pool = BlockManagerModel(num_blocks, block_size) if mode == PAGED and n else None  # no requests: no pool

    while waiting or running:
        # admission, first come first served
        while waiting:
            i = waiting[0]
            if mode == CONTIGUOUS:
                g = _first_fit(gaps, r[i])
                if g is None:
                    if sum(length for _, length in gaps) >= r[i]:
                        st["frag_blocked_steps"] += 1
                    break
                start, glen = gaps[g]
                slab[i] = start
                if glen == r[i]:
                    del gaps[g]
                else:
                    gaps[g] = (start + r[i], glen - r[i])
            else:
                try:
                    pool.create(i, p[i])
                except PoolExhausted:
                    break
            waiting.pop(0)
            running.append(i)
            length[i] = p[i]

        # the step's memory map
        st["steps"] += 1
        st["running_steps"] += len(running)
        st["max_running"] = max(st["max_running"], len(running))
        st["live_slot_steps"] += sum(length[i] for i in running)
        if mode == CONTIGUOUS:
            st["held_slot_steps"] += sum(r[i] for i in running)
        else:
            st["held_slot_steps"] += sum(len(pool.table(i)) * block_size for i in running)

        # one new token per running request
        k = 0
        while k < len(running):
            i = running[k]
            if mode == PAGED:
                while True:
                    try:
                        pool.append(i)
                        break
                    except PoolExhausted:
                        victim = running.pop()
                        pool.release(victim)
                        del length[victim]
                        waiting.insert(0, victim)
                        st["preemptions"] += 1
                        if victim == i:
                            break
                if i not in length:  # preempted itself
                    continue
            length[i] += 1
            st["decode_tokens"] += 1
            k += 1

        # finished requests leave
        for i in list(running):
            if length[i] == p[i] + o[i]:
                running.remove(i)
                del length[i]
                if mode == CONTIGUOUS:
                    _free_slab(gaps, slab.pop(i), r[i])
                else:
                    pool.release(i)
    return st
