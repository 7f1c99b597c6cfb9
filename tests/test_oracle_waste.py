"""Pins of the waste oracle (oracle/waste.py) to values worked out by hand,
closed forms and the pages' bound -- CPU only.

* the twelve-slot toy memory map of the aiacademy "Paged Attention" lesson
  (figure): two requests with three and two live slots in slabs of six and
  five leave one slot of twelve free; paged, the same data leaves at least
  five free (the figure's counts are invented for teaching: its paged row
  holds seven slots, which no single block size gives for three and two
  live tokens, so the pin is the contiguous row exactly and the paged row's
  bound);
* one request alone: steps, live and held slot-steps in closed form;
* the bound of the foundry "PagedAttention" ops page, Concept: paged waste is
  at most one partly filled block per running request;
* hand-worked runs of first-fit fragmentation and of preemption.
"""

import numpy as np
import pytest

from oracle import waste as WS


def run(mode, cap, bs, reqs):
    p, o, r = zip(*reqs)
    return WS.simulate(mode, cap, bs, p, o, r)


def test_toy_memory_map():
    reqs = [(3, 1, 6), (2, 1, 5)]  # one generated token each: the map is step 0's
    c = run(WS.CONTIGUOUS, 12, 1, reqs)
    assert (c["steps"], c["live_slot_steps"], c["held_slot_steps"]) == (1, 5, 11)
    assert 12 - c["held_slot_steps"] == 1                    # one free slot
    assert c.waste() == pytest.approx(6 / 11)                # six reserved-but-empty of eleven held
    for bs in (1, 2):
        pg = run(WS.PAGED, 12, bs, reqs)
        assert pg["live_slot_steps"] == 5
        assert 12 - pg["held_slot_steps"] >= 5                # five times as many free slots (or more)
        assert pg["held_slot_steps"] - pg["live_slot_steps"] <= 2 * (bs - 1)


@pytest.mark.parametrize("p,o,extra,bs", [(1, 1, 0, 1), (5, 9, 3, 4), (16, 16, 0, 16), (17, 40, 100, 16),
                                           (100, 1, 7, 8), (3, 30, 0, 32)])
def test_single_request_closed_forms(p, o, extra, bs):
    r = p + o + extra
    live = o * p + o * (o - 1) // 2                        # lengths p, p+1, ..., p+o-1 over o steps
    c = run(WS.CONTIGUOUS, r, 1, [(p, o, r)])
    assert (c["steps"], c["live_slot_steps"], c["held_slot_steps"]) == (o, live, o * r)
    assert (c["running_steps"], c["decode_tokens"], c["preemptions"]) == (o, o, 0)
    pg = run(WS.PAGED, -(-(p + o) // bs) * bs, bs, [(p, o, r)])
    held = sum(-(-(p + k) // bs) * bs for k in range(o))
    assert (pg["steps"], pg["live_slot_steps"], pg["held_slot_steps"]) == (o, live, held)


def test_fragmentation_hand_worked():
    """Capacity 10, first fit.  Step 0: A@0 (slab 3), B@3 (slab 4), C@7
    (slab 3) fill the pool; D (slab 5) waits with nothing free.  A and C
    finish: gaps [0,3) and [7,10), six free slots but no gap of five -- D is
    refused at steps 1 and 2 for fragmentation.  B finishes at step 2 (its
    slab merges both gaps); D runs at step 3."""
    reqs = [(1, 1, 3), (1, 3, 4), (1, 1, 3), (1, 1, 5)]
    c = run(WS.CONTIGUOUS, 10, 1, reqs)
    assert dict(c) == {"steps": 4, "live_slot_steps": 3 + 2 + 3 + 1, "held_slot_steps": 10 + 4 + 4 + 5,
                       "running_steps": 3 + 1 + 1 + 1, "max_running": 3, "preemptions": 0,
                       "frag_blocked_steps": 2, "decode_tokens": 6}
    pg = run(WS.PAGED, 10, 1, reqs)  # any free block fits: all four start at once
    assert dict(pg) == {"steps": 3, "live_slot_steps": 4 + 2 + 3, "held_slot_steps": 4 + 2 + 3,
                        "running_steps": 6, "max_running": 4, "preemptions": 0, "frag_blocked_steps": 0,
                        "decode_tokens": 6}


def test_preemption_hand_worked():
    """Two blocks of two slots.  Step 0: A (2 tokens) and B (2 tokens) hold a
    block each; A's next token needs a block, none is free: B (the latest
    admitted) is preempted and requeued, A takes its block.  Step 1: B does
    not fit; A finishes.  Step 2: B runs and finishes."""
    pg = run(WS.PAGED, 4, 2, [(2, 2, 4), (2, 1, 3)])
    assert dict(pg) == {"steps": 3, "live_slot_steps": 4 + 3 + 2, "held_slot_steps": 4 + 4 + 2,
                        "running_steps": 4, "max_running": 2, "preemptions": 1, "frag_blocked_steps": 0,
                        "decode_tokens": 3}


def test_paged_waste_bound_and_accounting():
    rng = np.random.default_rng(3)
    for trial in range(20):
        bs = int(rng.choice([1, 4, 16]))
        n = int(rng.integers(1, 25))
        p = rng.integers(1, 60, n)
        o = rng.integers(1, 60, n)
        r = p + o + rng.integers(0, 40, n)
        cap = int(max(r.max(), -(-(p + o).max() // bs) * bs) + rng.integers(0, 300))
        for mode in (WS.CONTIGUOUS, WS.PAGED):
            st = WS.simulate(mode, cap, bs, p, o, r)
            assert st["held_slot_steps"] <= st["steps"] * cap
            assert st["live_slot_steps"] <= st["held_slot_steps"]
            # every generated token is stored once, plus the ones lost to preemption
            assert st["decode_tokens"] >= int(o.sum())
            if mode == WS.PAGED:
                assert st["held_slot_steps"] - st["live_slot_steps"] <= (bs - 1) * st["running_steps"]
                assert st["frag_blocked_steps"] == 0
            else:
                assert st["preemptions"] == 0 and st["decode_tokens"] == int(o.sum())


def test_rejects_requests_that_never_fit():
    with pytest.raises(ValueError):
        run(WS.CONTIGUOUS, 5, 1, [(2, 2, 6)])
    with pytest.raises(ValueError):
        run(WS.PAGED, 8, 4, [(5, 4, 9)])       # 9 tokens need 3 blocks of 4, the pool has 2
    with pytest.raises(ValueError):
        run(WS.CONTIGUOUS, 10, 1, [(2, 2, 3)])  # slab below p + o
