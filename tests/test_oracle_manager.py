"""Pins for the block-manager model and the write / copy oracle (CPU only).

The manager model is tied to a hand-worked trace (tests/golden) and to the
invariants the pages state: allocation follows the actual length, waste is at
most one partly filled block per sequence, shared blocks are counted, copies
happen only on a write to a shared block, freed blocks return to the pool.
The write / copy oracle is tied to a contiguous model that never sees slots
or tables: gathering the pools through the tables must reproduce it bitwise.
"""

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import workloads as W
from oracle import block_manager as BM
from oracle import kvcache as KV

from trace_runner import replay


class ModelAdapter:
    def __init__(self, nb, bs, order):
        self.m = BM.BlockManagerModel(nb, bs, order)

    def __getattr__(self, name):
        return getattr(self.m, name)

    def refcount(self, b):
        return self.m.refcount[b]

    def free_order(self):
        return list(reversed(self.m.free))


def test_golden_trace():
    assert replay(ModelAdapter, BM.PoolExhausted) > 30


def check_invariants(m):
    used = {}
    for seq, table in m.tables.items():
        n = m.lens[seq]
        # allocation follows actual length: ceil(n / bs) blocks
        assert len(table) == W.ceil_div(n, m.block_size)
        # at most one partly filled block: empty slots < block size
        assert len(table) * m.block_size - n < m.block_size or n == 0
        for b in table:
            used[b] = used.get(b, 0) + 1
    for b in range(m.num_blocks):
        assert m.refcount[b] == used.get(b, 0)
    free = set(m.free)
    assert len(free) == len(m.free)
    assert free.isdisjoint(used)
    assert len(free) + len(used) == m.num_blocks


ops = st.lists(st.tuples(st.sampled_from(["create", "fork", "append", "cow", "release", "batch"]),
                         st.integers(0, 5), st.integers(0, 5), st.integers(0, 40)), max_size=60)


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(ops=ops, nb=st.integers(1, 24), bs=st.sampled_from([1, 2, 4, 16]), seed=st.integers(0, 10))
def test_model_invariants_under_random_ops(ops, nb, bs, seed):
    order = np.random.default_rng(seed).permutation(nb)
    m = BM.BlockManagerModel(nb, bs, order)
    for op, a, b, n in ops:
        before = (list(m.free), list(m.refcount), {k: list(v) for k, v in m.tables.items()}, dict(m.lens))
        try:
            if op == "create":
                m.create(a, n)
            elif op == "fork":
                m.fork(a, b)
            elif op == "append":
                m.append(a)
            elif op == "cow":
                m.cow(a, n % 4)
            elif op == "release":
                m.release(a)
            else:
                m.append_batch([a, b])
        except (BM.PoolExhausted, BM.StateError):
            after = (list(m.free), list(m.refcount), {k: list(v) for k, v in m.tables.items()}, dict(m.lens))
            assert after == before  # failed calls change nothing
        check_invariants(m)
    for seq in list(m.tables):
        m.release(seq)
    assert sorted(m.free) == list(range(nb)) and not any(m.refcount)


def test_cow_only_when_shared():
    m = BM.BlockManagerModel(8, 4)
    m.create(0, 6)
    assert m.append(0)[1] is None  # private block: written in place
    m.fork(0, 1)
    slot, pair = m.append(1)
    assert pair is not None and pair[0] == m.table(0)[1]
    slot, pair = m.append(0)  # the original is private again
    assert pair is None


def test_exhaustion_leaves_state_unchanged():
    m = BM.BlockManagerModel(3, 2)
    m.create(0, 6)
    with pytest.raises(BM.PoolExhausted):
        m.append(0)
    assert m.length(0) == 6 and m.num_free() == 0
    m.fork(0, 1)
    with pytest.raises(BM.PoolExhausted):
        m.cow(1, 0)
    with pytest.raises(BM.PoolExhausted):
        m.append_batch([0, 1])
    assert m.table(1) == m.table(0) and m.refcount == [2, 2, 2]


# --- write / copy oracle through the contiguous model ----------------------------

def drive(seed, dtype=W.F32, nb=40, bs=4, hkv=2, d=3, steps=60):
    """Random create / fork / append / copy-on-write / release through the model
    manager, with every byte movement done by the write / copy oracle."""
    rng = np.random.default_rng(seed)
    m = BM.BlockManagerModel(nb, bs, rng.permutation(nb))
    kc = W.normal(rng, (nb, hkv, bs, d), dtype)
    vc = W.normal(rng, (nb, hkv, bs, d), dtype)
    model = KV.ContiguousModel()
    live = []
    for step in range(steps):
        r = rng.random()
        try:
            if r < 0.15 or not live:
                seq = step
                n = int(rng.integers(0, 9))
                m.create(seq, n)
                k = W.normal(rng, (n, hkv, d), dtype)
                v = W.normal(rng, (n, hkv, d), dtype)
                kc, vc = KV.write_kv(kc, vc, k, v, np.array(m.slots(seq, 0, n), np.int64), bs)
                model.create(seq, k.transpose(1, 0, 2), v.transpose(1, 0, 2))
                live.append(seq)
            elif r < 0.3:
                parent = live[int(rng.integers(len(live)))]
                m.fork(parent, step)
                model.fork(parent, step)
                live.append(step)
            elif r < 0.45:
                seq = live[int(rng.integers(len(live)))]
                if m.length(seq):
                    lb = int(rng.integers(len(m.table(seq))))
                    pair = m.cow(seq, lb)
                    if pair is not None:
                        kc, vc = KV.copy_blocks(kc, vc, np.array([pair], np.int64))
            elif r < 0.55:
                seq = live.pop(int(rng.integers(len(live))))
                m.release(seq)
                model.free(seq)
            else:
                seqs = sorted(set(int(x) for x in rng.choice(live, size=min(3, len(live)), replace=False)))
                res = m.append_batch(seqs)
                pairs = [p for _, p in res if p is not None]
                if pairs:
                    kc, vc = KV.copy_blocks(kc, vc, np.array(pairs, np.int64))
                k = W.normal(rng, (len(seqs), hkv, d), dtype)
                v = W.normal(rng, (len(seqs), hkv, d), dtype)
                kc, vc = KV.write_kv(kc, vc, k, v, np.array([s for s, _ in res], np.int64), bs)
                for i, seq in enumerate(seqs):
                    model.append(seq, k[i], v[i])
        except BM.PoolExhausted:
            pass
        for seq in live:
            row = m.table(seq)
            n = m.length(seq)
            assert np.array_equal(KV.logical_view(kc, row, n, bs).view(np.uint8),
                                  model.k[seq].view(np.uint8))
            assert np.array_equal(KV.logical_view(vc, row, n, bs).view(np.uint8),
                                  model.v[seq].view(np.uint8))
    return m


@pytest.mark.parametrize("seed", range(6))
def test_pools_match_contiguous_model(seed):
    drive(seed, dtype=[W.F32, W.BF16][seed % 2])


def test_write_skips_negative_slots_and_touches_nothing_else():
    rng = np.random.default_rng(8)
    kc = W.normal(rng, (5, 2, 4, 3), W.BF16)
    vc = W.normal(rng, (5, 2, 4, 3), W.BF16)
    k = W.normal(rng, (3, 2, 3), W.BF16)
    v = W.normal(rng, (3, 2, 3), W.BF16)
    k2, v2 = KV.write_kv(kc, vc, k, v, np.array([9, -1, 0], np.int64), 4)
    changed = np.argwhere(np.any(k2 != kc, axis=(1, 3)))
    assert set(map(tuple, changed)) <= {(2, 1), (0, 0)}
    assert np.array_equal(k2[2, :, 1], k[0]) and np.array_equal(v2[0, :, 0], v[2])
    mask = np.ones(k2.shape[:3], bool)
    mask[2, :, 1] = mask[0, :, 0] = False
    assert np.array_equal(k2[mask], kc[mask]) and np.array_equal(v2[mask], vc[mask])


def test_copy_reads_a_snapshot():
    rng = np.random.default_rng(9)
    kc = W.normal(rng, (4, 1, 2, 2), W.F32)
    vc = kc + 1
    k2, v2 = KV.copy_blocks(kc, vc, np.array([[0, 1], [1, 2], [1, 3]], np.int64))
    assert np.array_equal(k2[1], kc[0])
    assert np.array_equal(k2[2], kc[1]) and np.array_equal(k2[3], kc[1])  # old block 1
    assert np.array_equal(v2[2], vc[1])
