"""Shared-prefix copy-on-write workload on the GPU, step by step.

256 sequences share the blocks of one 2048-token prefix (reference count 256)
and own private suffixes of U{0..512} tokens.  Each of 8 steps: 1% of the
shared (sequence, prefix block) references are made private (host manager
decisions, device block copies), then every sequence appends one token (slot
from the manager, K/V stored by pa_write_kv) and attends over its whole
context.  After every step:

* the device pools, gathered through the manager's block tables, equal each
  sequence's logical K/V kept as one contiguous run (bitwise), whichever
  physical blocks the manager chose, for every sequence;
* the manager's reference counts equal the number of table entries naming
  each block;
* pa_decode equals the fp64 oracle evaluated on the contiguous runs, for
  every sequence and query head.

Pages: foundry "PagedAttention" ops page, How it works and At a glance
(sharing with reference counts, copy only when a sequence writes, new token
into the current block).
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import kvcache as KV

from gpu_cases import announce, check_decode, out_to_f64, to_dev

pytestmark = pytest.mark.gpu

BAL = -1


def seq_pool(k_rows, v_rows, bs):
    """A one-sequence pool holding contiguous runs ``[Hkv][n][d]`` in order."""
    hkv, n, d = k_rows.shape
    nb = max(1, W.ceil_div(n, bs))
    out = []
    for rows in (k_rows, v_rows):
        padded = np.zeros((hkv, nb * bs, d), rows.dtype)
        padded[:, :n] = rows
        out.append(np.ascontiguousarray(padded.reshape(hkv, nb, bs, d).transpose(1, 0, 2, 3)))
    return out[0], out[1], np.arange(nb, dtype=np.int32)[None]


def gather_rows(cache, table, n, bs):
    """Device pool rows of one sequence in logical order, ``[Hkv][n][d]``."""
    nb = W.ceil_div(n, bs)
    blocks = cache[torch.as_tensor(table[:nb], device=cache.device, dtype=torch.long)]
    hkv, d = cache.shape[1], cache.shape[3]
    return blocks.permute(1, 0, 2, 3).reshape(hkv, nb * bs, d)[:, :n]


def test_shared_prefix_copy_on_write_steps(gpu_lib):
    pkv = gpu_lib
    plan = W.c4_shared_prefix()
    bs, B, hkv, d = plan.block_size, plan.num_seqs, plan.num_kv_heads, plan.head_dim
    prefix_blocks = plan.prefix_len // bs
    announce("shared prefix", B, "seqs", plan.num_blocks, "blocks")
    pool = pkv.BlockPool(plan.num_blocks, bs, plan.free_order)
    model = KV.ContiguousModel()
    kdev = torch.zeros((plan.num_blocks, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    vdev = torch.zeros_like(kdev)

    # sequence 0 holds the prefix; the others fork it, then append their suffix
    pool.create(0, plan.prefix_len)
    slots = pool.slots(0, 0, plan.prefix_len)
    kp = np.ascontiguousarray(plan.prefix_k.transpose(1, 0, 2))  # [n][Hkv][d]
    vp = np.ascontiguousarray(plan.prefix_v.transpose(1, 0, 2))
    pkv.pa_write_kv(to_dev(kp), to_dev(vp), to_dev(slots), kdev, vdev)
    model.create(0, plan.prefix_k, plan.prefix_v)
    for s in range(1, B):
        pool.fork(0, s)
        model.fork(0, s)
    for s in range(B):
        n = int(plan.suffix_lens[s])
        if n == 0:
            continue
        sl = np.array([pool.append(s)[0] for _ in range(n)], np.int64)
        ks = np.ascontiguousarray(plan.suffix_k[s].transpose(1, 0, 2))
        vs = np.ascontiguousarray(plan.suffix_v[s].transpose(1, 0, 2))
        pkv.pa_write_kv(to_dev(ks), to_dev(vs), to_dev(sl), kdev, vdev)
        model.k[s] = np.concatenate([model.k[s], plan.suffix_k[s]], axis=1)
        model.v[s] = np.concatenate([model.v[s], plan.suffix_v[s]], axis=1)
    assert all(pool.refcount(int(b)) == B for b in pool.table(0)[:prefix_blocks])

    seqs = list(range(B))
    rng = np.random.default_rng(77)
    total_copies = 0
    for step in range(plan.steps):
        announce("shared prefix step", step)
        # copy-on-write of 1% of the still-shared prefix references
        cands = [(s, lb) for s in seqs for lb, blk in enumerate(pool.table(s)[:prefix_blocks])
                 if pool.refcount(int(blk)) > 1]
        picks = plan.pick(cands)
        pairs = [pool.cow(s, lb) for s, lb in picks]
        pairs = np.array([p for p in pairs if p is not None], np.int64).reshape(-1, 2)
        assert len(pairs) == len(picks)  # every pick was shared, so each one copies
        total_copies += len(pairs)
        pkv.pa_copy_blocks(kdev, vdev, to_dev(pairs))
        # one new token per sequence
        q = plan.step_q()
        k_new, v_new = plan.step_tokens()
        slot_map, cow = pool.append_batch(seqs)
        assert cow.shape[0] == 0  # the tail block of every sequence is private
        pkv.pa_write_kv(to_dev(k_new), to_dev(v_new), to_dev(slot_map), kdev, vdev)
        for s in seqs:
            model.append(s, k_new[s], v_new[s])
        mb = max(len(pool.table(s)) for s in seqs)
        tables, lens = pool.tables(seqs, mb)
        assert all(int(lens[s]) == model.length(s) for s in seqs)

        # pools through the tables == contiguous runs, bitwise, every sequence
        kv16 = kdev.view(torch.int16)
        vv16 = vdev.view(torch.int16)
        for s in seqs:
            n = int(lens[s])
            gk = gather_rows(kv16, tables[s], n, bs).cpu().numpy().view(np.uint16)
            gv = gather_rows(vv16, tables[s], n, bs).cpu().numpy().view(np.uint16)
            assert np.array_equal(gk, model.k[s]) and np.array_equal(gv, model.v[s]), (step, s)
        # reference counts == table references
        counts = np.zeros(plan.num_blocks, np.int64)
        for s in seqs:
            for blk in pool.table(s):
                counts[int(blk)] += 1
        assert all(pool.refcount(b) == counts[b] for b in np.flatnonzero(counts))

        # decode against the oracle on the contiguous runs, every sequence
        dq, dt, dl = to_dev(q), to_dev(tables), to_dev(lens)
        sample = seqs
        refs = {}
        for s in sample:
            kc, vc, tb = seq_pool(model.k[s], model.v[s], bs)
            refs[s] = A.decode(q[s:s + 1], kc, vc, tb, np.array([model.length(s)], np.int32), plan.scale,
                               plan.dtype)[0]
        for part, out_dtype in ((0, torch.float32), (BAL, torch.float32), (BAL, None)):
            out = pkv.pa_decode(dq, kdev, vdev, dt, dl, int(lens.max()), plan.scale, partition_size=part,
                                out_dtype=out_dtype)
            got = out_to_f64(out)
            for s in sample:
                check_decode(got[s], refs[s], bf16_out=out_dtype is None)
    assert total_copies == plan.steps * plan.cow_per_step
    pool.close()
