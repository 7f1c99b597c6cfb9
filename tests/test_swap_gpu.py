"""Swap-out / swap-in of sequences between the device pool and a pinned host
swap pool, on the GPU.

The host manager decides the block moves (pa_seq_swap_out / pa_seq_swap_in),
pa_swap_blocks copies the blocks across the bus, and in between other
sequences reuse the device blocks that were freed (and write new data into
them).  After every step the pools, gathered through the manager's tables,
equal each resident sequence's logical K/V (bitwise), and the decode over
the swapped-back sequences equals the fp64 oracle.

Pages: foundry "PagedAttention" ops page, How it works and Trade-offs (a
preempted sequence's blocks can be swapped out to CPU memory and back).
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A

from gpu_cases import announce, check_decode, out_to_f64, to_dev

pytestmark = pytest.mark.gpu

HKV, HQ, D, BS = 8, 32, 128, 16


def rows(cache16, table, n):
    """[Hkv][n][d] int16 rows of a sequence read through its table."""
    nb = W.ceil_div(n, BS)
    blk = cache16[torch.as_tensor(np.asarray(table[:nb], np.int64), device=cache16.device)]
    return blk.permute(1, 0, 2, 3).reshape(HKV, nb * BS, D)[:, :n].cpu().numpy().view(np.uint16)


def test_swap_out_reuse_swap_in(gpu_lib):
    pkv = gpu_lib
    rng = np.random.default_rng(404)
    nb_dev, nb_host = 48, 40
    pool = pkv.BlockPool(nb_dev, BS, rng.permutation(nb_dev))
    pool.set_swap_space(nb_host, rng.permutation(nb_host))
    kdev = torch.zeros((nb_dev, HKV, BS, D), dtype=torch.bfloat16, device="cuda")
    vdev = torch.zeros_like(kdev)
    khost = torch.zeros((nb_host, HKV, BS, D), dtype=torch.bfloat16).pin_memory()
    vhost = torch.zeros_like(khost).pin_memory()
    model = {}

    def write(seq, n):
        """Append n tokens of fresh K/V to seq (through the manager and pa_write_kv)."""
        k = W.normal(rng, (n, HKV, D), W.BF16)
        v = W.normal(rng, (n, HKV, D), W.BF16)
        slots, pairs = [], []
        for _ in range(n):
            slot, pair = pool.append(seq)
            slots.append(slot)
            if pair is not None:
                pairs.append(pair)
        if pairs:
            pkv.pa_copy_blocks(kdev, vdev, to_dev(np.array(pairs, np.int64).reshape(-1, 2)))
        pkv.pa_write_kv(to_dev(k), to_dev(v), to_dev(np.array(slots, np.int64)), kdev, vdev)
        mk, mv = model.get(seq, (np.zeros((HKV, 0, D), np.uint16),) * 2)
        model[seq] = (np.concatenate([mk, k.transpose(1, 0, 2)], axis=1),
                      np.concatenate([mv, v.transpose(1, 0, 2)], axis=1))

    def swap(pairs, out):
        p = to_dev(np.asarray(pairs, np.int64).reshape(-1, 2))
        if out:
            pkv.pa_swap_blocks(kdev, vdev, khost, vhost, p)
        else:
            pkv.pa_swap_blocks(khost, vhost, kdev, vdev, p)

    def check(seqs):
        torch.cuda.synchronize()
        for s in seqs:
            n = pool.length(s)
            assert not pool.is_swapped(s)
            t = pool.table(s)
            assert np.array_equal(rows(kdev.view(torch.int16), t, n), model[s][0]), s
            assert np.array_equal(rows(vdev.view(torch.int16), t, n), model[s][1]), s

    announce("swap: build")
    pool.create(1, 0)
    write(1, 150)             # A: 10 blocks
    pool.create(2, 0)
    write(2, 90)              # B: 6 blocks
    pool.fork(1, 3)           # C shares A's blocks
    model[3] = model[1]
    write(3, 20)              # C: copy-on-write of the shared tail block, then new blocks
    check([1, 2, 3])

    announce("swap: out A (shared with C) and B")
    free0 = pool.num_free()
    swap(pool.swap_out(1), out=True)
    assert pool.num_free() == free0 + 1          # only A's private tail block came back
    swap(pool.swap_out(2), out=True)
    assert pool.num_free() == free0 + 1 + 6
    with pytest.raises(pkv.PoolStateError):
        pool.append(2)
    check([3])

    announce("swap: reuse the freed device blocks")
    pool.create(4, 0)
    write(4, pool.num_free() * BS - 5)           # takes every free block, B's old ones included
    check([3, 4])
    with pytest.raises(pkv.PoolExhausted):       # no room to bring A back yet
        pool.swap_in(1)

    announce("swap: in B, then A")
    pool.release(4)
    del model[4]
    swap(pool.swap_in(2), out=False)
    swap(pool.swap_in(1), out=False)
    check([1, 2, 3])
    write(1, 3)               # A keeps growing after swap-in
    check([1, 2, 3])

    announce("swap: decode after swap-in")
    seqs = [1, 2, 3]
    mb = max(len(pool.table(s)) for s in seqs)
    tables, lens = pool.tables(seqs, mb)
    q = W.normal(rng, (len(seqs), HQ, D), W.BF16)
    out = pkv.pa_decode(to_dev(q), kdev, vdev, to_dev(tables), to_dev(lens), int(lens.max()), 0.088,
                        partition_size=-1, out_dtype=torch.float32)
    got = out_to_f64(out)
    for i, s in enumerate(seqs):
        n = int(lens[i])
        nbk = W.ceil_div(n, BS)
        kc = np.zeros((nbk, HKV, BS, D), np.uint16)
        vc = np.zeros_like(kc)
        for t in range(n):
            kc[t // BS, :, t % BS] = model[s][0][:, t]
            vc[t // BS, :, t % BS] = model[s][1][:, t]
        ref = A.decode(q[i:i + 1], kc, vc, np.arange(nbk, dtype=np.int32)[None], np.array([n], np.int32), 0.088,
                       W.BF16)[0]
        check_decode(got[i], ref, bf16_out=False)
    pool.close()
