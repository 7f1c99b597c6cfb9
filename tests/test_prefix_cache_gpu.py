"""Prefix-cached prompts on the GPU: requests that share a prompt prefix reuse
its KV blocks through the host manager's prefix cache, store and attend only
their uncached tokens, and still get what a full prefill of the whole prompt
gives (the fp64 prefill oracle over each request's full logical KV).

The pools start as NaN everywhere, so a request that attended to a slot its
cache hit promised but nobody wrote would produce NaN.

Pages: aimodelwiki "PagedAttention" glossary entry, prefix-caching paragraph
(requests with a common prompt prefix reuse its KV pages), and the foundry
"PagedAttention" ops page, How it works (tokens are stored block by block
through the table, and attention reads KV through it).
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import prefill as P

from gpu_cases import announce, out_to_f64, to_dev
from test_prefill_gpu import check_prefill, out_to_f64_np

pytestmark = pytest.mark.gpu

HKV, HQ, D, BS = 8, 32, 128, 16
SCALE = float(np.float32(1.0 / np.sqrt(D)))
NAN_BF16 = 0x7FC0


def logical_pool(k_rows):
    """[n][Hkv][d] rows -> a private contiguous pool [nb][Hkv][bs][d] and its table."""
    n = k_rows.shape[0]
    nb = W.ceil_div(n, BS)
    pad = np.zeros((nb * BS, HKV, D), k_rows.dtype)
    pad[:n] = k_rows
    return pad.reshape(nb, BS, HKV, D).transpose(0, 2, 1, 3).copy(), np.arange(nb, dtype=np.int32)


def test_prefix_reuse_repeat_and_eviction(gpu_lib):
    pkv = gpu_lib
    rng = np.random.default_rng(808)
    nb = 12
    pool = pkv.BlockPool(nb, BS, rng.permutation(nb))
    pool.enable_prefix_cache()
    kdev = torch.full((nb, HKV, BS, D), NAN_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vdev = torch.full_like(kdev.view(torch.int16), NAN_BF16).view(torch.bfloat16)

    # token ids -> K/V rows: one row per (position, token), the same for every request
    prefix = rng.integers(0, 1000, 40).astype(np.int32)
    kv_of = {}

    def kv_rows(tokens):
        ks, vs = [], []
        for pos, tok in enumerate(tokens):
            key = (pos, int(tok))
            if key not in kv_of:
                kv_of[key] = (W.normal(rng, (HKV, D), W.BF16), W.normal(rng, (HKV, D), W.BF16))
            ks.append(kv_of[key][0])
            vs.append(kv_of[key][1])
        return np.stack(ks), np.stack(vs)

    def admit(seq, tokens, expect_cached):
        """create_cached, store the uncached tokens, prefill their queries,
        compare with the oracle's full prefill of the whole prompt."""
        announce("prefix cache: admit", seq, len(tokens), "tokens")
        cached = pool.create_cached(seq, tokens)
        assert cached == expect_cached
        n = len(tokens)
        new = n - cached
        k, v = kv_rows(tokens)
        slots = np.asarray(pool.slots(seq, cached, new), np.int64)
        pkv.pa_write_kv(to_dev(k[cached:]), to_dev(v[cached:]), to_dev(slots), kdev, vdev)
        q = W.normal(rng, (new, HQ, D), W.BF16)
        tables, lens = pool.tables([seq], W.ceil_div(n, BS))
        cu = np.array([0, new], np.int32)
        out = pkv.pa_prefill(to_dev(q), kdev, vdev, to_dev(tables), to_dev(lens), to_dev(cu), new, n, SCALE,
                             out_dtype=torch.float32)
        kc, table = logical_pool(k)
        vc, _ = logical_pool(v)
        ref = P.prefill(q, kc, vc, table[None], np.array([n], np.int32), cu, SCALE, W.BF16)
        check_prefill(out_to_f64(out), ref, float(np.max(np.abs(out_to_f64_np(vc)))), bf16_out=False)
        return k, v

    a_tokens = np.concatenate([prefix, [7, 7, 7, 1, 2, 3, 4]]).astype(np.int32)
    b_tokens = np.concatenate([prefix, np.arange(500, 520)]).astype(np.int32)
    admit(1, a_tokens, 0)            # blocks 0-1 of the prompt registered
    kb, vb = admit(2, b_tokens, 32)  # shares them, stores 28 tokens
    ta, tb = pool.table(1), pool.table(2)
    assert list(ta[:2]) == list(tb[:2]) and ta[2] != tb[2]

    announce("prefix cache: shared blocks untouched")
    torch.cuda.synchronize()
    shared = torch.as_tensor(np.asarray(ta[:2], np.int64), device="cuda")
    rows = kdev[shared].permute(0, 2, 1, 3).reshape(32, HKV, D).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(rows, kb[:32])

    pool.release(1)
    pool.release(2)
    # A's partial block went back to the free stack; B's third block is full, so it stays cached
    assert [int(x) for x in pool.lru_order()] == [int(ta[0]), int(ta[1]), int(tb[2])]
    admit(3, b_tokens, 48)           # the same prompt again: three full blocks cached, 12 tokens stored
    pool.release(3)

    announce("prefix cache: eviction under pressure")
    pool.create(9, pool.num_free() * BS)  # takes the free stack ...
    pool.release(9)
    pool.create(9, (pool.num_free() + pool.num_cached()) * BS)  # ... and then every cached block
    assert pool.num_cached() == 0
    pool.release(9)
    admit(4, a_tokens, 0)            # the prefix was evicted: computed again
    pool.close()


def test_batched_admission_one_prefill_call(gpu_lib):
    """Requests admitted together (pa_seq_create_cached_batch) with different
    cached prefix lengths (none, one block, all full blocks, a repeat of a
    whole prompt) are stored and prefilled in one pa_prefill call over all of
    them; each request's rows equal the oracle's prefill of its whole prompt."""
    pkv = gpu_lib
    rng = np.random.default_rng(909)
    nb = 64
    pool = pkv.BlockPool(nb, BS, rng.permutation(nb))
    pool.enable_prefix_cache()
    kdev = torch.full((nb, HKV, BS, D), NAN_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vdev = torch.full_like(kdev.view(torch.int16), NAN_BF16).view(torch.bfloat16)
    kv_of = {}

    def kv_rows(tokens):
        ks, vs = [], []
        for pos, tok in enumerate(tokens):
            key = (pos, int(tok))
            if key not in kv_of:
                kv_of[key] = (W.normal(rng, (HKV, D), W.BF16), W.normal(rng, (HKV, D), W.BF16))
            ks.append(kv_of[key][0])
            vs.append(kv_of[key][1])
        return np.stack(ks), np.stack(vs)

    sys_prompt = rng.integers(0, 1000, 50).astype(np.int32)  # 3 full blocks + 2 tokens
    first = [np.concatenate([sys_prompt, rng.integers(2000, 3000, 9)]).astype(np.int32),
             rng.integers(5000, 6000, 37).astype(np.int32)]

    def admit(seqs, prompts, expect):
        announce("prefix cache batch: admit", seqs)
        cached, slots, refused = pool.create_cached_batch(seqs, prompts)
        assert refused is None and cached.tolist() == expect
        ks, vs, qs, cu, lens, refs = [], [], [], [0], [], []
        for c, toks in zip(cached.tolist(), prompts):
            k, v = kv_rows(toks)
            ks.append(k[c:])
            vs.append(v[c:])
            q = W.normal(rng, (len(toks) - c, HQ, D), W.BF16)
            qs.append(q)
            cu.append(cu[-1] + len(toks) - c)
            lens.append(len(toks))
            kc, table = logical_pool(k)
            vc, _ = logical_pool(v)
            refs.append((P.prefill(q, kc, vc, table[None], np.array([len(toks)], np.int32),
                                   np.array([0, len(toks) - c], np.int32), SCALE, W.BF16),
                         float(np.max(np.abs(out_to_f64_np(vc))))))
        assert slots.shape[0] == cu[-1]
        pkv.pa_write_kv(to_dev(np.concatenate(ks)), to_dev(np.concatenate(vs)), to_dev(slots), kdev, vdev)
        mb = max(W.ceil_div(n, BS) for n in lens)
        tables, tl = pool.tables(seqs, mb)
        assert tl.tolist() == lens
        cu = np.array(cu, np.int32)
        out = pkv.pa_prefill(to_dev(np.concatenate(qs)), kdev, vdev, to_dev(tables), to_dev(tl), to_dev(cu),
                             int(np.max(np.diff(cu))), max(lens), SCALE, out_dtype=torch.float32)
        got = out_to_f64(out)
        for i, (ref, vmax) in enumerate(refs):
            check_prefill(got[cu[i]:cu[i + 1]], ref, vmax, bf16_out=False)

    admit([1, 2], first, [0, 0])
    second = [np.concatenate([sys_prompt, rng.integers(7000, 8000, 20)]).astype(np.int32),  # 3 blocks cached
              np.concatenate([sys_prompt[:16], rng.integers(9000, 9500, 30)]).astype(np.int32),  # 1 block
              first[1].copy(),  # the whole prompt again: its 2 full blocks cached
              rng.integers(10000, 11000, 5).astype(np.int32)]  # nothing cached
    admit([3, 4, 5, 6], second, [48, 16, 32, 0])
    pool.close()
