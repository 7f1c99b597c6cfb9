"""pa_prefill_write on the GPU: the chunk's keys and values stored, then the
causal attention, as one call, bitwise equal to the two calls it stands for
(pa_write_kv, then pa_prefill) on both pools and on the output.

The pools hold NaN wherever no stored key lives, and in every slot the chunk
goes to, before the call: an attention that read a chunk key from the pools
before its store landed, or a store that missed its slot or wrote another,
changes the output or the pools.  Chunk starts that are not multiples of 4
put keys from the pools and from the chunk's rows in one 4-key load group.
Shapes with head_dim 128 and blocks of 8 tokens or more run one kernel; the
others run the two calls inside pa_prefill_write.
"""

import numpy as np
import pytest
import torch

import workloads as W

from gpu_cases import announce, to_dev, to_host

pytestmark = pytest.mark.gpu


def poison_chunk_slots(pc):
    c = pc.case
    bad = W.nan_value(c.dtype)
    for slot in pc.slot_mapping:
        if slot >= 0:
            blk, off = divmod(int(slot), c.block_size)
            c.k_cache[blk, :, off, :] = bad
            c.v_cache[blk, :, off, :] = bad


def bits(t):
    h = to_host(t)
    return h.view(np.uint16) if h.dtype == np.uint16 else h.view(np.uint32)


def check_fused_equals_two_calls(pkv, pc, out_dtypes=(torch.float32, None)):
    c = pc.case
    tables, lens, cu = to_dev(c.block_tables), to_dev(c.context_lens), to_dev(pc.cu_seqlens)
    q, kn, vn, slots = to_dev(pc.q), to_dev(pc.k_new), to_dev(pc.v_new), to_dev(pc.slot_mapping)
    for od in out_dtypes:
        announce(c.name, "prefill_write out", od)
        ka, va = to_dev(c.k_cache), to_dev(c.v_cache)
        kb, vb = to_dev(c.k_cache), to_dev(c.v_cache)
        pkv.pa_write_kv(kn, vn, slots, ka, va)
        oa = pkv.pa_prefill(q, ka, va, tables, lens, cu, pc.max_query_len, c.max_context, c.scale, out_dtype=od)
        ob = pkv.pa_prefill_write(kn, vn, slots, q, kb, vb, tables, lens, cu, pc.max_query_len, c.max_context,
                                  c.scale, out_dtype=od)
        torch.cuda.synchronize()
        assert np.array_equal(bits(ka), bits(kb)), "key pools differ"
        assert np.array_equal(bits(va), bits(vb)), "value pools differ"
        ga, gb = bits(oa), bits(ob)
        assert np.array_equal(ga, gb), f"{int((ga != gb).sum())} outputs differ"
        if od is torch.float32:
            assert np.isfinite(to_host(oa)).all(), "non-finite output"  # no poison reached the attention


LENS = [1, 15, 16, 17, 100, 333, 64, 40, 700, 9]
CHUNKS = [1, 15, 3, 17, 37, 50, 64, 0, 300, 9]  # starts 0, 0, 13, 0, 63, 283, 0, -, 400, 0


@pytest.mark.parametrize("hq,hkv,d,bs", [(32, 8, 128, 16), (32, 8, 128, 8), (16, 8, 128, 256), (64, 8, 128, 32),
                                         (8, 8, 128, 16), (16, 8, 128, 16), (32, 8, 64, 16), (32, 8, 128, 4)])
def test_chunks_after_cached_contexts(gpu_lib, hq, hkv, d, bs):
    pc = W.make_prefill(f"prefill_write_{hq}_{hkv}_{d}_{bs}", seed=hq + d + bs, context_lens=LENS,
                        chunk_lens=CHUNKS, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                        poison=True)
    poison_chunk_slots(pc)
    check_fused_equals_two_calls(gpu_lib, pc)


@pytest.mark.parametrize("seed", range(400, 410))
def test_random_batches(gpu_lib, seed):
    # seeded random batches: 2 to 64 sequences, whole prompts (chunk =
    # context), chunks after cached keys (the fused kernel's input-row,
    # mixed and pool loads), empty chunks and chunks past their context
    rng = np.random.default_rng(seed)
    nseq = int(rng.choice([2, 5, 17, 33, 64]))
    g = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([4, 8, 16, 32, 256]))
    lens = [int(x) for x in rng.integers(1, 900, size=nseq)]
    chunks = []
    for l in lens:
        kind = rng.integers(4)
        chunks.append(l if kind == 0 else int(rng.integers(0, min(l, 300) + 1)) if kind < 3 else l + int(rng.integers(1, 9)))
    pc = W.make_prefill(f"prefill_write_random_{seed}", seed=seed, context_lens=lens, chunk_lens=chunks,
                        num_q_heads=8 * g, num_kv_heads=8, head_dim=d, block_size=bs, poison=True)
    poison_chunk_slots(pc)
    check_fused_equals_two_calls(gpu_lib, pc)


def test_whole_prompts_many_tiles(gpu_lib):
    pc = W.make_prefill("prefill_write_prompts", seed=41, context_lens=[1500, 37, 900, 4], num_q_heads=32,
                        num_kv_heads=8, head_dim=128, block_size=16, poison=True)
    poison_chunk_slots(pc)
    check_fused_equals_two_calls(gpu_lib, pc)


def test_chunk_longer_than_context(gpu_lib):
    # positions below 0 attend to nothing and have no slot (-1): only the
    # chunk's rows at positions >= 0 are stored
    pc = W.make_prefill("prefill_write_long_chunk", seed=43, context_lens=[5, 20, 33], chunk_lens=[9, 25, 40],
                        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, poison=True)
    assert (pc.slot_mapping < 0).any()
    poison_chunk_slots(pc)
    check_fused_equals_two_calls(gpu_lib, pc)


def test_store_only_when_nothing_attends(gpu_lib):
    # max_query_len == 0: the rows are stored, no attention runs
    pc = W.make_prefill("prefill_write_store_only", seed=47, context_lens=[20, 40], num_q_heads=32,
                        num_kv_heads=8, head_dim=128, block_size=16, poison=True)
    poison_chunk_slots(pc)
    c = pc.case
    ka, va = to_dev(c.k_cache), to_dev(c.v_cache)
    kb, vb = to_dev(c.k_cache), to_dev(c.v_cache)
    kn, vn, slots = to_dev(pc.k_new), to_dev(pc.v_new), to_dev(pc.slot_mapping)
    gpu_lib.pa_write_kv(kn, vn, slots, ka, va)
    out = torch.zeros((pc.num_tokens, 32, 128), dtype=torch.float32, device="cuda")
    gpu_lib.pa_prefill_write(kn, vn, slots, to_dev(pc.q), kb, vb, to_dev(c.block_tables), to_dev(c.context_lens),
                             to_dev(pc.cu_seqlens), 0, c.max_context, c.scale, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ka), bits(kb)) and np.array_equal(bits(va), bits(vb))
    assert not to_host(out).any()


@pytest.mark.parametrize("name", ["prefill_llama3_8b", "prefill_chunked"])
def test_full_size(gpu_lib, name):
    pc = W.c6_prefill_llama8b() if name == "prefill_llama3_8b" else W.c6_chunked_prefill()
    announce("prefill_write full", name)
    check_fused_equals_two_calls(gpu_lib, pc, out_dtypes=(torch.float32,))
