"""pa_write_kv and pa_copy_blocks on the GPU: bitwise against the oracle."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import kvcache as KV

from gpu_cases import DevCase, announce, oracle_after_write, to_dev, to_host

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("maker", ["tiny_f32", "small_bf16", "small_bf16_bs8_poison"])
def test_write_matches_oracle_whole_pool(gpu_lib, maker):
    announce("write", maker)
    if maker == "tiny_f32":
        case = W.c1_tiny_f32()
    elif maker == "small_bf16":
        case = W.c2_llama8b_b64(seed=12, num_seqs=9, lo=1, hi=300)
    else:
        case = W.c5_mha_sweep(seed=13, num_seqs=7, block_size=8, poison=True)
    # pad with skipped tokens
    case.slot_mapping[::3] = -1
    dc = DevCase(case)
    dc.write(gpu_lib)
    torch.cuda.synchronize()
    kc, vc = oracle_after_write(case)
    assert same_bits(to_host(dc.k_cache), kc)
    assert same_bits(to_host(dc.v_cache), vc)


def test_write_many_tokens_and_out_of_pool_slots(gpu_lib):
    announce("write bulk")
    rng = np.random.default_rng(21)
    nb, hkv, bs, d = 40, 4, 16, 64
    kc = W.normal(rng, (nb, hkv, bs, d), W.BF16)
    vc = W.normal(rng, (nb, hkv, bs, d), W.BF16)
    slots = rng.permutation(nb * bs)[:500].astype(np.int64)
    slots[::7] = -5
    slots[3] = nb * bs + 11  # outside the pool: skipped
    k = W.normal(rng, (500, hkv, d), W.BF16)
    v = W.normal(rng, (500, hkv, d), W.BF16)
    dk, dv = to_dev(kc), to_dev(vc)
    gpu_lib.pa_write_kv(to_dev(k), to_dev(v), to_dev(slots), dk, dv)
    torch.cuda.synchronize()
    ok = slots.copy()
    ok[3] = -1
    ek, ev = KV.write_kv(kc, vc, k, v, ok, bs)
    assert same_bits(to_host(dk), ek) and same_bits(to_host(dv), ev)


def test_write_zero_tokens_is_noop(gpu_lib):
    announce("write empty")
    kc = torch.zeros((4, 2, 8, 64), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    empty = torch.zeros((0, 2, 64), dtype=torch.float32, device="cuda")
    gpu_lib.pa_write_kv(empty, empty, torch.zeros(0, dtype=torch.int64, device="cuda"), kc, vc)
    torch.cuda.synchronize()
    assert not kc.any()


@pytest.mark.parametrize("dtype,hkv,bs,d", [(W.F32, 4, 16, 64), (W.BF16, 8, 16, 128), (W.BF16, 40, 8, 128),
                                            (W.BF16, 2, 32, 256)])
def test_copy_blocks_matches_oracle(gpu_lib, dtype, hkv, bs, d):
    announce("copy", dtype, hkv, bs, d)
    rng = np.random.default_rng(hkv * 100 + bs)
    nb = 64
    kc = W.normal(rng, (nb, hkv, bs, d), dtype)
    vc = W.normal(rng, (nb, hkv, bs, d), dtype)
    perm = rng.permutation(nb)
    src = perm[:12].copy()
    src[5] = src[2]  # a source used twice
    dst = perm[12:24]
    pairs = np.stack([src, dst], axis=1).astype(np.int64)
    dk, dv = to_dev(kc), to_dev(vc)
    gpu_lib.pa_copy_blocks(dk, dv, to_dev(pairs))
    torch.cuda.synchronize()
    ek, ev = KV.copy_blocks(kc, vc, pairs)
    assert same_bits(to_host(dk), ek) and same_bits(to_host(dv), ev)


def test_copy_blocks_skips_out_of_pool_pairs(gpu_lib):
    announce("copy out-of-pool")
    rng = np.random.default_rng(5)
    kc = W.normal(rng, (8, 2, 16, 64), W.BF16)
    vc = W.normal(rng, (8, 2, 16, 64), W.BF16)
    pairs = np.array([[1, 2], [9, 3], [4, -1], [5, 6]], np.int64)
    dk, dv = to_dev(kc), to_dev(vc)
    gpu_lib.pa_copy_blocks(dk, dv, to_dev(pairs))
    torch.cuda.synchronize()
    ek, ev = KV.copy_blocks(kc, vc, pairs[[0, 3]])
    assert same_bits(to_host(dk), ek) and same_bits(to_host(dv), ev)


# --- full-size workloads: exact checks done on the device side --------------------

def _changed_rows(before, after):
    """Indices (block, head, slot) whose row differs bitwise."""
    b = before.view(torch.int16) if before.dtype == torch.bfloat16 else before.view(torch.int32)
    a = after.view(torch.int16) if after.dtype == torch.bfloat16 else after.view(torch.int32)
    diff = (a != b).any(dim=-1)
    return torch.nonzero(diff).cpu().numpy()


@pytest.mark.parametrize("name", ["llama3_8b_b64", "long_ctx_32k", "mha_b256_bs8", "mha_b256_bs16",
                                  "mha_b256_bs32"])
def test_write_full_size(gpu_lib, name):
    announce("write full", name)
    if name == "llama3_8b_b64":
        case = W.c2_llama8b_b64()
    elif name == "long_ctx_32k":
        case = W.c3_long_context()
    else:
        case = W.c5_mha_sweep(block_size=int(name.split("bs")[1]))
    dc = DevCase(case)
    k0, v0 = dc.k_cache.clone(), dc.v_cache.clone()
    dc.write(gpu_lib)
    torch.cuda.synchronize()
    bs = case.block_size
    expect = set()
    for s, slot in enumerate(case.slot_mapping):
        blk, off = divmod(int(slot), bs)
        for h in range(case.num_kv_heads):
            expect.add((blk, h, off))
    for before, after, new in ((k0, dc.k_cache, case.k_new), (v0, dc.v_cache, case.v_new)):
        changed = {tuple(x) for x in _changed_rows(before, after)}
        assert changed <= expect  # nothing else moved (a row may equal what was there)
        got = to_host(after[torch.as_tensor([e[0] for e in sorted(expect)]),
                            torch.as_tensor([e[1] for e in sorted(expect)]),
                            torch.as_tensor([e[2] for e in sorted(expect)])])
        inv = {}
        for s, slot in enumerate(case.slot_mapping):
            blk, off = divmod(int(slot), bs)
            for h in range(case.num_kv_heads):
                inv[(blk, h, off)] = new[s, h]
        want = np.stack([inv[e] for e in sorted(expect)])
        assert same_bits(got, want)
    del dc, k0, v0
    torch.cuda.empty_cache()


def test_copy_full_size_pool(gpu_lib):
    """1% of a Llama-3-8B-shaped pool's blocks copied in one call (328 pairs)."""
    announce("copy full")
    case = W.c2_llama8b_b64()
    rng = np.random.default_rng(44)
    perm = rng.permutation(case.num_blocks)
    pairs = np.stack([perm[:328], perm[328:656]], axis=1).astype(np.int64)
    dc = DevCase(case)
    k0, v0 = dc.k_cache.clone(), dc.v_cache.clone()
    gpu_lib.pa_copy_blocks(dc.k_cache, dc.v_cache, to_dev(pairs))
    torch.cuda.synchronize()
    src = torch.as_tensor(pairs[:, 0], device="cuda")
    dst = torch.as_tensor(pairs[:, 1], device="cuda")
    for before, after in ((k0, dc.k_cache), (v0, dc.v_cache)):
        assert torch.equal(after[dst].view(torch.int16), before[src].view(torch.int16))
        keep = torch.ones(case.num_blocks, dtype=torch.bool, device="cuda")
        keep[dst] = False
        assert torch.equal(after[keep].view(torch.int16), before[keep].view(torch.int16))
    del dc, k0, v0
    torch.cuda.empty_cache()
