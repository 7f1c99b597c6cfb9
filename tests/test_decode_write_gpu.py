"""pa_decode_write on the GPU: storing the new tokens and attending in one call.

The pools after the call and the output equal those of pa_write_kv followed
by pa_decode, bitwise, on every path: the balanced split (one kernel: the
tokens are stored while it runs and position context_lens[i] - 1 is read
from the input rows) and the paths that run the two kernels.  The output is
also held to the fp64 oracle on the pools after the write.  Cases are
poisoned: unused blocks, the tails of last blocks and the write slots hold
NaN before the call, so a newest position read from the pool before its
store (or never stored) shows.

Pages: foundry "PagedAttention" ops page, How it works (the new token's key
and value go into the sequence's current block; attention reads the whole
context through the block table).
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A

from gpu_cases import DevCase, announce, check_decode, oracle_after_write, out_to_f64, small_bf16_case, to_dev

pytestmark = pytest.mark.gpu

BAL = -1


def both_ways(pkv, case, partition, out_dtype=None, max_context=None, tokens=None):
    """(pools, out) of write-then-decode and of pa_decode_write on fresh copies."""
    mc = case.max_context if max_context is None else max_context
    t = case.num_seqs if tokens is None else tokens
    res = []
    for fused in (False, True):
        dc = DevCase(case)
        k_new, v_new, slots = dc.k_new[:t], dc.v_new[:t], dc.slot_mapping[:t]
        if fused:
            out = pkv.pa_decode_write(k_new, v_new, slots, dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                      dc.context_lens, mc, case.scale, partition_size=partition,
                                      out_dtype=out_dtype)
        else:
            pkv.pa_write_kv(k_new, v_new, slots, dc.k_cache, dc.v_cache)
            out = pkv.pa_decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, mc,
                                case.scale, partition_size=partition, out_dtype=out_dtype)
        torch.cuda.synchronize()
        res.append((dc.k_cache, dc.v_cache, out))
    return res


def assert_same(res):
    (ka, va, oa), (kb, vb, ob) = res
    assert torch.equal(ka.view(torch.int16) if ka.dtype == torch.bfloat16 else ka.view(torch.int32),
                       kb.view(torch.int16) if kb.dtype == torch.bfloat16 else kb.view(torch.int32))
    assert torch.equal(va.view(torch.int16) if va.dtype == torch.bfloat16 else va.view(torch.int32),
                       vb.view(torch.int16) if vb.dtype == torch.bfloat16 else vb.view(torch.int32))
    # NaN-free outputs compared bitwise
    assert not torch.isnan(ob).any()
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("hq,hkv,d,bs", [(32, 8, 128, 16), (64, 8, 128, 8), (32, 4, 64, 32),
                                         (16, 2, 256, 16), (16, 4, 128, 4), (32, 8, 128, 64)])
def test_fused_equals_write_then_decode(gpu_lib, hq, hkv, d, bs):
    case = small_bf16_case(81 + bs, num_seqs=9, hi=900, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                           block_size=bs, poison=True)
    kc, vc = oracle_after_write(case)
    ref = A.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
    for p in (BAL, 0, 4 * bs):
        for od in (None, torch.float32):
            announce("decode_write", hq, hkv, d, bs, "P", p, "out", od)
            res = both_ways(gpu_lib, case, p, od)
            assert_same(res)
            check_decode(out_to_f64(res[1][2]), ref, bf16_out=od is None)


def test_fused_with_empty_sequences_and_many_of_them(gpu_lib):
    rng = np.random.default_rng(91)
    lens = rng.integers(0, 200, size=300)
    lens[::13] = 0
    lens[7] = 2000
    case = W.make_case("write_many", seed=92, dtype=W.BF16, context_lens=lens, num_q_heads=32,
                       num_kv_heads=8, head_dim=128, block_size=16, poison=True)
    kc, vc = oracle_after_write(case)
    ref = A.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
    announce("decode_write many")
    res = both_ways(gpu_lib, case, BAL, torch.float32)
    assert_same(res)
    check_decode(out_to_f64(res[1][2]), ref, bf16_out=False)


def test_fused_fallbacks(gpu_lib):
    """Fewer tokens than sequences, and lengths clamped by max_context_len:
    still the two calls' result."""
    case = small_bf16_case(95, num_seqs=8, lo=100, hi=600, poison=False)
    announce("decode_write half the tokens")
    assert_same(both_ways(gpu_lib, case, BAL, torch.float32, tokens=case.num_seqs // 2))
    announce("decode_write clamped lengths")
    assert_same(both_ways(gpu_lib, case, BAL, torch.float32, max_context=300))


def test_fused_no_sequences_still_stores(gpu_lib):
    case = small_bf16_case(97, num_seqs=3)
    dc = DevCase(case)
    ref = DevCase(case)
    ref.write(gpu_lib)
    q0 = dc.q[:0]
    gpu_lib.pa_decode_write(dc.k_new, dc.v_new, dc.slot_mapping, q0, dc.k_cache, dc.v_cache,
                            dc.block_tables[:0], dc.context_lens[:0], case.max_context, case.scale,
                            partition_size=BAL)
    torch.cuda.synchronize()
    assert torch.equal(dc.k_cache.view(torch.int16), ref.k_cache.view(torch.int16))
    assert torch.equal(dc.v_cache.view(torch.int16), ref.v_cache.view(torch.int16))
