"""Every output row of the full-size decode workloads against the fp64
oracle, in each launch configuration the benchmark times.

For each workload (Llama-3-8B-shaped batch of 64; 8 x 32,768-token contexts;
256 MHA sequences of lognormal lengths at block sizes 8, 16 and 32), after
the step's one-token-per-sequence store:

* pa_decode with an fp32 output: every element within 1e-4 of the oracle
  (bf16 inputs are exact in the oracle, so only fp32 accumulation order and
  exp2 remain);
* pa_decode with a bf16 output: every element within 2e-2 + 1e-2 |ref|, and
  bitwise the fp32 output rounded to nearest even;
* pa_decode_write (store and attend in one call, the benchmarked launch):
  pools and output bitwise those of pa_write_kv followed by pa_decode, and
  every element against the oracle.

Partition sizes: 0 (one workgroup per sequence and KV head), the balanced
split (the benchmark's default), and the workload's fixed partition size
where it names one (512 tokens for the long contexts).

Pages: foundry "PagedAttention" ops page, How it works (attention reads the
whole context through the block table; storage is transparent to the math).
"""

import numpy as np
import pytest
import torch

import workloads as W

from gpu_cases import (DevCase, announce, check_bf16_is_rounded_f32, check_decode, oracle_after_write,
                       oracle_decode_all, out_to_f64, to_dev)

pytestmark = pytest.mark.gpu

BAL = -1

CASES = {
    "llama3_8b_b64": (lambda: W.c2_llama8b_b64(), [BAL, 0, 512]),
    "long_ctx_32k": (lambda: W.c3_long_context(), [BAL, 512, 0]),
    "mha_b256_bs8": (lambda: W.c5_mha_sweep(block_size=8), [BAL, 0]),
    "mha_b256_bs16": (lambda: W.c5_mha_sweep(block_size=16), [BAL, 0, 256]),
    "mha_b256_bs32": (lambda: W.c5_mha_sweep(block_size=32), [BAL, 0]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_every_row(gpu_lib, name):
    pkv = gpu_lib
    make, parts = CASES[name]
    announce("full size", name, "drawing inputs")
    case = make()
    announce("full size", name, "oracle over", case.num_seqs, "x", case.num_q_heads, "rows")
    kc, vc = oracle_after_write(case)
    ref = oracle_decode_all(case, kc, vc)
    del kc, vc

    # two-call path on one device copy: store, then every partition mode
    dc = DevCase(case)
    dc.write(pkv)
    two_call_f32 = {}
    for p in parts:
        announce("full size", name, "P", p)
        o32 = dc.decode(pkv, partition_size=p, out_dtype=torch.float32)
        obf = dc.decode(pkv, partition_size=p)
        torch.cuda.synchronize()
        check_decode(out_to_f64(o32), ref, bf16_out=False)
        check_decode(out_to_f64(obf), ref, bf16_out=True)
        check_bf16_is_rounded_f32(obf, o32)
        two_call_f32[p] = o32
        del obf
    k_two, v_two = dc.k_cache, dc.v_cache
    del dc

    # the benchmarked launch: store and attend in one call (balanced split)
    announce("full size", name, "decode_write")
    fc = DevCase(case)
    out = pkv.pa_decode_write(fc.k_new, fc.v_new, fc.slot_mapping, fc.q, fc.k_cache, fc.v_cache,
                              fc.block_tables, fc.context_lens, case.max_context, case.scale,
                              partition_size=BAL, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(fc.k_cache.view(torch.int16), k_two.view(torch.int16))
    assert torch.equal(fc.v_cache.view(torch.int16), v_two.view(torch.int16))
    assert torch.equal(out, two_call_f32[BAL])
    check_decode(out_to_f64(out), ref, bf16_out=False)
    del fc, out, k_two, v_two, two_call_f32
    torch.cuda.empty_cache()
