"""pa_decode_write_noalloc (the decode for callers that cannot allocate: a
static scratch array in the library instead of a workspace) against
pa_decode_write with a caller's workspace, through the C ABI.

Two calls in a row, the second on a smaller batch (the scratch keeps the
first call's contents, which must not matter), on the balanced split, a
fixed partition size and the vector-ALU kernel's partitions: pools and
output bitwise those of pa_decode_write, and the output within the stated
tolerance of the fp64 oracle.  A call that needs more scratch than the array
holds is refused and enqueues nothing.
"""

import numpy as np
import pytest
import torch

import workloads as W

from gpu_cases import DevCase, announce, check_decode, oracle_after_write, oracle_decode_all, out_to_f64, \
    small_bf16_case

pytestmark = pytest.mark.gpu

BAL = -1


def _pair(pkv, case, partition, out_dtype):
    """(reference pools and out from pa_decode_write with a workspace,
    pools and out from pa_decode_write_noalloc), each on a fresh copy."""
    ref = DevCase(case)
    ro = pkv.pa_decode_write(ref.k_new, ref.v_new, ref.slot_mapping, ref.q, ref.k_cache, ref.v_cache,
                             ref.block_tables, ref.context_lens, case.max_context, case.scale,
                             partition_size=partition, out_dtype=out_dtype)
    dc = DevCase(case)
    out = torch.full_like(ro, float("nan"))
    got = pkv.pa_decode_write_noalloc(dc.k_new, dc.v_new, dc.slot_mapping, dc.q, dc.k_cache, dc.v_cache,
                                      dc.block_tables, dc.context_lens, case.max_context, case.scale, out,
                                      partition_size=partition)
    torch.cuda.synchronize()
    return ref, ro, dc, got


def _same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("partition", [BAL, 512])
def test_noalloc_matches_decode_write_two_calls(gpu_lib, partition):
    pkv = gpu_lib
    big = small_bf16_case(301, num_seqs=64, lo=128, hi=4096, poison=True)
    small = small_bf16_case(302, num_seqs=5, lo=1, hi=300, poison=True)
    for case, od in ((big, torch.float32), (small, None)):
        announce("noalloc", case.name, "P", partition, "out", od)
        ref, ro, dc, got = _pair(pkv, case, partition, od)
        assert _same_bits(dc.k_cache, ref.k_cache) and _same_bits(dc.v_cache, ref.v_cache)
        assert not torch.isnan(got).any()
        assert _same_bits(got, ro)
        kc, vc = oracle_after_write(case)
        check_decode(out_to_f64(got), oracle_decode_all(case, kc, vc), bf16_out=od is None)


def test_noalloc_vector_kernel_partitions(gpu_lib):
    """fp32 pools: the vector-ALU kernel's 1024-token partitions under the
    balanced mode, then a smaller batch."""
    pkv = gpu_lib
    cases = [W.make_case("noalloc_f32_long", seed=311, dtype=W.F32, context_lens=[1, 1500, 3000, 17, 1025],
                         num_q_heads=8, num_kv_heads=4, head_dim=64, block_size=16, poison=True),
             W.c1_tiny_f32(seed=312)]
    for case in cases:
        announce("noalloc", case.name)
        ref, ro, dc, got = _pair(pkv, case, BAL, None)
        assert _same_bits(dc.k_cache, ref.k_cache) and _same_bits(dc.v_cache, ref.v_cache)
        assert _same_bits(got, ro)
        kc, vc = oracle_after_write(case)
        check_decode(out_to_f64(got), oracle_decode_all(case, kc, vc), bf16_out=False)


def test_noalloc_refuses_more_than_its_scratch(gpu_lib):
    """A batch whose partitioned scratch exceeds the static array is refused
    before anything is enqueued: pools and out untouched."""
    pkv = gpu_lib
    case = small_bf16_case(321, num_seqs=4, lo=100, hi=200)
    dc = DevCase(case)
    k0, v0 = dc.k_cache.clone(), dc.v_cache.clone()
    out = torch.full((case.num_seqs, case.num_q_heads, case.head_dim), 7.0, dtype=torch.float32, device="cuda")
    huge = 1 << 24  # 16 tokens per partition over a 16M-token bound: far more scratch than 64 MiB
    need = pkv.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                         huge, 16)
    assert need > pkv.PA_NOALLOC_SCRATCH_BYTES
    announce("noalloc refuses", need, "bytes")
    with pytest.raises(pkv.PagedKVError, match="scratch"):
        pkv.pa_decode_write_noalloc(dc.k_new, dc.v_new, dc.slot_mapping, dc.q, dc.k_cache, dc.v_cache,
                                    dc.block_tables, dc.context_lens, huge, case.scale, out, partition_size=16)
    torch.cuda.synchronize()
    assert torch.equal(dc.k_cache.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(dc.v_cache.view(torch.int16), v0.view(torch.int16))
    assert bool((out == 7.0).all())
