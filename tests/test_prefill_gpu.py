"""pa_prefill on the GPU against the fp64 prefill oracle.

Tolerance, derived from the arithmetic (scores, softmax and sums in fp32;
the probabilities enter the product with V rounded to bf16, relative error
at most 2^-9 each, while the normaliser keeps them in fp32): the output is a
weighted mean of value rows with weights off by at most 2^-9 relative, so

    |gpu - ref| <= 2^-9 * max|V| + 1e-4          (fp32 output)
    |gpu - ref| <= 2^-9 * max|V| + 2^-8 |ref| + 1e-4   (bf16 output)

with max|V| over the values the sequence attends to, and 1e-4 for fp32
accumulation order and exp2 (the decode kernels' fp32 bar).

Cases cover whole prompts, chunks after a cached context, one query per
sequence, empty chunks and chunks longer than the context (zero rows),
batches on both sides of the longest-first ordering's size limit, on
pools poisoned with NaN wherever no visible key lives.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import prefill as P

from gpu_cases import DevCase, announce, oracle_after_write, out_to_f64, to_dev

pytestmark = pytest.mark.gpu


def make_prefill(seed, lens, nq, hq, hkv, d, bs, poison=True):
    case = W.make_case(f"prefill_s{seed}", seed=seed, dtype=W.BF16, context_lens=lens, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, poison=poison)
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    rng = np.random.default_rng(seed + 17)
    q = W.normal(rng, (int(cu[-1]), hq, d), W.BF16)
    return case, q, cu


def check_prefill(got, ref, vmax, bf16_out):
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), "non-finite output"
    bound = 2.0 ** -9 * vmax + 1e-4 + (2.0 ** -8 * np.abs(ref) if bf16_out else 0.0)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} elements out of bound (max err {err.max():.3g})"
    return float(err.max())


def run_case(pkv, case, q, cu, max_query=None):
    dc = DevCase(case)
    dc.write(pkv)  # the newest token of each sequence (its slot was poisoned)
    kc, vc = oracle_after_write(case)
    ref = P.prefill(q, kc, vc, case.block_tables, case.context_lens, cu, case.scale, W.BF16)
    vmax = float(np.max(np.abs(out_to_f64_np(vc))))
    mq = int(np.max(np.diff(cu))) if max_query is None else max_query
    dq, dcu = to_dev(q), to_dev(cu)
    for od in (torch.float32, None):
        announce(case.name, "prefill out", od)
        out = pkv.pa_prefill(dq, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, dcu, mq,
                             case.max_context, case.scale, out_dtype=od)
        check_prefill(out_to_f64(out), ref, vmax, bf16_out=od is None)
    return dc


def out_to_f64_np(a):
    from oracle.numerics import bf16_bits_to_f64
    a = np.asarray(a)
    finite = bf16_bits_to_f64(a)
    return np.where(np.isfinite(finite), finite, 0.0)


# head_dim 128 at block sizes 8..256 runs the kernel that loads tiles
# straight into LDS (groups of 4 keys must not straddle a block: 8 is the
# smallest size it takes); head_dim 64, and head_dim 128 below block size
# 8, run the register-staged kernel.
@pytest.mark.parametrize("hq,hkv,d,bs", [(32, 8, 128, 16), (64, 8, 128, 16), (16, 8, 128, 32),
                                         (8, 8, 128, 16), (32, 8, 128, 8), (32, 8, 128, 64), (16, 8, 128, 256),
                                         (32, 8, 128, 4), (32, 8, 128, 1), (16, 4, 64, 8), (32, 8, 64, 1),
                                         (16, 8, 64, 16), (64, 8, 64, 32)])
def test_prompts_and_chunks(gpu_lib, hq, hkv, d, bs):
    rng = np.random.default_rng(hq + d + bs)
    lens = [1, 15, 16, 17, 100, 333, 64, 40]
    nq = [1, 15, 16, 17, 100, 50, 1, 0]  # whole prompts, a chunk after cached keys, decode-like, empty
    case, q, cu = make_prefill(int(rng.integers(1 << 20)), lens, nq, hq, hkv, d, bs)
    run_case(gpu_lib, case, q, cu)


@pytest.mark.parametrize("nseq", [1, 32, 33, 64, 65, 100])
def test_length_ordered_work_with_ties(gpu_lib, nseq):
    # batches of 2..32 sequences are taken longest context first (ties by
    # index), larger ones in index order; repeated lengths make ties.  Up to
    # 64 sequences the grid holds only the query blocks that exist.
    rng = np.random.default_rng(71 + nseq)
    lens = [int(x) for x in rng.choice([16, 48, 48, 130, 1], size=nseq)]
    nq = [int(min(l, x)) for l, x in zip(lens, rng.integers(0, 40, size=nseq))]
    case, q, cu = make_prefill(int(rng.integers(1 << 20)), lens, nq, 32, 8, 128, 16)
    run_case(gpu_lib, case, q, cu)


# In a batch of 2..32 sequences the shortest contexts, up to 8 of them
# holding at most 2 MiB of keys and values per KV head (4,096 tokens at
# head_dim 128, 8,192 at 64), run their query blocks merged by key count.
# Cases: a tail of 8 equal lengths summing to exactly the bound (equal keys,
# ties by index) and one token over it (7 merged), chunks whose blocks end on the same key in different
# sequences, empty chunks and chunks past the context inside the tail,
# 64- and 128-row query blocks (2 and 1 query heads per KV head), head_dim 64.
@pytest.mark.parametrize("lens,nq,hq,hkv,d", [
    ([600] + [512] * 8, [600] + [512] * 8, 32, 8, 128),
    ([600, 513] + [512] * 7, [600, 513] + [512] * 7, 32, 8, 128),
    ([600, 600, 332, 300, 700, 96, 64], [64, 32, 64, 0, 100, 96, 80], 32, 8, 128),
    ([900, 500, 500, 260, 130, 129], [900, 500, 244, 260, 130, 1], 8, 8, 128),
    ([700, 450, 450, 200, 77], [300, 450, 450, 200, 77], 16, 8, 128),
    ([5000, 4100, 4092, 3000, 100], [64, 256, 300, 1000, 100], 32, 8, 64),
])
def test_merged_tail_of_short_sequences(gpu_lib, lens, nq, hq, hkv, d):
    case, q, cu = make_prefill(sum(lens) + hq + d, lens, nq, hq, hkv, d, 16)
    run_case(gpu_lib, case, q, cu)


@pytest.mark.parametrize("seed", range(300, 312))
def test_random_batches(gpu_lib, seed):
    # seeded random batches over the work lookup's branches: 1 to 64
    # sequences (ranked up to 32, compact grid up to 64), whole prompts,
    # chunks after cached keys, empty chunks and chunks past their context;
    # both kernels (head_dim 128 at block size 8+ loads tiles into LDS)
    rng = np.random.default_rng(seed)
    nseq = int(rng.choice([1, 2, 5, 17, 32, 33, 48, 64]))
    hkv = int(rng.choice([2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([1, 8, 16, 32, 256]))
    lens = [int(x) for x in rng.integers(1, 600, size=nseq)]
    nq = []
    for l in lens:
        kind = rng.integers(4)
        nq.append(l if kind == 0 else int(rng.integers(0, min(l, 200) + 1)) if kind < 3 else min(l + 7, 200))
    case, q, cu = make_prefill(seed, lens, nq, hkv * g, hkv, d, bs)
    run_case(gpu_lib, case, q, cu)


def test_chunk_longer_than_context_gives_zero_rows(gpu_lib):
    case, q, cu = make_prefill(31, [5, 40], [9, 40], 32, 8, 128, 16)
    dc = run_case(gpu_lib, case, q, cu)
    out = gpu_lib.pa_prefill(to_dev(q), dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, to_dev(cu), 40,
                             case.max_context, case.scale, out_dtype=torch.float32).cpu().numpy()
    assert np.all(out[:4] == 0.0)  # positions -4 .. -1


def test_long_prompts_many_tiles(gpu_lib):
    case, q, cu = make_prefill(41, [1500, 777, 2049], [1500, 300, 2049], 32, 8, 128, 16)
    run_case(gpu_lib, case, q, cu)


def test_table_read_from_hbm_past_2048_blocks(gpu_lib):
    # 1-token blocks: a workgroup that needs more than 2048 block ids reads
    # them from the table in HBM instead of staging them in LDS
    case, q, cu = make_prefill(47, [2100, 3000, 2049], [33, 64, 1], 32, 8, 128, 1)
    run_case(gpu_lib, case, q, cu)


def test_placement_permutation_is_bitwise_invariant(gpu_lib):
    case, q, cu = make_prefill(51, [300, 129], [300, 65], 32, 8, 128, 16, poison=False)
    perm = np.random.default_rng(5).permutation(case.num_blocks)
    k2, v2 = np.empty_like(case.k_cache), np.empty_like(case.v_cache)
    k2[perm], v2[perm] = case.k_cache, case.v_cache
    t2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    outs = []
    for kc, vc, tb in ((case.k_cache, case.v_cache, case.block_tables), (k2, v2, t2)):
        outs.append(gpu_lib.pa_prefill(to_dev(q), to_dev(kc), to_dev(vc), to_dev(tb), to_dev(case.context_lens),
                                       to_dev(cu), 300, case.max_context, case.scale, out_dtype=torch.float32))
    assert torch.equal(outs[0], outs[1])


def test_argument_errors(gpu_lib):
    case, q, cu = make_prefill(61, [20], [20], 32, 8, 128, 16, poison=False)
    dc = DevCase(case)
    f32 = torch.zeros((4, 4, 2, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.PagedKVError):  # fp32 pools are not built
        gpu_lib.pa_prefill(torch.zeros((20, 32, 128), dtype=torch.float32, device="cuda"), f32, f32,
                           dc.block_tables, dc.context_lens, to_dev(cu), 20, 20, 1.0)
    with pytest.raises(gpu_lib.PagedKVError):  # 12 / 8 query heads
        gpu_lib.pa_prefill(to_dev(q)[:, :12].contiguous(), dc.k_cache, dc.v_cache, dc.block_tables,
                           dc.context_lens, to_dev(cu), 20, 20, 1.0)
    for bad in (0.0, -0.1, float("inf"), float("nan")):  # the softmax scale must be positive and finite
        with pytest.raises(gpu_lib.PagedKVError):
            gpu_lib.pa_prefill(to_dev(q), dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, to_dev(cu), 20,
                               20, bad)


@pytest.mark.parametrize("name", ["prefill_llama3_8b", "prefill_chunked"])
def test_full_size_every_row(gpu_lib, name):
    """The benchmarked prefill step (store the chunk's tokens, then attend) at
    full size: every (query, head) row against the oracle (fp32 output within
    the derived bound; bf16 output bitwise the fp32 output rounded to nearest
    even).  The oracle runs sequence by sequence on threads."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import kvcache as KV

    from gpu_cases import check_bf16_is_rounded_f32

    pc = W.c6_prefill_llama8b() if name == "prefill_llama3_8b" else W.c6_chunked_prefill()
    c = pc.case
    announce("prefill full", name)
    dc = DevCase(c)
    gpu_lib.pa_write_kv(to_dev(pc.k_new), to_dev(pc.v_new), to_dev(pc.slot_mapping), dc.k_cache, dc.v_cache)
    args = (to_dev(pc.q), dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, to_dev(pc.cu_seqlens),
            pc.max_query_len, c.max_context, c.scale)
    o32 = gpu_lib.pa_prefill(*args, out_dtype=torch.float32)
    obf = gpu_lib.pa_prefill(*args)
    torch.cuda.synchronize()
    check_bf16_is_rounded_f32(obf, o32)
    out = o32.cpu().numpy().astype(np.float64)
    del dc, o32, obf
    torch.cuda.empty_cache()
    kc, vc = KV.write_kv(c.k_cache, c.v_cache, pc.k_new, pc.v_new, pc.slot_mapping, c.block_size)
    vmax = float(np.max(np.abs(out_to_f64_np(vc))))
    cu = pc.cu_seqlens
    announce("prefill full", name, "oracle over", int(cu[-1]), "query rows")

    def oracle_seq(s):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        return P.prefill(pc.q[rows], kc, vc, c.block_tables[s:s + 1], c.context_lens[s:s + 1],
                         np.array([0, cu[s + 1] - cu[s]], np.int32), c.scale, W.BF16)

    with ThreadPoolExecutor(16) as ex:
        ref = np.concatenate(list(ex.map(oracle_seq, range(c.num_seqs))), axis=0)
    check_prefill(out, ref, vmax, bf16_out=False)


@pytest.mark.parametrize("d,bs", [(128, 16), (128, 1), (64, 32)])
def test_needles_strict(gpu_lib, d, bs):
    """q = 0 makes every visible weight exactly 1, so with one-hot value rows
    (key t has a 1 in channel t % d) each output is the exact ratio of the
    visible keys in a channel to all visible keys: the causal mask, the gather
    through the table and the tails are checked to fp32 division rounding
    (1e-6 relative), far tighter than the bf16-weight bound.  Poisoned pools:
    NaN in every slot no sequence attends to."""
    rng = np.random.default_rng(d + bs)
    lens = [1, 16, 17, 100, 333, 777, 40]
    nq = [1, 16, 5, 100, 64, 300, 0]
    case = W.make_case(f"needles_{d}_{bs}", seed=int(rng.integers(1 << 20)), dtype=W.BF16, context_lens=lens,
                       num_q_heads=32, num_kv_heads=8, head_dim=d, block_size=bs, poison=True)
    one = W.round_to_bf16(np.ones(1, np.float32))[0]
    for s, ctx in enumerate(lens):
        for t in range(ctx):
            blk, off = int(case.block_tables[s, t // bs]), t % bs
            case.v_cache[blk, :, off, :] = 0
            case.v_cache[blk, :, off, t % d] = one
        blk, off = int(case.block_tables[s, (ctx - 1) // bs]), (ctx - 1) % bs
        case.k_cache[blk, :, off, :] = case.k_new[s]  # the newest key's slot was poisoned
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = np.zeros((int(cu[-1]), 32, d), np.uint16)
    dc = DevCase(case)  # every position already in the pools: no store
    announce("needles", d, bs)
    out = gpu_lib.pa_prefill(to_dev(q), dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, to_dev(cu),
                             int(max(nq)), case.max_context, case.scale, out_dtype=torch.float32)
    got = out.cpu().numpy().astype(np.float64)
    ref = P.prefill(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, cu, case.scale, W.BF16)
    # closed form, independent of the oracle: row i of sequence s sees keys 0 .. ctx - n + i
    for s, (ctx, n) in enumerate(zip(lens, nq)):
        for i in range(n):
            seen = ctx - n + i + 1
            counts = np.bincount(np.arange(seen) % d, minlength=d)
            np.testing.assert_allclose(ref[cu[s] + i], np.broadcast_to(counts / seen, (32, d)), rtol=1e-12, atol=0)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=0)


def _log2_scores(kind, n):
    """Scores, in log2 units, that move the softmax's reference max."""
    t = np.arange(n)
    if kind == "staircase":  # every 32-key tile passes the previous maximum by about 12
        return 12.0 * (t // 32)
    if kind == "crowd":  # one whole tile 6 above the rest: no weight above 2^8, but 8 of them sum past it
        return np.where(t // 32 == 5, 6.0, 0.0)
    if kind == "spike":  # one key 20 above the rest
        return np.where(t == 250, 20.0, 0.0)
    return -0.05 * t  # falling: the first tile's maximum holds throughout


@pytest.mark.parametrize("d,bs", [(128, 16), (64, 16)])
def test_scores_past_the_running_max(gpu_lib, d, bs):
    """The kernels keep a reference maximum per row and move it only when a
    lane's weights against it grow large; scores built to pass it mid-sequence
    (by ~12 every tile, by 6 across a whole tile, by 20 at one key) and to
    fall behind it, through channel 0 (q is one-hot there, the other key
    channels are noise it ignores), must still give the oracle's output."""
    kinds = ["staircase", "crowd", "spike", "falling"]
    lens, nq = [800, 600, 500, 300], [800, 600, 200, 300]
    case = W.make_case(f"running_max_{d}_{bs}", seed=7 + d + bs, dtype=W.BF16, context_lens=lens, num_q_heads=32,
                       num_kv_heads=8, head_dim=d, block_size=bs, poison=True)
    rng = np.random.default_rng(d * bs)
    qscale = float(np.float32(case.scale)) * np.log2(np.e)
    for s, (kind, ctx) in enumerate(zip(kinds, lens)):
        k = W.normal(rng, (ctx, 8, d), W.BF16)
        k[:, :, 0] = W.round_to_bf16((_log2_scores(kind, ctx) / qscale).astype(np.float32))[:, None]
        v = W.normal(rng, (ctx, 8, d), W.BF16)
        for t in range(ctx):  # every position, the newest (poisoned) one included
            blk, off = int(case.block_tables[s, t // bs]), t % bs
            case.k_cache[blk, :, off, :] = k[t]
            case.v_cache[blk, :, off, :] = v[t]
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = np.zeros((int(cu[-1]), 32, d), np.uint16)
    q[:, :, 0] = W.round_to_bf16(np.ones(1, np.float32))[0]
    ref = P.prefill(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, cu, case.scale, W.BF16)
    vmax = float(np.max(np.abs(out_to_f64_np(case.v_cache))))
    dc = DevCase(case)
    for od in (torch.float32, None):
        announce(case.name, "prefill out", od)
        out = gpu_lib.pa_prefill(to_dev(q), dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, to_dev(cu),
                                 int(max(nq)), case.max_context, case.scale, out_dtype=od)
        check_prefill(out_to_f64(out), ref, vmax, bf16_out=od is None)
