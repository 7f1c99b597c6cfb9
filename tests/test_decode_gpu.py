"""pa_decode on the GPU against the fp64 oracle.

Tolerances (stated by the workload definition): fp32 KV -> max abs 1e-4;
bf16 KV with fp32 accumulation and bf16 output -> |err| <= 2e-2 + 1e-2|ref|.
Stricter diagnostics: every bf16 case also runs with an fp32 output, where
the only error left is fp32 accumulation order and exp2, held to 1e-4 abs;
and a needle test that pins gathering, tails and lengths exactly.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A

from gpu_cases import (DevCase, announce, check_decode, oracle_after_write, out_to_f64,
                       small_bf16_case, to_dev)

pytestmark = pytest.mark.gpu

BAL = -1  # PA_PARTITION_BALANCED: equal shares of all work per workgroup slot


def run_and_check(pkv, case, partitions, f32_out_too=True):
    dc = DevCase(case)
    dc.write(pkv)
    kc, vc = oracle_after_write(case)
    ref = A.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
    errs = {}
    for p in partitions:
        outs = [None] if case.dtype == W.F32 else ([None, torch.float32] if f32_out_too else [None])
        for od in outs:
            announce(case.name, "P", p, "out", od)
            got = out_to_f64(dc.decode(pkv, partition_size=p, out_dtype=od))
            bf16_out = case.dtype == W.BF16 and od is None
            errs[(p, od)] = check_decode(got, ref, bf16_out)
    return errs


@pytest.mark.parametrize("seed", [1, 101, 102, 103])
def test_tiny_f32(gpu_lib, seed):
    case = W.c1_tiny_f32(seed=seed)
    run_and_check(gpu_lib, case, [0, 16, 32, 48, 112, BAL])


@pytest.mark.parametrize("seed", [2, 101, 102])
def test_small_bf16_gqa4(gpu_lib, seed):
    case = small_bf16_case(seed)
    run_and_check(gpu_lib, case, [0, 16, 64, 512, BAL])


@pytest.mark.parametrize("dtype,hq,hkv,d,bs", [
    (W.BF16, 8, 8, 128, 8), (W.BF16, 8, 4, 128, 32), (W.BF16, 16, 2, 128, 16),
    (W.BF16, 4, 4, 64, 16), (W.BF16, 8, 2, 256, 16), (W.BF16, 4, 4, 128, 1),
    (W.BF16, 8, 4, 128, 2), (W.BF16, 4, 1, 64, 4), (W.F32, 8, 2, 64, 8), (W.F32, 4, 4, 128, 16),
    (W.F32, 2, 1, 256, 32), (W.BF16, 8, 1, 128, 64), (W.BF16, 2, 2, 128, 256),
    # grouped-query matrix-core kernel: G 4 / 8, d 64 / 128 / 256, blocks under 16 tokens
    (W.BF16, 16, 4, 128, 8), (W.BF16, 16, 2, 64, 16), (W.BF16, 8, 1, 256, 32), (W.BF16, 8, 1, 128, 2),
    (W.BF16, 8, 2, 64, 1), (W.BF16, 32, 8, 128, 16)])
def test_shape_grid(gpu_lib, dtype, hq, hkv, d, bs):
    rng = np.random.default_rng(hq * 7 + d + bs)
    lens = [1, bs, bs + 1, 2 * bs - 1] + list(rng.integers(1, 400, size=4))
    case = W.make_case(f"grid_{dtype}_{hq}_{hkv}_{d}_{bs}", seed=int(rng.integers(1 << 30)), dtype=dtype,
                       context_lens=lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs)
    parts = [0, bs * max(1, 64 // bs), 256 if bs <= 256 else bs]
    run_and_check(gpu_lib, case, sorted(set(parts)) + [BAL])


@pytest.mark.parametrize("dtype,hq,hkv,d,bs", [(W.F32, 4, 4, 64, 16), (W.BF16, 8, 8, 128, 16),
                                               (W.BF16, 8, 8, 128, 8), (W.BF16, 8, 4, 128, 32),
                                               (W.F32, 4, 2, 128, 8)])
def test_balanced_vector_kernel_partitions_long_contexts(gpu_lib, dtype, hq, hkv, d, bs):
    """Under the balanced mode the vector-ALU kernel (fp32 pools, 1 or 2 query
    heads per KV head) cuts contexts longer than 1024 tokens into 1024-token
    partitions and merges them; lengths on both sides of the cut and at its
    multiples, poisoned tails, against the fp64 oracle, through a workspace
    filled with random bytes first."""
    lens = [1, 1023, 1024, 1025, 2048, 2049, 3000, 17]
    case = W.make_case(f"valu_bal_{dtype}_{hq}_{hkv}_{d}_{bs}", seed=hq * 31 + d + bs, dtype=dtype,
                       context_lens=lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                       poison=True)
    dc = DevCase(case)
    dc.write(gpu_lib)
    kc, vc = oracle_after_write(case)
    ref = A.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
    need = gpu_lib.pa_decode_workspace_bytes(case.num_seqs, hq, hkv, d, case.max_context, BAL)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    for od in ([None] if dtype == W.F32 else [None, torch.float32]):
        announce(case.name, "BAL", "out", od)
        got = gpu_lib.pa_decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.max_context,
                                case.scale, partition_size=BAL, workspace=ws, out_dtype=od)
        check_decode(out_to_f64(got), ref, dtype == W.BF16 and od is None)


@pytest.mark.parametrize("hq,hkv,parts", [(8, 2, [0, 4096, BAL]), (4, 4, [2048, BAL])])
def test_tables_past_4096_blocks(gpu_lib, hq, hkv, parts):
    # 1-token blocks: a sequence of more than 4096 blocks outgrows the block
    # ids one workgroup stages in LDS; the matrix-core kernel stages them in
    # sub-ranges one after another, the vector kernel runs partitioned
    case = W.make_case(f"bs1_long_{hq}_{hkv}", seed=59, dtype=W.BF16, context_lens=[9000, 4097, 1, 300],
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=1)
    run_and_check(gpu_lib, case, parts)


def test_poisoned_tails_unused_blocks_and_write_slot(gpu_lib):
    case = small_bf16_case(7, poison=True)
    run_and_check(gpu_lib, case, [0, 16, 128, BAL])
    f32case = W.c1_tiny_f32(seed=9, poison=True)
    run_and_check(gpu_lib, f32case, [0, 16, BAL])


def test_table_padding_is_never_read(gpu_lib):
    # -1 padding plus extra columns beyond every sequence's blocks
    case = small_bf16_case(8, max_blocks=80)
    assert (case.block_tables[:, -1] == -1).all()
    run_and_check(gpu_lib, case, [0, 32, BAL])


def test_zero_and_one_token_sequences(gpu_lib):
    announce("ctx 0/1")
    case = W.make_case("ctx01", seed=3, dtype=W.BF16, context_lens=[0, 1, 5, 0, 1],
                       num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16)
    dc = DevCase(case)
    for p in (0, 16, BAL):
        out = dc.decode(gpu_lib, partition_size=p, out_dtype=torch.float32).cpu().numpy()
        assert not out[0].any() and not out[3].any()
        from oracle.numerics import to_f64
        v = to_f64(case.v_cache, W.BF16)  # a 1-token softmax returns that token's V row exactly
        for s in (1, 4):
            blk = case.block_tables[s, 0]
            for h in range(8):
                assert np.array_equal(out[s, h].astype(np.float64), v[blk, h // 4, 0])


@pytest.mark.parametrize("dtype,hq,bs", [(W.F32, 4, 16), (W.BF16, 4, 16), (W.BF16, 8, 16),
                                         (W.BF16, 16, 16), (W.BF16, 8, 8)])
def test_needle_coverage(gpu_lib, dtype, hq, bs):
    """q = 0 gives p = 1/ctx exactly; one-hot V probes every block, the first and
    last token and the tail, so a missed / duplicated / foreign token shows up
    as an error >= 1/ctx.  Query heads per KV head 2, 4 and 8 cover both
    decode kernels."""
    announce("needle", dtype, hq, bs)
    d, hkv = 128 if dtype == W.BF16 else 64, 2
    grp = hq // hkv
    lens = [1, 17, 100, 257, 1000, 2049]
    case = W.make_case("needle", seed=5, dtype=dtype, context_lens=lens, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, poison=True)
    one = np.uint16(0x3F80) if dtype == W.BF16 else np.float32(1)
    zero = np.uint16(0) if dtype == W.BF16 else np.float32(0)
    case.q[...] = zero
    expect = np.zeros((len(lens), hq, d))
    vc = case.v_cache
    for s, n in enumerate(lens):
        nb = W.ceil_div(n, bs)
        for t in range(n):  # zero all valid rows (poison stays past the ends)
            vc[case.block_tables[s, t // bs], :, t % bs, :] = zero
        probes = sorted(set([0, n - 1] + [b * bs + (b * 5) % bs for b in range(nb)]))
        probes = [t for t in probes if t < n][:d]
        for j, t in enumerate(probes):
            for g in range(hkv):
                vc[case.block_tables[s, t // bs], g, t % bs, (j + g) % d] = one
                expect[s, grp * g:grp * g + grp, (j + g) % d] = 1.0 / n
    # the write puts the new token (position n - 1) back: make it zero except its probe
    case.k_new[...] = zero
    case.v_new[...] = zero
    for s, n in enumerate(lens):
        blk, off = divmod(int(case.slot_mapping[s]), bs)
        case.v_new[s] = vc[blk, :, off, :]
    dc = DevCase(case)
    dc.write(gpu_lib)
    for p in (0, 16, 512, BAL):
        got = dc.decode(gpu_lib, partition_size=p, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(got, expect, rtol=1e-5, atol=1e-7)


def test_placement_permutation_is_bitwise_invariant(gpu_lib):
    announce("placement invariance")
    a = small_bf16_case(31)
    b = small_bf16_case(31)
    rng = np.random.default_rng(3)
    newpos = rng.permutation(a.num_blocks)
    b.k_cache = np.empty_like(a.k_cache)
    b.v_cache = np.empty_like(a.v_cache)
    b.k_cache[newpos] = a.k_cache
    b.v_cache[newpos] = a.v_cache
    b.block_tables = np.where(a.block_tables >= 0, newpos[np.maximum(a.block_tables, 0)], -1).astype(np.int32)
    b.slot_mapping = np.array([newpos[s // a.block_size] * a.block_size + s % a.block_size
                               for s in a.slot_mapping], np.int64)
    da, db = DevCase(a), DevCase(b)
    da.write(gpu_lib)
    db.write(gpu_lib)
    for p in (0, 64, BAL):
        oa = da.decode(gpu_lib, partition_size=p, out_dtype=torch.float32)
        ob = db.decode(gpu_lib, partition_size=p, out_dtype=torch.float32)
        assert torch.equal(oa, ob)


def test_partition_sizes_agree(gpu_lib):
    announce("partition agreement")
    case = small_bf16_case(41, hi=3000)
    dc = DevCase(case)
    outs = [dc.decode(gpu_lib, partition_size=p, out_dtype=torch.float32).cpu().numpy()
            for p in (0, 16, 64, 256, 1024, BAL)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 2e-6


def test_balanced_many_sequences_and_empty_ones(gpu_lib):
    """More sequences than one scan pass of the balanced split (256), with
    zero-length ones mixed in, and lengths that make share boundaries cut
    sequences at many places."""
    rng = np.random.default_rng(61)
    lens = rng.integers(0, 90, size=600)
    lens[::37] = 0
    lens[5] = 1500
    case = W.make_case("many_seqs", seed=62, dtype=W.BF16, context_lens=lens, num_q_heads=16,
                       num_kv_heads=4, head_dim=128, block_size=16, poison=True)
    run_and_check(gpu_lib, case, [0, BAL])


@pytest.mark.parametrize("lens", [
    [1000] + [0] * 62 + [1000],        # a share runs past 62 empty sequences: the one-at-a-time walk
    [0, 0, 5, 0, 700, 0, 0, 3, 0, 0],  # empty sequences at both ends and between
    [4096, 0, 7],                      # shares cross from one KV head to the next
    [1] * 64,                          # 64 one-token sequences
])
def test_balanced_split_of_small_batches(gpu_lib, lens):
    """Up to 64 sequences one wave scans the lengths and finds every segment
    of a share at once (a share spanning more than 64 (KV head, sequence)
    pairs takes them one at a time instead); the split must cover every
    token of every KV head once, whatever empty sequences lie between."""
    case = W.make_case(f"small_batch_{len(lens)}_{sum(lens)}", seed=len(lens) + 3, dtype=W.BF16, context_lens=lens,
                       num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, poison=True)
    run_and_check(gpu_lib, case, [BAL])


@pytest.mark.parametrize("seed", range(200, 212))
def test_balanced_random_shapes(gpu_lib, seed):
    """Seeded random batches for the balanced split: 1 to 300 sequences (both
    sides of the one-wave scan's 64), lengths from 0 to 3,000 with runs of
    empty sequences, 4 or 8 query heads per KV head (1 or 2: the vector-ALU
    kernel's 1024-token partitions under the same mode), head_dim 64 or
    128, blocks of 8, 16 or 32 tokens."""
    rng = np.random.default_rng(seed)
    b = int(rng.choice([1, 2, 3, 7, 33, 63, 64, 65, 130, 300]))
    lens = rng.integers(0, 3001, size=b) if b <= 64 else rng.integers(0, 400, size=b)
    lens[rng.random(b) < 0.3] = 0
    if b > 4:
        start = int(rng.integers(0, b - 3))
        lens[start:start + int(rng.integers(2, min(b - start, 40) + 1))] = 0
    hkv = int(rng.choice([2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    case = W.make_case(f"balanced_random_{seed}", seed=seed, dtype=W.BF16, context_lens=lens, num_q_heads=g * hkv,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, poison=True)
    run_and_check(gpu_lib, case, [BAL])


def test_balanced_workspace_reuse_garbage_and_repeats(gpu_lib):
    """One balanced-split workspace, filled with random bytes first, serves
    cases of different shapes in turn (one of them a single long sequence cut
    into ~100 pieces per KV head), each with two query sets alternating, so
    that a partial or split left by the previous call would show; every call
    matches the unpartitioned kernel and repeats are bitwise equal."""
    cases = [small_bf16_case(71), small_bf16_case(72, num_seqs=40, hi=300),
             W.make_case("one_long", seed=73, dtype=W.BF16, context_lens=[30001], num_q_heads=32,
                         num_kv_heads=8, head_dim=128, block_size=16)]
    dcs = [DevCase(c) for c in cases]
    qsets = [(dc.q, torch.flip(dc.q, dims=[2]).contiguous()) for dc in dcs]
    need = max(gpu_lib.pa_decode_workspace_bytes(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                                 c.max_context, BAL) for c in cases)
    for fill in ("random", "zeros"):
        if fill == "random":
            ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
        else:
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        first = {}
        for rep in range(4):
            for i, (c, dc) in enumerate(zip(cases, dcs)):
                announce("workspace reuse", fill, rep, c.name)
                q = qsets[i][rep % 2]
                run = lambda p, ws_: gpu_lib.pa_decode(q, dc.k_cache, dc.v_cache, dc.block_tables,
                                                       dc.context_lens, c.max_context, c.scale,
                                                       partition_size=p, workspace=ws_,
                                                       out_dtype=torch.float32)
                got = run(BAL, ws)
                key = (i, rep % 2)
                if key not in first:
                    ref = run(0, None)
                    assert torch.max(torch.abs(got - ref)).item() < 2e-6, (c.name, rep)
                    first[key] = got
                else:
                    assert torch.equal(got, first[key]), (c.name, rep)


def test_balanced_under_graph_replay(gpu_lib):
    """The balanced split (decode kernel + merge kernel) captured in a HIP
    graph and replayed, on a batch whose shares cut most sequences (16
    sequences of U{1500..2500} tokens, 32/8 heads), with a workspace filled
    with random bytes first.  Eager calls on the same workspace run between
    replays.  Every replay and every eager call is bitwise equal to the first
    eager result, which matches the fp64 oracle."""
    rng = np.random.default_rng(81)
    lens = rng.integers(1500, 2500, size=16, endpoint=True)
    case = W.make_case("graph_replay", seed=82, dtype=W.BF16, context_lens=lens, num_q_heads=32,
                       num_kv_heads=8, head_dim=128, block_size=16, poison=True)
    dc = DevCase(case)
    dc.write(gpu_lib)
    kc, vc = oracle_after_write(case)
    ref = A.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
    need = gpu_lib.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                             case.head_dim, case.max_context, BAL)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.num_seqs, case.num_q_heads, case.head_dim), dtype=torch.float32, device="cuda")

    def call():
        gpu_lib.pa_decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.max_context,
                          case.scale, partition_size=BAL, workspace=ws, out=out, out_dtype=torch.float32)

    announce(case.name, "eager")
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    check_decode(out_to_f64(eager), ref, False)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        announce(case.name, "replay", rep)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), ("replay", rep)
        if rep % 2:
            out.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), ("eager between replays", rep)


def test_balanced_concurrent_callers(gpu_lib):
    """Two host threads call the balanced decode at once, each on its own
    stream, with batches of different sizes (different dynamic LDS, so the
    library's per-device launch-limit entry alternates between them); every
    call's output is bitwise the single-threaded one."""
    import threading

    cases = [small_bf16_case(91, num_seqs=12), small_bf16_case(92, num_seqs=300, hi=200)]
    dcs = [DevCase(c) for c in cases]
    refs = [dc.decode(gpu_lib, partition_size=BAL, out_dtype=torch.float32) for dc in dcs]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            c, dc = cases[i], dcs[i]
            stream = torch.cuda.Stream()
            ws = torch.empty(gpu_lib.pa_decode_workspace_bytes(c.num_seqs, c.num_q_heads, c.num_kv_heads,
                                                               c.head_dim, c.max_context, BAL),
                             dtype=torch.uint8, device="cuda")
            outs = []
            with torch.cuda.stream(stream):
                for _ in range(40):
                    outs.append(gpu_lib.pa_decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                                  dc.context_lens, c.max_context, c.scale, partition_size=BAL,
                                                  workspace=ws, out_dtype=torch.float32, stream=stream))
            stream.synchronize()
            for o in outs:
                if not torch.equal(o, refs[i]):
                    errors.append(f"case {i}: output differs")
                    break
        except Exception as e:  # reported below
            errors.append(f"case {i}: {e!r}")

    announce("concurrent balanced callers")
    threads = [threading.Thread(target=worker, args=(i,)) for i in (0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a caller did not finish"
    assert not errors, errors


def test_argument_errors(gpu_lib):
    announce("argument errors")
    case = small_bf16_case(51, num_seqs=2)
    dc = DevCase(case)
    with pytest.raises(gpu_lib.PagedKVError):
        dc.decode(gpu_lib, partition_size=24)  # not a multiple of the block size
    with pytest.raises(gpu_lib.PagedKVError):
        gpu_lib.pa_decode(dc.q[:, :12].contiguous(), dc.k_cache, dc.v_cache, dc.block_tables,
                          dc.context_lens, case.max_context, case.scale)  # 12 / 8 heads
    with pytest.raises(ValueError):
        gpu_lib.pa_decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables[:1], dc.context_lens,
                          case.max_context, case.scale)
