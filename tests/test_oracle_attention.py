"""Pins for the fp64 decode-attention oracle (CPU only).

Each test ties ``oracle.attention`` to something other than itself:
pure-Python brute force on tiny inputs written into the pool by the test's own
scatter, PyTorch's scaled-dot-product attention in fp64 on contiguous data,
closed forms, and the invariants the PagedAttention pages state (storage
placement is transparent to the math; shared blocks read like private ones;
the unused tail of the last block never matters).
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from widen import torch_to_f64 as to_f64


def scatter_case(rng, lens, hq, hkv, d, bs, dtype=W.F32, num_blocks=None, scale=None):
    """Build a paged case from logical rows with the test's own scatter.

    Returns the case plus the logical K/V rows (fp64) per sequence, so a
    reference can be computed without any block-table reading.
    """
    nbs = [W.ceil_div(c, bs) for c in lens]
    used = sum(nbs)
    nb = num_blocks or used + 3
    perm = rng.permutation(nb)
    mb = max(1, max(nbs) if nbs else 1)
    tables = np.full((len(lens), mb), -1, dtype=np.int32)
    pool_k = W.normal(rng, (nb, hkv, bs, d), dtype)
    pool_v = W.normal(rng, (nb, hkv, bs, d), dtype)
    logical_k, logical_v = [], []
    o = 0
    for s, c in enumerate(lens):
        tables[s, :nbs[s]] = perm[o:o + nbs[s]]
        o += nbs[s]
        lk = W.normal(rng, (hkv, c, d), dtype)
        lv = W.normal(rng, (hkv, c, d), dtype)
        for t in range(c):
            blk = tables[s, t // bs]
            pool_k[blk, :, t % bs, :] = lk[:, t, :]
            pool_v[blk, :, t % bs, :] = lv[:, t, :]
        logical_k.append(to_f64(lk, dtype))
        logical_v.append(to_f64(lv, dtype))
    q = W.normal(rng, (len(lens), hq, d), dtype)
    if scale is None:
        scale = float(np.float32(1 / math.sqrt(d)))
    return dict(q=q, k=pool_k, v=pool_v, tables=tables, lens=np.array(lens, np.int32),
                scale=scale, dtype=dtype), logical_k, logical_v


def run_oracle(c):
    return A.decode(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["scale"], c["dtype"])


def brute_force(c, logical_k, logical_v):
    """Pure-Python loops: z_t = s * sum_c q_c K_tc; out_c = sum_t e^z_t V_tc / sum_t e^z_t."""
    q = to_f64(c["q"], c["dtype"])
    b, hq, d = q.shape
    hkv = logical_k[0].shape[0] if logical_k else 1
    grp = hq // hkv
    s64 = float(np.float32(c["scale"]))
    out = np.zeros((b, hq, d))
    for s in range(b):
        n = int(c["lens"][s])
        for h in range(hq):
            g = h // grp
            if n == 0:
                continue
            z = [s64 * math.fsum(float(q[s, h, j]) * float(logical_k[s][g, t, j]) for j in range(d))
                 for t in range(n)]
            w = [math.exp(x) for x in z]  # tiny shapes: no overflow, no max shift needed
            den = math.fsum(w)
            for j in range(d):
                out[s, h, j] = math.fsum(w[t] * float(logical_v[s][g, t, j]) for t in range(n)) / den
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(1000 + seed)
    bs = [1, 2, 4][seed % 3]
    hkv = [1, 2][seed % 2]
    hq = hkv * [1, 2, 4][(seed // 2) % 3]
    d = [1, 3, 8][seed % 3]
    lens = [int(x) for x in rng.integers(0, 41, size=1 + seed % 3)]
    lens[0] = max(lens[0], 1)
    c, lk, lv = scatter_case(rng, lens, hq, hkv, d, bs, dtype=[W.F32, W.BF16][seed % 2])
    np.testing.assert_allclose(run_oracle(c), brute_force(c, lk, lv), rtol=0, atol=1e-12)


def test_brute_force_ctx_zero_row_is_zero():
    rng = np.random.default_rng(7)
    c, lk, lv = scatter_case(rng, [5, 0, 3], 2, 1, 4, 2)
    out = run_oracle(c)
    assert np.all(out[1] == 0.0)
    np.testing.assert_allclose(out, brute_force(c, lk, lv), rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype,hq,hkv,d,bs", [(W.F32, 4, 4, 64, 16), (W.BF16, 8, 2, 128, 16),
                                               (W.BF16, 6, 3, 32, 8), (W.F32, 4, 1, 16, 32)])
def test_matches_torch_sdpa_fp64(dtype, hq, hkv, d, bs):
    """Identity placement vs torch SDPA on contiguous fp64 K/V (KV heads repeated per group)."""
    rng = np.random.default_rng(hq * 131 + d)
    lens = [1, bs, bs + 1, 3 * bs - 1, 300]
    case = W.make_case("sdpa", seed=int(rng.integers(1 << 30)), dtype=dtype, context_lens=lens,
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                       placement="identity")
    ours = A.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                    case.scale, dtype)
    grp = hq // hkv
    kf = to_f64(case.k_cache, dtype)
    vf = to_f64(case.v_cache, dtype)
    qf = to_f64(case.q, dtype)
    for s, n in enumerate(lens):
        nb = W.ceil_div(n, bs)
        first = int(case.block_tables[s, 0])
        # identity placement: the sequence's blocks are consecutive in the pool
        kk = kf[first:first + nb].transpose(1, 0, 2, 3).reshape(hkv, nb * bs, d)[:, :n]
        vv = vf[first:first + nb].transpose(1, 0, 2, 3).reshape(hkv, nb * bs, d)[:, :n]
        kt = torch.from_numpy(np.ascontiguousarray(kk)).repeat_interleave(grp, dim=0)[None]
        vt = torch.from_numpy(np.ascontiguousarray(vv)).repeat_interleave(grp, dim=0)[None]
        qt = torch.from_numpy(qf[s])[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=float(np.float32(case.scale)))[0, :, 0, :].numpy()
        np.testing.assert_allclose(ours[s], ref, rtol=0, atol=1e-12)


def single_seq(k_rows, v_rows, q_row, bs, scale=1.0):
    """Pack one sequence (fp32 logical rows [n][d]) with a reversed placement."""
    n, d = k_rows.shape
    nb = W.ceil_div(n, bs)
    pool_k = np.full((nb + 2, 1, bs, d), np.nan, np.float32)
    pool_v = np.full((nb + 2, 1, bs, d), np.nan, np.float32)
    table = np.array([[nb + 1 - i for i in range(nb)]], np.int32)
    for t in range(n):
        pool_k[table[0, t // bs], 0, t % bs] = k_rows[t]
        pool_v[table[0, t // bs], 0, t % bs] = v_rows[t]
    return A.decode(q_row[None, None].astype(np.float32), pool_k, pool_v, table,
                    np.array([n], np.int32), scale, W.F32)[0, 0]


def test_closed_form_ctx1_returns_value_row():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 16), dtype=np.float32)
    v = rng.standard_normal((1, 16), dtype=np.float32)
    q = rng.standard_normal(16, dtype=np.float32)
    out = single_seq(k, v, q, bs=4)
    assert np.array_equal(out, v[0].astype(np.float64))


def test_closed_form_zero_query_is_mean():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((37, 8), dtype=np.float32)
    v = rng.standard_normal((37, 8), dtype=np.float32)
    out = single_seq(k, v, np.zeros(8, np.float32), bs=8)
    np.testing.assert_allclose(out, v.astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)


def test_closed_form_three_logits():
    """z = (0, 1, 2): weights (1, e, e^2) / (1 + e + e^2)."""
    k = np.array([[0, 0], [1, 0], [2, 0]], np.float32)
    v = np.array([[1, 0], [0, 1], [0, 0]], np.float32)
    out = single_seq(k, v, np.array([1, 0], np.float32), bs=2)
    den = 1 + math.e + math.e ** 2
    np.testing.assert_allclose(out, [1 / den, math.e / den], rtol=1e-15, atol=0)


def test_closed_form_dominant_logit():
    rng = np.random.default_rng(5)
    n, d = 50, 8
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    k = np.zeros((n, d), np.float32)
    k[17, 0] = 60.0  # z_17 = 60, every other z = 0
    v = rng.standard_normal((n, d), dtype=np.float32)
    out = single_seq(k, v, q, bs=16)
    assert np.max(np.abs(out - v[17])) < n * math.exp(-60) * 10


def test_needle_coverage():
    """q = 0 and one-hot V at probe positions: probed channels read exactly 1/ctx."""
    bs, d, n = 8, 16, 83
    probes = [0, 7, 8, 40, 81, 82]
    v = np.zeros((n, d), np.float32)
    for j, t in enumerate(probes):
        v[t, j] = 1.0
    k = np.random.default_rng(6).standard_normal((n, d), dtype=np.float32)
    out = single_seq(k, v, np.zeros(d, np.float32), bs=bs)
    expect = np.zeros(d)
    expect[:len(probes)] = 1.0 / n
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=0)


def test_placement_permutation_is_exactly_invariant():
    base = W.c2_llama8b_b64(seed=11, num_seqs=5, lo=1, hi=200)
    other = W.c2_llama8b_b64(seed=11, num_seqs=5, lo=1, hi=200)
    # move every block to a new physical home and rewrite the tables to match
    rng = np.random.default_rng(99)
    newpos = rng.permutation(base.num_blocks)
    k2 = np.empty_like(base.k_cache)
    v2 = np.empty_like(base.v_cache)
    k2[newpos] = base.k_cache
    v2[newpos] = base.v_cache
    t2 = np.where(base.block_tables >= 0, newpos[np.maximum(base.block_tables, 0)], -1).astype(np.int32)
    a = A.decode(base.q, base.k_cache, base.v_cache, base.block_tables, base.context_lens, base.scale, W.BF16)
    b = A.decode(other.q, k2, v2, t2, other.context_lens, other.scale, W.BF16)
    assert np.array_equal(a, b)


def test_shared_blocks_read_like_private_copies():
    rng = np.random.default_rng(12)
    bs, hkv, d = 4, 2, 8
    shared = W.normal(rng, (3, hkv, bs, d), W.F32)
    private = W.normal(rng, (4, hkv, bs, d), W.F32)
    # pool layout: [shared 0..2][private 3..6][copies of shared 7..9]
    pool_k = np.concatenate([shared, private, shared])
    pool_v = pool_k[::-1].copy()
    lens = np.array([14, 16], np.int32)
    q = W.normal(rng, (2, 4, d), W.F32)
    t_shared = np.array([[0, 1, 2, 3], [0, 1, 2, 4]], np.int32)
    t_priv = np.array([[0, 1, 2, 3], [7, 8, 9, 4]], np.int32)
    pool_v_priv = pool_v.copy()
    pool_v_priv[7:10] = pool_v[0:3]
    a = A.decode(q, pool_k, pool_v_priv, t_shared, lens, 0.3, W.F32)
    b = A.decode(q, pool_k, pool_v_priv, t_priv, lens, 0.3, W.F32)
    assert np.array_equal(a, b)


def test_poisoned_tails_and_unused_blocks_do_not_leak():
    clean = W.c2_llama8b_b64(seed=21, num_seqs=4, lo=1, hi=90)
    dirty = W.c2_llama8b_b64(seed=21, num_seqs=4, lo=1, hi=90, poison=True)
    # the write slot is poisoned in `dirty`; restore it so both hold the same valid tokens
    for s in range(4):
        blk, o = divmod(int(clean.slot_mapping[s]), clean.block_size)
        dirty.k_cache[blk, :, o] = clean.k_cache[blk, :, o]
        dirty.v_cache[blk, :, o] = clean.v_cache[blk, :, o]
    a = A.decode(clean.q, clean.k_cache, clean.v_cache, clean.block_tables, clean.context_lens, clean.scale, W.BF16)
    b = A.decode(dirty.q, dirty.k_cache, dirty.v_cache, dirty.block_tables, dirty.context_lens, dirty.scale, W.BF16)
    assert np.isfinite(b).all()
    assert np.array_equal(a, b)


def test_gqa_equals_mha_with_repeated_kv_heads():
    case = W.c2_llama8b_b64(seed=31, num_seqs=3, lo=20, hi=70)
    grp = case.num_q_heads // case.num_kv_heads
    a = A.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale, W.BF16)
    k_rep = np.repeat(case.k_cache, grp, axis=1)
    v_rep = np.repeat(case.v_cache, grp, axis=1)
    b = A.decode(case.q, k_rep, v_rep, case.block_tables, case.context_lens, case.scale, W.BF16)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("part", [16, 48, 512, 4096])
def test_partition_merge_identity(part):
    case = W.c2_llama8b_b64(seed=41, num_seqs=4, lo=1, hi=600)
    ref = A.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale, W.BF16)
    m, l, acc, valid = A.partials(case.q, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, case.scale, W.BF16, part)
    np.testing.assert_allclose(A.merge(m, l, acc, valid), ref, rtol=0, atol=1e-13)


def test_decode_one_matches_batch():
    case = W.c5_mha_sweep(seed=51, num_seqs=3, block_size=8)
    full = A.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale, W.BF16)
    for s in range(3):
        for h in (0, 17, 39):
            one = A.decode_one(case.q[s, h], case.k_cache, case.v_cache, case.block_tables[s],
                               case.context_lens[s], case.scale, W.BF16, h)
            assert np.array_equal(one, full[s, h])


# --- planted mistakes: the pins above must catch them --------------------------

def _mutants():
    orig = A.gather_sequence

    def drop_last(cache, row, ctx, bs):
        g = orig(cache, row, ctx, bs)
        return g if ctx <= 1 else np.concatenate([g[:, :-1], g[:, :1]], axis=1)

    def wrong_block(cache, row, ctx, bs):
        # read a block that belongs to no sequence instead of the first one
        # (swapping two of the sequence's own blocks would be harmless: the
        # single-query softmax does not depend on token order)
        r = np.array(row, copy=True)
        nb = W.ceil_div(ctx, bs)
        r[0] = next(b for b in range(cache.shape[0]) if b not in set(r[:nb].tolist()))
        return orig(cache, r, ctx, bs)

    def head_major_misread(cache, row, ctx, bs):
        nb = W.ceil_div(ctx, bs)
        blocks = cache[np.asarray(row[:nb])]
        run = blocks.reshape(nb * cache.shape[1] * bs, cache.shape[3])
        return run.reshape(cache.shape[1], nb * bs, cache.shape[3])[:, :ctx]

    return {"drop_last": drop_last, "wrong_block": wrong_block, "layout": head_major_misread}


@pytest.mark.parametrize("name", ["drop_last", "wrong_block", "layout"])
def test_planted_gather_mistakes_are_caught(monkeypatch, name):
    rng = np.random.default_rng(77)
    c, lk, lv = scatter_case(rng, [9, 13], 4, 2, 4, 4)
    expect = brute_force(c, lk, lv)
    monkeypatch.setattr(A, "gather_sequence", _mutants()[name])
    got = run_oracle(c)
    assert np.max(np.abs(got - expect)) > 1e-6


def test_planted_head_mapping_mistake_is_caught(monkeypatch):
    rng = np.random.default_rng(78)
    c, lk, lv = scatter_case(rng, [11], 4, 2, 4, 4)
    expect = brute_force(c, lk, lv)
    real = A.decode

    def modulo_grouping(q, k, v, t, lens, scale, dtype):
        # query head h wrongly reads KV head h % Hkv
        hq, hkv = q.shape[1], k.shape[1]
        perm = [h % hkv for h in range(hq)]
        order = np.argsort([p * hq + h for h, p in enumerate(perm)], kind="stable")
        out = real(q[:, order], k, v, t, lens, scale, dtype)
        back = np.empty_like(out)
        back[:, order] = out
        return back

    got = modulo_grouping(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["scale"], c["dtype"])
    assert np.max(np.abs(got - expect)) > 1e-6
