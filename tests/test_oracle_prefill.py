"""Pins for the fp64 paged-prefill oracle (CPU only).

Each test ties ``oracle.prefill`` to something other than itself: pure-Python
brute force on tiny inputs written into the pool by the test's own scatter,
PyTorch's scaled-dot-product attention in fp64 with an explicit causal mask
on contiguous data, the separately pinned decode oracle (a query at position
p sees what a decode with p + 1 keys sees), closed forms, and invariants
(storage placement; keys after a query's position never matter).
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import prefill as P
from widen import torch_to_f64 as to_f64


def scatter_prefill(rng, lens, nq, hq, hkv, d, bs, dtype=W.BF16, scale=None):
    """Paged case from logical rows, scattered by this test: sequence s has
    lens[s] keys and nq[s] queries (its last nq[s] positions)."""
    nbs = [W.ceil_div(c, bs) for c in lens]
    nb = sum(nbs) + 3
    perm = rng.permutation(nb)
    tables = np.full((len(lens), max(1, max(nbs))), -1, dtype=np.int32)
    pool_k = W.normal(rng, (nb, hkv, bs, d), dtype)
    pool_v = W.normal(rng, (nb, hkv, bs, d), dtype)
    lk, lv = [], []
    o = 0
    for s, c in enumerate(lens):
        tables[s, :nbs[s]] = perm[o:o + nbs[s]]
        o += nbs[s]
        k = W.normal(rng, (hkv, c, d), dtype)
        v = W.normal(rng, (hkv, c, d), dtype)
        for t in range(c):
            pool_k[tables[s, t // bs], :, t % bs] = k[:, t]
            pool_v[tables[s, t // bs], :, t % bs] = v[:, t]
        lk.append(to_f64(k, dtype))
        lv.append(to_f64(v, dtype))
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = W.normal(rng, (int(cu[-1]), hq, d), dtype)
    if scale is None:
        scale = float(np.float32(1 / math.sqrt(d)))
    return dict(q=q, k=pool_k, v=pool_v, tables=tables, lens=np.array(lens, np.int32), cu=cu,
                scale=scale, dtype=dtype), lk, lv


def run(c):
    return P.prefill(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["cu"], c["scale"], c["dtype"])


def brute_force(c, lk, lv):
    """Loops: query i of sequence s at p = ctx - n + i; weights e^{z_t} for t <= p."""
    q = to_f64(c["q"], c["dtype"])
    t_all, hq, d = q.shape
    s64 = float(np.float32(c["scale"]))
    out = np.zeros((t_all, hq, d))
    for s in range(len(c["lens"])):
        ctx = int(c["lens"][s])
        lo, hi = int(c["cu"][s]), int(c["cu"][s + 1])
        n = hi - lo
        hkv = lk[s].shape[0]
        grp = hq // hkv
        for i in range(n):
            p = ctx - n + i
            for h in range(hq):
                g = h // grp
                keys = range(0, min(p, ctx - 1) + 1) if p >= 0 else range(0)
                if not keys:
                    continue
                z = [s64 * math.fsum(float(q[lo + i, h, j]) * float(lk[s][g, t, j]) for j in range(d))
                     for t in keys]
                w = [math.exp(x) for x in z]
                den = math.fsum(w)
                for j in range(d):
                    out[lo + i, h, j] = math.fsum(w[k] * float(lv[s][g, t, j]) for k, t in enumerate(keys)) / den
    return out


@pytest.mark.parametrize("seed", range(10))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(2000 + seed)
    bs = [1, 2, 4, 8][seed % 4]
    hkv = [1, 2][seed % 2]
    hq = hkv * [1, 2, 4][(seed // 2) % 3]
    d = [2, 3, 8][seed % 3]
    nseq = 1 + seed % 3
    lens = [int(x) for x in rng.integers(1, 30, size=nseq)]
    nq = [int(rng.integers(0, c + 1)) for c in lens]  # chunks: 0 .. whole prompt
    nq[0] = max(nq[0], 1)
    c, lk, lv = scatter_prefill(rng, lens, nq, hq, hkv, d, bs, dtype=[W.F32, W.BF16][seed % 2])
    np.testing.assert_allclose(run(c), brute_force(c, lk, lv), rtol=0, atol=1e-12)


def test_more_queries_than_keys_gives_zero_rows():
    rng = np.random.default_rng(5)
    c, lk, lv = scatter_prefill(rng, [3, 4], [5, 2], 2, 1, 4, 2)
    out = run(c)
    assert np.all(out[:2] == 0.0)  # positions -2, -1
    assert np.all(np.abs(out[2]).sum(axis=-1) > 0)
    np.testing.assert_allclose(out, brute_force(c, lk, lv), rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype,hq,hkv,d,bs", [(W.BF16, 8, 2, 64, 16), (W.F32, 4, 4, 32, 8),
                                               (W.BF16, 4, 1, 128, 32)])
def test_matches_torch_sdpa_fp64_with_causal_mask(dtype, hq, hkv, d, bs):
    """Identity placement; KV heads repeated per group; mask key j <= ctx - n + i."""
    rng = np.random.default_rng(hq * 37 + d)
    lens = [1, bs + 3, 3 * bs, 150]
    nq = [1, bs + 3, bs, 40]  # whole prompts and chunks after a cached context
    case = W.make_case("sdpa_prefill", seed=int(rng.integers(1 << 30)), dtype=dtype, context_lens=lens,
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, placement="identity")
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = W.normal(rng, (int(cu[-1]), hq, d), dtype)
    ours = P.prefill(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, cu, case.scale, dtype)
    grp = hq // hkv
    kf, vf, qf = to_f64(case.k_cache, dtype), to_f64(case.v_cache, dtype), to_f64(q, dtype)
    for s, (ctx, n) in enumerate(zip(lens, nq)):
        nb = W.ceil_div(ctx, bs)
        first = int(case.block_tables[s, 0])
        kk = kf[first:first + nb].transpose(1, 0, 2, 3).reshape(hkv, nb * bs, d)[:, :ctx]
        vv = vf[first:first + nb].transpose(1, 0, 2, 3).reshape(hkv, nb * bs, d)[:, :ctx]
        kt = torch.from_numpy(np.ascontiguousarray(kk)).repeat_interleave(grp, dim=0)[None]
        vt = torch.from_numpy(np.ascontiguousarray(vv)).repeat_interleave(grp, dim=0)[None]
        qt = torch.from_numpy(np.ascontiguousarray(qf[cu[s]:cu[s + 1]].transpose(1, 0, 2)))[None]
        mask = torch.from_numpy(np.arange(ctx)[None, :] <= (ctx - n + np.arange(n))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=float(np.float32(case.scale)))[0].numpy().transpose(1, 0, 2)
        np.testing.assert_allclose(ours[cu[s]:cu[s + 1]], ref, rtol=0, atol=1e-12)


def test_one_query_per_sequence_is_decode():
    """n_s = 1: the query is the newest position, i.e. the decode oracle."""
    case = W.make_case("pre_dec", seed=9, dtype=W.BF16, context_lens=[1, 17, 64, 200, 0], num_q_heads=8,
                       num_kv_heads=2, head_dim=32, block_size=16)
    nq = [1, 1, 1, 1, 0]
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = case.q[:4]
    got = P.prefill(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, cu, case.scale, W.BF16)
    ref = A.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale,
                   W.BF16)[:4]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_every_row_is_a_decode_over_its_prefix():
    """Query at position p equals the decode oracle with context p + 1."""
    case = W.make_case("pre_rows", seed=10, dtype=W.BF16, context_lens=[40, 33], num_q_heads=4,
                       num_kv_heads=2, head_dim=16, block_size=8)
    nq = [12, 33]
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    rng = np.random.default_rng(10)
    q = W.normal(rng, (int(cu[-1]), 4, 16), W.BF16)
    got = P.prefill(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, cu, case.scale, W.BF16)
    for s in range(2):
        ctx, n = int(case.context_lens[s]), nq[s]
        for i in range(n):
            pos = ctx - n + i
            lens = np.array([pos + 1], np.int32)
            ref = A.decode(q[cu[s] + i][None], case.k_cache, case.v_cache, case.block_tables[s:s + 1], lens,
                           case.scale, W.BF16)[0]
            np.testing.assert_allclose(got[cu[s] + i], ref, rtol=0, atol=1e-12)
            for h in range(4):
                row = P.prefill_row(q[cu[s] + i, h], case.k_cache, case.v_cache, case.block_tables[s], ctx, pos,
                                    case.scale, W.BF16, h // 2)
                np.testing.assert_allclose(row, ref[h], rtol=0, atol=1e-12)


def test_keys_after_a_query_never_matter():
    rng = np.random.default_rng(12)
    c, lk, lv = scatter_prefill(rng, [20], [20], 2, 1, 4, 4, dtype=W.F32)
    base = run(c)
    # perturb the logical rows at positions >= 11 through the table
    k2, v2 = c["k"].copy(), c["v"].copy()
    for t in range(11, 20):
        blk = c["tables"][0, t // 4]
        k2[blk, :, t % 4] += 5.0
        v2[blk, :, t % 4] -= 3.0
    c2 = dict(c, k=k2, v=v2)
    out = run(c2)
    assert np.array_equal(out[:11], base[:11])          # positions 0 .. 10 unchanged
    assert np.all(np.abs(out[11:] - base[11:]).max(axis=(1, 2)) > 1e-6)


def test_closed_forms():
    rng = np.random.default_rng(13)
    c, lk, lv = scatter_prefill(rng, [9], [9], 1, 1, 4, 2, dtype=W.F32)
    # equal value rows: every output is that row
    v_const = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0], np.float32), c["v"].shape).copy()
    out = run(dict(c, v=v_const))
    np.testing.assert_allclose(out[:, 0], np.broadcast_to(v_const[0, 0, 0], (9, 4)), rtol=0, atol=1e-12)
    # zero query: the mean of the value rows up to the position
    out = run(dict(c, q=np.zeros_like(c["q"])))
    for i in range(9):
        np.testing.assert_allclose(out[i, 0], lv[0][0, :i + 1].mean(axis=0), rtol=0, atol=1e-12)


def test_placement_permutation_is_exactly_invariant():
    rng = np.random.default_rng(14)
    c, lk, lv = scatter_prefill(rng, [30, 17], [10, 17], 4, 2, 8, 4)
    base = run(c)
    nb = c["k"].shape[0]
    newpos = rng.permutation(nb)
    k2, v2 = np.empty_like(c["k"]), np.empty_like(c["v"])
    k2[newpos], v2[newpos] = c["k"], c["v"]
    t2 = np.where(c["tables"] >= 0, newpos[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    assert np.array_equal(run(dict(c, k=k2, v=v2, tables=t2)), base)


@pytest.mark.parametrize("shift", [-1, 1])
def test_planted_causal_offset_is_caught(monkeypatch, shift):
    rng = np.random.default_rng(15)
    c, lk, lv = scatter_prefill(rng, [13, 9], [6, 9], 2, 1, 4, 2)
    expect = brute_force(c, lk, lv)
    real = P._causal_rows
    monkeypatch.setattr(P, "_causal_rows", lambda z, first: real(z, first + shift))
    assert np.max(np.abs(run(c) - expect)) > 1e-6
