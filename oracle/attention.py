"""Paged single-query decode attention, plain definition in fp64.

Test infrastructure only (see the package docstring).

Source of the definition:

* foundry "PagedAttention" ops page, *Concept*: each sequence's KV cache is cut
  into fixed-size blocks that may sit anywhere in GPU memory; a per-sequence
  block table maps logical token positions to physical blocks.
* same page, *How it works*: the attention kernel reads KV through the block
  table, gathering the scattered blocks, which keeps non-contiguous storage
  transparent to the math.  *Cost & effort*: no change to output quality.
* the attention itself is the textbook single-query softmax(q K^T * scale) V.

So the oracle first gathers a sequence's blocks into one contiguous run of
``ctx`` token rows (dropping the unused tail slots of the last block), and then
evaluates the softmax directly, in fp64, one query head at a time.

Readings where the pages are silent (each is listed in the design notes):

* pool layout ``[num_blocks][num_kv_heads][block_size][head_dim]``, separate
  key and value pools of identical shape;
* grouped query heads: query head ``h`` uses KV head ``h // (Hq // Hkv)``;
* ``context_lens`` counts every token the query attends to, including the token
  written in the same step;
* a sequence with ``ctx == 0`` yields an all-zero output row;
* table entries at index >= ceil(ctx / block_size) are never read.
"""

import numpy as np

from .numerics import scale_f64, to_f64


def blocks_for(ctx, block_size):
    """Number of blocks that hold ``ctx`` tokens: ceil(ctx / block_size)."""
    return -(-int(ctx) // int(block_size))


def gather_sequence(cache, table_row, ctx, block_size):
    """One sequence's keys (or values) as a contiguous ``[Hkv][ctx][d]`` array.

    Looks up the physical block of every logical block ``0 .. ceil(ctx/bs)-1``
    in ``table_row``, stacks those blocks in logical order and keeps the first
    ``ctx`` token rows, so slots past the sequence's length in its last block
    never enter the result.
    """
    ctx = int(ctx)
    nb = blocks_for(ctx, block_size)
    num_blocks, hkv, bs, d = cache.shape
    if bs != block_size:
        raise ValueError("cache block dimension does not match block_size")
    if ctx == 0:
        return cache[:0].reshape(hkv, 0, d)
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    if phys.min() < 0 or phys.max() >= num_blocks:
        raise IndexError("block table names a block outside the pool")
    blocks = cache[phys]  # [nb][Hkv][bs][d], logical order
    run = blocks.transpose(1, 0, 2, 3).reshape(hkv, nb * bs, d)
    return run[:, :ctx]


def _softmax_weights(z):
    """Textbook softmax of a 1-D fp64 vector (max subtracted for range only)."""
    z = z - z.max()
    p = np.exp(z)
    return p / p.sum()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    """Paged decode attention for a batch; returns fp64 ``[B][Hq][d]``.

    q            ``[B][Hq][d]`` of ``dtype`` ('f32' float32, 'bf16' uint16 bits)
    k_cache      ``[NB][Hkv][bs][d]`` of ``dtype``
    v_cache      same shape as ``k_cache``
    block_tables ``int32 [B][MB]``, physical block of each logical block
    context_lens ``int32 [B]``, tokens attended per sequence
    scale        the fp32 softmax scale
    """
    q = np.asarray(q)
    b, hq, d = q.shape
    _, hkv, bs, dk = k_cache.shape
    if dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("q / cache shape mismatch")
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    s64 = scale_f64(scale)
    out = np.zeros((b, hq, d), dtype=np.float64)
    for s in range(b):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        ks = to_f64(gather_sequence(k_cache, block_tables[s], ctx, bs), dtype)
        vs = to_f64(gather_sequence(v_cache, block_tables[s], ctx, bs), dtype)
        qs = to_f64(q[s], dtype)
        for h in range(hq):
            g = h // group
            z = s64 * (ks[g] @ qs[h])
            p = _softmax_weights(z)
            out[s, h] = p @ vs[g]
    return out


def decode_one(q_row, k_cache, v_cache, table_row, ctx, scale, dtype, kv_head):
    """Decode output of one (sequence, query head), fp64 ``[d]``.

    Same definition as :func:`decode`, restricted to one row so that large
    batches can be checked on a sample of rows.
    """
    bs = k_cache.shape[2]
    ctx = int(ctx)
    if ctx == 0:
        return np.zeros(k_cache.shape[3], dtype=np.float64)
    ks = to_f64(gather_sequence(k_cache[:, kv_head:kv_head + 1], table_row, ctx, bs), dtype)[0]
    vs = to_f64(gather_sequence(v_cache[:, kv_head:kv_head + 1], table_row, ctx, bs), dtype)[0]
    z = scale_f64(scale) * (ks @ to_f64(q_row, dtype))
    return _softmax_weights(z) @ vs


def partials(q, k_cache, v_cache, block_tables, context_lens, scale, dtype, partition_size):
    """Per-partition softmax statistics, fp64.

    The tokens ``[0, ctx)`` of a sequence are cut into consecutive partitions of
    ``partition_size`` tokens (the last one may be shorter).  For partition
    ``p`` and query head ``h`` this returns

        m[s,h,p]   = max_t z_t
        l[s,h,p]   = sum_t exp(z_t - m)
        acc[s,h,p] = sum_t exp(z_t - m) * V_t

    over the partition's tokens, with ``z_t = scale * <q, K_t>``.  Partitions
    that start at or after ``ctx`` are marked with ``valid[s,p] = False``.
    """
    q = np.asarray(q)
    b, hq, d = q.shape
    _, hkv, bs, _ = k_cache.shape
    group = hq // hkv
    max_ctx = int(np.max(context_lens)) if b else 0
    npart = max(1, -(-max_ctx // partition_size))
    m = np.full((b, hq, npart), -np.inf)
    l = np.zeros((b, hq, npart))
    acc = np.zeros((b, hq, npart, d))
    valid = np.zeros((b, npart), dtype=bool)
    s64 = scale_f64(scale)
    for s in range(b):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        ks = to_f64(gather_sequence(k_cache, block_tables[s], ctx, bs), dtype)
        vs = to_f64(gather_sequence(v_cache, block_tables[s], ctx, bs), dtype)
        qs = to_f64(q[s], dtype)
        for p in range(-(-ctx // partition_size)):
            lo, hi = p * partition_size, min(ctx, (p + 1) * partition_size)
            valid[s, p] = True
            for h in range(hq):
                g = h // group
                z = s64 * (ks[g, lo:hi] @ qs[h])
                mp = z.max()
                e = np.exp(z - mp)
                m[s, h, p] = mp
                l[s, h, p] = e.sum()
                acc[s, h, p] = e @ vs[g, lo:hi]
    return m, l, acc, valid


def merge(m, l, acc, valid):
    """Combine partition statistics into the attention output, fp64.

    With M = max_p m_p over valid partitions:
        L   = sum_p l_p * exp(m_p - M)
        out = sum_p exp(m_p - M) * acc_p / L
    which equals the unpartitioned softmax(z) V exactly in real arithmetic.
    Rows with no valid partition (ctx == 0) give zeros.
    """
    b, hq, npart, d = acc.shape
    out = np.zeros((b, hq, d))
    for s in range(b):
        vp = np.flatnonzero(valid[s])
        if vp.size == 0:
            continue
        for h in range(hq):
            ms = m[s, h, vp]
            big = ms.max()
            w = np.exp(ms - big)
            total = (l[s, h, vp] * w).sum()
            out[s, h] = (w[:, None] * acc[s, h, vp]).sum(axis=0) / total
    return out
