"""Paged prefill attention, plain definition in fp64.

Test infrastructure only (see the package docstring).

Source of the definition:

* foundry "PagedAttention" ops page, *How it works*: tokens' keys and values
  are stored block by block into the blocks the sequence's table names, and
  the attention kernel reads KV through the table; *Concept*: the table maps
  logical positions to physical blocks anywhere in the pool.  A prompt (or a
  chunk of one) is many such tokens at once.
* the attention itself is the textbook causal softmax(q K^T * scale) V: a
  query at position ``p`` of its sequence attends to the keys at positions
  ``0 .. p``.

Readings where the pages are silent (each is listed in the design notes):

* queries of all sequences are packed ``[T][Hq][d]`` in sequence order;
  ``cu_seqlens int32 [B + 1]`` gives sequence ``s`` the rows
  ``cu_seqlens[s] .. cu_seqlens[s + 1] - 1`` (``n_s`` of them);
* ``context_lens[s]`` counts every key of sequence ``s`` after its new
  tokens were stored, and the ``n_s`` queries are its last ``n_s`` positions:
  query ``i`` sits at position ``context_lens[s] - n_s + i``;
* a query at a position below 0 (``n_s > context_lens[s]``) attends to
  nothing and yields zeros;
* pool layout and grouped query heads as in ``attention`` (query head ``h``
  uses KV head ``h // (Hq // Hkv)``).
"""

import numpy as np

from .attention import gather_sequence
from .numerics import scale_f64, to_f64


def _causal_rows(z, first_pos):
    """Row-wise softmax of ``z [n][ctx]`` where row ``i`` may only use
    columns ``0 .. first_pos + i``; rows with no usable column give zeros."""
    n, ctx = z.shape
    out = np.zeros_like(z)
    for i in range(n):
        last = first_pos + i  # last key position this query sees
        if last < 0:
            continue
        zi = z[i, :min(last + 1, ctx)]
        w = np.exp(zi - zi.max())
        out[i, :zi.shape[0]] = w / w.sum()
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens, scale, dtype):
    """Causal paged attention for packed queries; returns fp64 ``[T][Hq][d]``.

    q            ``[T][Hq][d]`` of ``dtype`` ('f32' or 'bf16' uint16 bits)
    k_cache      ``[NB][Hkv][bs][d]`` of ``dtype``; v_cache the same shape
    block_tables ``int32 [B][MB]``
    context_lens ``int32 [B]``: keys per sequence, new tokens included
    cu_seqlens   ``int32 [B + 1]``: query row offsets per sequence
    scale        the fp32 softmax scale
    """
    q = np.asarray(q)
    t, hq, d = q.shape
    _, hkv, bs, dk = k_cache.shape
    if dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("q / cache shape mismatch")
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != t or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to the number of query rows")
    group = hq // hkv
    s64 = scale_f64(scale)
    out = np.zeros((t, hq, d), dtype=np.float64)
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        ctx = int(context_lens[s])
        if n == 0 or ctx == 0:
            continue
        ks = to_f64(gather_sequence(k_cache, block_tables[s], ctx, bs), dtype)  # [Hkv][ctx][d]
        vs = to_f64(gather_sequence(v_cache, block_tables[s], ctx, bs), dtype)
        qs = to_f64(q[cu[s]:cu[s + 1]], dtype)  # [n][Hq][d]
        for h in range(hq):
            g = h // group
            z = s64 * (qs[:, h, :] @ ks[g].T)  # [n][ctx]
            out[cu[s]:cu[s + 1], h] = _causal_rows(z, ctx - n) @ vs[g]
    return out


def prefill_row(q_row, k_cache, v_cache, table_row, ctx, pos, scale, dtype, kv_head):
    """One query row at position ``pos`` of a sequence with ``ctx`` keys:
    softmax over the keys ``0 .. min(pos, ctx - 1)``, fp64 ``[d]`` (zeros
    when ``pos < 0``).  For sampled checks of large batches."""
    d = k_cache.shape[3]
    pos = int(pos)
    if pos < 0 or int(ctx) == 0:
        return np.zeros(d, dtype=np.float64)
    bs = k_cache.shape[2]
    ks = to_f64(gather_sequence(k_cache[:, kv_head:kv_head + 1], table_row, ctx, bs), dtype)[0]
    vs = to_f64(gather_sequence(v_cache[:, kv_head:kv_head + 1], table_row, ctx, bs), dtype)[0]
    last = min(pos, int(ctx) - 1)
    z = scale_f64(scale) * (ks[:last + 1] @ to_f64(q_row, dtype))
    w = np.exp(z - z.max())
    return (w / w.sum()) @ vs[:last + 1]
