"""Seeded synthetic inputs for paged decode, shared by tests, smoke and bench.

This module only draws and lays out input data.  It holds none of the
attention arithmetic, and it imports neither the oracle nor the HIP library,
so both sides can consume exactly the same arrays.

Element types: fp32 data is ``float32``; bf16 data is carried as ``uint16``
bit patterns (rounded to nearest-even from fp32 draws).

Layouts (the library's ABI):

* pools ``k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim]``
* ``block_tables : int32 [num_seqs][max_blocks]``, padded with -1
* ``context_lens : int32 [num_seqs]`` -- tokens attended, including the token
  written in the same step (it sits at position ``ctx - 1``)
* ``slot_mapping : int64 [num_tokens]`` -- ``block * block_size + offset``

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream, drawn in this
order): context lengths, block placement permutation, q, K pool, V pool, new
K rows, new V rows.  Values are N(0, 1); arrays above 2**24 elements are
drawn chunk by chunk from PCG64 streams seeded from the main stream (see
``normal``).  The pool holds
ceil(1.25 * blocks in use) blocks unless a size is given; the blocks in use are
the first entries of the permutation, handed to sequences in order.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"

_CHUNK = 1 << 24


def round_to_bf16(x):
    """float32 array -> uint16 bf16 patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def nan_value(dtype):
    return np.uint16(0x7FC0) if dtype == BF16 else np.float32(np.nan)


def storage_dtype(dtype):
    return np.uint16 if dtype == BF16 else np.float32


def _fill_chunk(seed, out, dtype):
    x = np.random.default_rng(seed).standard_normal(out.size, dtype=np.float32)
    out[...] = x if dtype == F32 else round_to_bf16(x)


def normal(rng, shape, dtype):
    """N(0, 1) draws of ``shape`` stored as ``dtype``.

    Small arrays come straight from ``rng``.  Large ones are cut into fixed
    chunks of 2**24 elements; chunk i is drawn from a PCG64 seeded with the
    i-th of a list of 63-bit integers taken from ``rng``, so the values do
    not depend on how many threads fill the chunks.
    """
    out = np.empty(shape, dtype=storage_dtype(dtype))
    flat = out.reshape(-1)
    if flat.size <= _CHUNK:
        x = rng.standard_normal(flat.size, dtype=np.float32)
        flat[:] = x if dtype == F32 else round_to_bf16(x)
        return out
    n = -(-flat.size // _CHUNK)
    seeds = rng.integers(0, 2 ** 63 - 1, size=n)
    workers = max(1, min(16, os.cpu_count() or 1, n))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda i: _fill_chunk(int(seeds[i]), flat[i * _CHUNK:(i + 1) * _CHUNK], dtype),
                    range(n)))
    return out


def ceil_div(a, b):
    return -(-int(a) // int(b))


@dataclass
class DecodeCase:
    """One decode step's inputs in the library's layout (host arrays)."""

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    partition_size: int
    context_lens: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self):
        return int(self.k_cache.shape[0])

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])

    @property
    def max_context(self):
        return int(self.context_lens.max()) if self.num_seqs else 0

    def elt_bytes(self):
        return 2 if self.dtype == BF16 else 4

    def kv_bytes(self):
        """Algorithmic K+V bytes one decode reads: valid tokens, each KV head once."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * 2 * self.head_dim * self.elt_bytes()

    def table_bytes(self):
        """Block-table bytes one decode reads: ceil(ctx / bs) int32 entries per sequence."""
        return 4 * sum(ceil_div(c, self.block_size) for c in self.context_lens)


def make_case(name, *, seed, dtype, context_lens, num_q_heads, num_kv_heads, head_dim,
              block_size, num_blocks=None, pool_factor=1.25, placement="shuffled",
              poison=False, scale=None, partition_size=0, max_blocks=None, rng=None):
    """Draw one decode case.

    ``context_lens`` is an int sequence, or a callable ``rng -> int array``
    drawn first from the stream.  ``placement`` is ``"shuffled"`` (seeded
    permutation of the pool) or ``"identity"`` (each sequence's blocks
    consecutive, in logical order).  With ``poison`` the slots past each
    sequence's length, the slot the new token goes to and every unused block
    hold NaN, so any stray read shows up in the output.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = np.asarray(context_lens(rng) if callable(context_lens) else context_lens, dtype=np.int32)
    bsz = lens.shape[0]
    nbs = np.array([ceil_div(c, block_size) for c in lens], dtype=np.int64)
    used = int(nbs.sum())
    if num_blocks is None:
        num_blocks = max(1, int(np.ceil(pool_factor * used)))
    if used > num_blocks:
        raise ValueError("pool too small for the requested lengths")
    if placement == "shuffled":
        perm = rng.permutation(num_blocks).astype(np.int32)
    elif placement == "identity":
        perm = np.arange(num_blocks, dtype=np.int32)
    else:
        raise ValueError(placement)
    mb = max(1, int(nbs.max()) if bsz else 1) if max_blocks is None else int(max_blocks)
    tables = np.full((bsz, mb), -1, dtype=np.int32)
    off = 0
    for s in range(bsz):
        tables[s, :nbs[s]] = perm[off:off + nbs[s]]
        off += nbs[s]
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    q = normal(rng, (bsz, num_q_heads, head_dim), dtype)
    pool_shape = (num_blocks, num_kv_heads, block_size, head_dim)
    k_cache = normal(rng, pool_shape, dtype)
    v_cache = normal(rng, pool_shape, dtype)
    k_new = normal(rng, (bsz, num_kv_heads, head_dim), dtype)
    v_new = normal(rng, (bsz, num_kv_heads, head_dim), dtype)
    slots = np.full(bsz, -1, dtype=np.int64)
    for s in range(bsz):
        if lens[s] > 0:
            pos = int(lens[s]) - 1
            slots[s] = int(tables[s, pos // block_size]) * block_size + pos % block_size
    if poison:
        bad = nan_value(dtype)
        in_use = np.zeros(num_blocks, dtype=bool)
        in_use[perm[:used]] = True
        k_cache[~in_use] = bad
        v_cache[~in_use] = bad
        for s in range(bsz):
            c = int(lens[s])
            if c == 0:
                continue
            last = int(tables[s, nbs[s] - 1])
            tail = c - (nbs[s] - 1) * block_size
            k_cache[last, :, tail:, :] = bad
            v_cache[last, :, tail:, :] = bad
            blk, o = divmod(int(slots[s]), block_size)
            k_cache[blk, :, o, :] = bad
            v_cache[blk, :, o, :] = bad
    return DecodeCase(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                      head_dim=head_dim, block_size=block_size, scale=scale,
                      partition_size=partition_size, context_lens=lens, block_tables=tables,
                      q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                      slot_mapping=slots, meta={"seed": seed, "placement": placement, "poison": poison})


# --- the five workloads --------------------------------------------------------

def c1_tiny_f32(seed=1, **kw):
    """Tiny fp32 decode: 4 seqs, 4 = 4 heads, d 64, bs 16, ctx {17,33,64,100}, 64-block pool."""
    return make_case("tiny_f32", seed=seed, dtype=F32, context_lens=[17, 33, 64, 100],
                     num_q_heads=4, num_kv_heads=4, head_dim=64, block_size=16, num_blocks=64,
                     scale=0.125, **kw)


def c2_llama8b_b64(seed=2, num_seqs=64, lo=128, hi=4096, **kw):
    """Llama-3-8B-shaped layer, bf16: 64 seqs, 32 q / 8 KV heads, d 128, bs 16, ctx U{128..4096}."""
    return make_case("llama3_8b_b64", seed=seed, dtype=BF16,
                     context_lens=lambda r: r.integers(lo, hi, size=num_seqs, endpoint=True),
                     num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, **kw)


def c3_long_context(seed=3, num_seqs=8, ctx=32768, partition_size=512, **kw):
    """Long-context split decode, bf16: 8 seqs x 32768 tokens, 32 / 8 heads, d 128, bs 16, P 512."""
    return make_case("long_ctx_32k", seed=seed, dtype=BF16, context_lens=[ctx] * num_seqs,
                     num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                     partition_size=partition_size, **kw)


def c5_lengths(rng, num_seqs=256, median=600.0, sigma=1.0, lo=16, hi=8192):
    """Lognormal context lengths: clip(rint(exp(N(ln median, sigma))), lo, hi)."""
    x = rng.lognormal(mean=np.log(median), sigma=sigma, size=num_seqs)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def c5_mha_sweep(seed=5, block_size=16, num_seqs=256, **kw):
    """High-concurrency MHA, bf16: 256 seqs, 40 = 40 heads, d 128, lognormal ctx, bs in {8,16,32}."""
    return make_case(f"mha_b256_bs{block_size}", seed=seed, dtype=BF16,
                     context_lens=lambda r: c5_lengths(r, num_seqs=num_seqs),
                     num_q_heads=40, num_kv_heads=40, head_dim=128, block_size=block_size, **kw)


# --- prompt prefill -------------------------------------------------------------

@dataclass
class PrefillCase:
    """A batch of prompt chunks to prefill through the paged pools.

    ``case`` carries the pools, tables, context lengths and scale (its
    single-token q / new rows are not used).  Sequence s's chunk is its last
    ``n_s`` positions: queries ``q[cu_seqlens[s]:cu_seqlens[s+1]]`` and the
    chunk tokens' keys / values ``k_new, v_new`` (same rows), to be stored at
    ``slot_mapping`` (the table's slots of those positions) before the
    attention.  Drawn after the case, from a second stream seeded
    ``seed + 1``: chunk lengths (when drawn), q, K rows, V rows.
    """

    case: "DecodeCase"
    q: np.ndarray             # [T][Hq][d]
    cu_seqlens: np.ndarray    # int32 [B + 1]
    k_new: np.ndarray         # [T][Hkv][d]
    v_new: np.ndarray
    slot_mapping: np.ndarray  # int64 [T]

    @property
    def num_tokens(self):
        return int(self.cu_seqlens[-1])

    @property
    def max_query_len(self):
        return int(np.max(np.diff(self.cu_seqlens))) if len(self.cu_seqlens) > 1 else 0


def make_prefill(name, *, seed, context_lens, chunk_lens=None, num_q_heads, num_kv_heads, head_dim,
                 block_size, dtype=BF16, **kw):
    """Prefill case: ``chunk_lens`` None means whole prompts (n_s = ctx_s)."""
    case = make_case(name, seed=seed, dtype=dtype, context_lens=context_lens, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size, **kw)
    rng = np.random.default_rng(seed + 1)
    lens = case.context_lens.astype(np.int64)
    if chunk_lens is None:
        nq = lens.copy()
    elif callable(chunk_lens):
        nq = np.minimum(np.asarray(chunk_lens(rng), dtype=np.int64), lens)
    else:
        nq = np.asarray(chunk_lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    t = int(cu[-1])
    q = normal(rng, (t, num_q_heads, head_dim), dtype)
    k_new = normal(rng, (t, num_kv_heads, head_dim), dtype)
    v_new = normal(rng, (t, num_kv_heads, head_dim), dtype)
    slots = np.full(t, -1, dtype=np.int64)
    for s in range(len(lens)):
        for i in range(int(nq[s])):
            pos = int(lens[s] - nq[s] + i)
            if pos >= 0:
                slots[cu[s] + i] = int(case.block_tables[s, pos // block_size]) * block_size + pos % block_size
    return PrefillCase(case=case, q=q, cu_seqlens=cu, k_new=k_new, v_new=v_new, slot_mapping=slots)


def c6_prefill_llama8b(seed=6, num_seqs=8, lo=512, hi=4096):
    """Llama-3-8B-shaped prompt prefill, bf16: 8 whole prompts of U{512..4096} tokens,
    32 q / 8 KV heads, d 128, bs 16."""
    return make_prefill("prefill_llama3_8b", seed=seed,
                        context_lens=lambda r: r.integers(lo, hi, size=num_seqs, endpoint=True),
                        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16)


def c6_chunked_prefill(seed=7, num_seqs=16, lo=1024, hi=8192, chunk=512):
    """Chunked prefill after a cached context, bf16: 16 sequences of U{1024..8192} keys whose last
    512 positions are the new chunk, 32 q / 8 KV heads, d 128, bs 16."""
    return make_prefill("prefill_chunked", seed=seed,
                        context_lens=lambda r: r.integers(lo, hi, size=num_seqs, endpoint=True),
                        chunk_lens=lambda r: np.full(num_seqs, chunk),
                        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16)


# --- shared-prefix copy-on-write workload -------------------------------------

@dataclass
class SharedPrefixPlan:
    """Inputs of the shared-prefix copy-on-write workload.

    256 sequences share the KV of one 2048-token prefix (128 blocks of 16) and
    each owns a private suffix of U{0..512} tokens.  Every step copies-on-write
    1% of the shared (sequence, prefix block) references, then writes one token
    per sequence and decodes.
    """

    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    prefix_len: int
    steps: int
    cow_per_step: int
    num_blocks: int
    scale: float
    free_order: np.ndarray
    prefix_k: np.ndarray       # [Hkv][prefix_len][d]
    prefix_v: np.ndarray
    suffix_lens: np.ndarray    # int32 [B]
    suffix_k: list             # per sequence [Hkv][n][d]
    suffix_v: list
    rng: np.random.Generator   # stream for q, new tokens and copy-on-write picks

    def step_q(self):
        return normal(self.rng, (self.num_seqs, self.num_q_heads, self.head_dim), self.dtype)

    def step_tokens(self):
        shape = (self.num_seqs, self.num_kv_heads, self.head_dim)
        return normal(self.rng, shape, self.dtype), normal(self.rng, shape, self.dtype)

    def pick(self, candidates):
        """Choose ``cow_per_step`` of ``candidates`` uniformly, without replacement."""
        n = min(self.cow_per_step, len(candidates))
        idx = self.rng.choice(len(candidates), size=n, replace=False)
        return [candidates[i] for i in sorted(idx)]


def c4_shared_prefix(seed=4, num_seqs=256, prefix_len=2048, suffix_hi=512, steps=8,
                     cow_fraction=0.01, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     block_size=16, dtype=BF16):
    rng = np.random.default_rng(seed)
    suffix = rng.integers(0, suffix_hi, size=num_seqs, endpoint=True).astype(np.int32)
    prefix_blocks = ceil_div(prefix_len, block_size)
    cow_per_step = int(np.ceil(cow_fraction * num_seqs * prefix_blocks))
    # blocks in use at the end: prefix + every suffix (+ new tokens) + copies
    final = [ceil_div(prefix_len + int(n) + steps, block_size) - prefix_blocks for n in suffix]
    need = prefix_blocks + sum(final) + steps * cow_per_step
    num_blocks = int(np.ceil(1.25 * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    prefix_k = normal(rng, (num_kv_heads, prefix_len, head_dim), dtype)
    prefix_v = normal(rng, (num_kv_heads, prefix_len, head_dim), dtype)
    sk, sv = [], []
    for n in suffix:
        sk.append(normal(rng, (num_kv_heads, int(n), head_dim), dtype))
        sv.append(normal(rng, (num_kv_heads, int(n), head_dim), dtype))
    return SharedPrefixPlan(dtype=dtype, num_seqs=num_seqs, num_q_heads=num_q_heads,
                            num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                            prefix_len=prefix_len, steps=steps, cow_per_step=cow_per_step,
                            num_blocks=num_blocks, scale=float(np.float32(1.0 / np.sqrt(head_dim))),
                            free_order=free_order, prefix_k=prefix_k, prefix_v=prefix_v,
                            suffix_lens=suffix, suffix_k=sk, suffix_v=sv, rng=rng)


# --- prefix-cached prompt admission ------------------------------------------

@dataclass
class CachedPromptsPlan:
    """Inputs of the prefix-cached prompt workload.

    Every step admits ``num_seqs`` new requests whose prompts are one shared
    ``prefix_len``-token system prompt followed by a private suffix of
    ``suffix_lens[s]`` tokens (the same lengths every step, fresh token ids,
    so only the system prompt can be found in the cache).  Token ids are
    int32; K/V/q rows are token-major ``[n][heads][d]``.  Queries and K/V of
    the prefix are drawn once (the same tokens give the same KV); those of
    each request's suffix are drawn per request and reused by every step.
    """

    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    prefix_len: int
    num_blocks: int
    scale: float
    free_order: np.ndarray
    prefix_tokens: np.ndarray  # int32 [prefix_len]
    suffix_lens: np.ndarray    # int32 [B]
    prefix_q: np.ndarray       # [prefix_len][Hq][d]
    prefix_k: np.ndarray       # [prefix_len][Hkv][d]
    prefix_v: np.ndarray
    suffix_q: np.ndarray       # [sum suffix_lens][Hq][d], request after request
    suffix_k: np.ndarray       # [sum suffix_lens][Hkv][d]
    suffix_v: np.ndarray

    @property
    def suffix_cu(self):
        return np.concatenate([[0], np.cumsum(self.suffix_lens)]).astype(np.int32)

    def prompt(self, step, s):
        """Token ids of request ``s`` admitted at ``step``: the system prompt,
        then ids no other (step, request) uses."""
        n = int(self.suffix_lens[s])
        base = 1 << 20  # above every system-prompt id
        uniq = base + ((step * self.num_seqs + s) * 1024 + np.arange(n)) % ((1 << 31) - base)
        return np.concatenate([self.prefix_tokens, uniq.astype(np.int32)]).astype(np.int32)


def c8_prefix_cached_prompts(seed=8, num_seqs=64, prefix_len=2048, suffix_lo=64, suffix_hi=512,
                             num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype=BF16):
    """Llama-3-8B-shaped prompt admission with a cached 2048-token system
    prompt: 64 requests per step, private suffixes of U{64..512} tokens."""
    rng = np.random.default_rng(seed)
    suffix = rng.integers(suffix_lo, suffix_hi, size=num_seqs, endpoint=True).astype(np.int32)
    prefix_tokens = rng.integers(0, 1 << 20, size=prefix_len).astype(np.int32)
    # the uncached comparison holds every prompt privately
    need = sum(ceil_div(prefix_len + int(n), block_size) for n in suffix)
    num_blocks = int(np.ceil(1.25 * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    t = int(suffix.sum())
    return CachedPromptsPlan(
        dtype=dtype, num_seqs=num_seqs, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=block_size, prefix_len=prefix_len, num_blocks=num_blocks,
        scale=float(np.float32(1.0 / np.sqrt(head_dim))), free_order=free_order, prefix_tokens=prefix_tokens,
        suffix_lens=suffix,
        prefix_q=normal(rng, (prefix_len, num_q_heads, head_dim), dtype),
        prefix_k=normal(rng, (prefix_len, num_kv_heads, head_dim), dtype),
        prefix_v=normal(rng, (prefix_len, num_kv_heads, head_dim), dtype),
        suffix_q=normal(rng, (t, num_q_heads, head_dim), dtype),
        suffix_k=normal(rng, (t, num_kv_heads, head_dim), dtype),
        suffix_v=normal(rng, (t, num_kv_heads, head_dim), dtype))


# --- KV waste of a serving loop ----------------------------------------------

# One MI355X serving Llama-3-8B in bf16: 288 GB of HBM, 90% of it for the
# engine (the glossary entry's launch example), minus the 8.03e9 bf16 weights;
# each token's KV is 32 layers x (K + V) x 8 heads x 128 x 2 bytes.
LLAMA3_8B_KV_BYTES_PER_TOKEN = 32 * 2 * 8 * 128 * 2
MI355X_KV_CAPACITY_SLOTS = int((0.90 * 288e9 - 8.03e9 * 2) // LLAMA3_8B_KV_BYTES_PER_TOKEN)


@dataclass
class WasteCase:
    """Requests of one serving run: prompt ``p``, generated tokens ``o`` and
    contiguous slab ``r = p + max_tokens`` (the longest output the request
    may produce), all int32 [n]."""

    name: str
    capacity: int
    block_size: int
    prompt_lens: np.ndarray
    output_lens: np.ndarray
    reserve_lens: np.ndarray

    def scaled(self, k):
        """The first n / k requests on a pool k times smaller (a bounded sample)."""
        n = max(1, len(self.prompt_lens) // k)
        cap = max(self.capacity // k, int(self.reserve_lens[:n].max()))
        return WasteCase(f"{self.name}/{k}", cap, self.block_size, self.prompt_lens[:n], self.output_lens[:n],
                         self.reserve_lens[:n])


def waste_case(name="waste_llama3_8b_c2", seed=9, num_requests=4096, capacity=None, block_size=16,
               max_tokens_choices=(256, 512, 1024, 2048)):
    """Prompts from the decode workloads' length mixes (``_c2``: U{128..4096};
    ``_c5``: lognormal, median 600, sigma 1, clipped to [16, 4096]); each
    request's max_tokens drawn from ``max_tokens_choices`` and its output
    length from U{1..max_tokens} (requests stop early)."""
    rng = np.random.default_rng(seed)
    if name.endswith("_c2"):
        p = rng.integers(128, 4096, size=num_requests, endpoint=True)
    elif name.endswith("_c5"):
        p = c5_lengths(rng, num_requests, hi=4096)
    else:
        raise ValueError(name)
    m = rng.choice(np.asarray(max_tokens_choices), size=num_requests)
    o = rng.integers(1, m, endpoint=True)
    cap = MI355X_KV_CAPACITY_SLOTS if capacity is None else capacity
    return WasteCase(name, int(cap), block_size, p.astype(np.int32), o.astype(np.int32), (p + m).astype(np.int32))


CONFIGS = {
    "tiny_f32": c1_tiny_f32,
    "llama3_8b_b64": c2_llama8b_b64,
    "long_ctx_32k": c3_long_context,
    "shared_prefix_cow": c4_shared_prefix,
    "mha_b256": c5_mha_sweep,
}
