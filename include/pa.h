/*
 * pa.h -- C ABI of libpagedkv: the PagedAttention decode hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * What the operations are (PagedAttention pages):
 *   - foundry "PagedAttention" ops page, section "Concept": each sequence's KV
 *     cache is cut into fixed-size blocks that can sit anywhere in GPU memory;
 *     a per-sequence block table maps logical token positions to physical
 *     blocks; blocks are handed out on demand and freed blocks return to a
 *     shared pool.
 *   - same page, "How it works": each decode step writes the new token's key
 *     and value into the sequence's current block (pa_write_kv); a full block
 *     means a fresh block from the free pool and one more table entry
 *     (pa_seq_append); the attention kernel reads KV through the block table
 *     (pa_decode); sequences with identical content share physical blocks and
 *     copy on write when they diverge (pa_seq_cow / pa_copy_blocks); an empty
 *     pool is where a scheduler preempts (PA_ENOMEM here).
 *   - same page, "At a glance": shared blocks carry reference counts and a
 *     block is copied only when a sequence writes to it.
 *   - aiacademy lesson "Paged Attention", virtual-memory analogy table: token
 *     positions are contiguous while physical blocks are scattered; a block is
 *     allocated only when decode fills the last one.
 *
 * Layout conventions (the pages fix none of them; this header does):
 *   - KV pools: k_cache and v_cache are each
 *       [num_blocks][num_kv_heads][block_size][head_dim]
 *     of the cache element type, densely packed; one (block, head) is one
 *     contiguous run of block_size * head_dim elements.
 *   - slot of a token = physical_block * block_size + offset_in_block (int64).
 *   - block_tables: int32 [num_seqs][max_blocks_per_seq]; entry i is the
 *     physical block of logical block i; entries at or past
 *     ceil(context_len / block_size) are never read (pad them with -1).
 *   - context_lens: int32 [num_seqs]; the number of tokens each query attends
 *     to, including a token written earlier in the same step.
 *   - grouped query heads: query head h reads KV head h / (num_q_heads /
 *     num_kv_heads).
 *   - decode output: out[s][h][:] = softmax(scale * q[s][h] . K_s^T) V_s over
 *     the sequence's first context_lens[s] tokens; a sequence with length 0
 *     yields zeros.
 *   - bf16 is stored as its 16-bit pattern; fp32 accumulation throughout.
 *
 * Memory and ownership: every data pointer of a device call is a device
 * pointer owned by the caller; the library never allocates, frees or
 * synchronises.  Device calls are enqueued on `stream` (a hipStream_t passed
 * as void*; NULL is the default stream) and return after enqueueing.
 *
 * Errors: every call returns a pa_status_t; no exception crosses the ABI.
 * Argument errors visible on the host return PA_EINVAL or PA_EUNSUPPORTED and
 * enqueue nothing.  A failed launch returns PA_EHIP.  pa_last_error() gives a
 * message for the calling thread's last failure.  Values that live in device
 * memory (slots, block ids, lengths, copy pairs) are preconditions: the
 * kernels never read or write outside the buffers described by the host-side
 * sizes, and the results for out-of-range values are stated per call.
 *
 * Threading: device entry points are thread-safe.  A pa_pool is not: callers
 * serialise access to one pool.
 */
#ifndef PAGEDKV_PA_H
#define PAGEDKV_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,       /* bad argument (null pointer, size, shape)            */
  PA_EUNSUPPORTED = 2, /* valid but not built (head_dim, dtype, group size)   */
  PA_ENOMEM = 3,       /* free pool too small; pool state unchanged           */
  PA_ESTATE = 4,       /* unknown / duplicate sequence id, bad pool request   */
  PA_EHIP = 5          /* HIP runtime error while launching                   */
} pa_status_t;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype_t;

/* Shape of a pair of KV pools.  dtype is a pa_dtype_t. */
typedef struct {
  int32_t num_blocks;   /* physical blocks in each pool, > 0                 */
  int32_t block_size;   /* tokens per block: a power of two in [1, 256]      */
  int32_t num_kv_heads; /* > 0                                               */
  int32_t head_dim;     /* 64, 128 or 256                                    */
  int32_t dtype;        /* PA_F32 or PA_BF16                                 */
} pa_cache_t;

/* Library version string, e.g. "pagedkv 0.1 gfx950". */
const char *pa_version(void);

/* Message for the calling thread's most recent non-OK status. */
const char *pa_last_error(void);

/* ---------------------------------------------------------------------------
 * pa_write_kv -- store new tokens' keys and values into their slots.
 * (foundry PagedAttention page, "How it works": the new token's key and
 * value go into the sequence's current block.)
 *
 *   k, v          device [num_tokens][num_kv_heads][head_dim], cache dtype
 *   slot_mapping  device int64 [num_tokens]; token i goes to block
 *                 slot / block_size, offset slot % block_size, for every
 *                 KV head.  slot < 0 means padding: nothing is written.
 *                 Slots >= num_blocks * block_size are skipped as well.
 *   k_cache, v_cache  device pools described by *cache.
 * Distinct tokens must name distinct slots (otherwise the stored row is one
 * of the writers', unspecified which).  num_tokens == 0 is a no-op.
 * Bytes are copied unchanged: the result is bitwise the input rows.
 * ------------------------------------------------------------------------ */
pa_status_t pa_write_kv(const void *k, const void *v, const int64_t *slot_mapping,
                        int32_t num_tokens, void *k_cache, void *v_cache,
                        const pa_cache_t *cache, void *stream);

/* ---------------------------------------------------------------------------
 * pa_copy_blocks -- duplicate whole blocks for copy-on-write.
 * (foundry PagedAttention page, "How it works" and "At a glance": a shared
 * block is copied only when a sequence writes to it.)
 *
 *   src_dst_pairs  device int64 [num_pairs][2] of (src, dst) block ids.
 * Every KV head and every slot of block src is copied to block dst, in both
 * pools.  Preconditions: all dst distinct and no dst is also a src (then the
 * result equals copying from a snapshot, in any order).  Pairs with an id
 * outside [0, num_blocks) are skipped.  num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------ */
pa_status_t pa_copy_blocks(void *k_cache, void *v_cache, const pa_cache_t *cache,
                           const int64_t *src_dst_pairs, int32_t num_pairs, void *stream);

/* ---------------------------------------------------------------------------
 * pa_swap_blocks -- copy whole blocks between two pools, typically a device
 * pool and a swap pool in pinned host memory (in either direction).
 * (foundry PagedAttention page, How it works and Trade-offs: a preempted
 * sequence's blocks can be swapped out to CPU memory and back in.)
 *
 *   src_k, src_v / dst_k, dst_v  pools described by *src_cache / *dst_cache
 *                 (the same block shape and dtype; num_blocks may differ).
 *                 Device memory, or host memory the device can address
 *                 (hipHostMalloc, e.g. torch pin_memory): the kernel reads
 *                 and writes it directly.  16-byte aligned.
 *   src_dst_pairs device-addressable int64 [num_pairs][2]: block src of the
 *                 source pools goes to block dst of the destination pools,
 *                 every KV head and slot, K and V.  Pairs naming a block
 *                 outside its pool are skipped.
 * Preconditions: distinct destinations; source and destination pools do not
 * overlap.  Bytes are copied unchanged.  num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------ */
pa_status_t pa_swap_blocks(const void *src_k, const void *src_v, const pa_cache_t *src_cache,
                           void *dst_k, void *dst_v, const pa_cache_t *dst_cache,
                           const int64_t *src_dst_pairs, int32_t num_pairs, void *stream);

/* ---------------------------------------------------------------------------
 * pa_decode -- single-query paged decode attention.
 * (foundry PagedAttention page, "How it works": the attention kernel reads
 * KV through the block table, gathering scattered blocks, so non-contiguous
 * storage leaves the math unchanged.)
 *
 *   q             device [num_seqs][num_q_heads][head_dim], cache dtype
 *   k_cache, v_cache, *cache   the pools (as above)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  device int32 [num_seqs]
 *   max_context_len  host bound >= every context_lens[s]; sizes the launch.
 *                 Lengths are clamped to min(max_context_len,
 *                 max_blocks_per_seq * block_size).
 *   scale         softmax scale (usually 1/sqrt(head_dim))
 *   partition_size how each (sequence, KV head) context is cut into
 *                 workgroup ranges:
 *                 0: one range per (sequence, KV head), no workspace;
 *                 a multiple of block_size: ranges of that many tokens,
 *                   processed in parallel and merged by a second kernel
 *                   (online-softmax merge);
 *                 PA_PARTITION_BALANCED (-1): the library divides all
 *                   (sequence, KV head, token) work into equal shares, one per
 *                   workgroup slot of the GPU, and merges the sequences a
 *                   share boundary cuts.  Used for bf16 pools with 4 or 8 query
 *                   heads per KV head, up to 8192 sequences and
 *                   num_seqs * (max_context_len + 271) < 2^31.  Other
 *                   bf16 batches with 4 or 8 query heads per KV head run in
 *                   4096-token partitions when a context is longer than
 *                   that; fp32 pools and 1 or 2 query heads per KV head run
 *                   in 1024-token partitions when a context is longer than
 *                   that; anything shorter runs unpartitioned.  The result
 *                   is the same from call to call for the same inputs.
 *   workspace     device scratch of at least pa_decode_workspace_bytes(...)
 *                 bytes, 256-byte aligned, when partition_size != 0 (may be
 *                 NULL otherwise); its contents on entry do not matter.
 *   out           device [num_seqs][num_q_heads][head_dim] of out_dtype
 *                 (PA_F32, or the cache dtype).
 * num_q_heads must be a multiple of num_kv_heads, with a ratio of 1, 2, 4 or
 * 8.  Block ids outside [0, num_blocks) inside a sequence's length are a
 * precondition violation: the kernel stays inside the pools but that
 * sequence's output is unspecified.  The result does not depend on where the
 * blocks sit in the pool; it depends on partition_size only through fp32
 * rounding of the summation order.
 * ------------------------------------------------------------------------ */
#define PA_PARTITION_BALANCED (-1)

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size);

pa_status_t pa_decode(const void *q, int32_t num_seqs, int32_t num_q_heads,
                      const void *k_cache, const void *v_cache, const pa_cache_t *cache,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t max_context_len, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *out, int32_t out_dtype, void *stream);

/* ---------------------------------------------------------------------------
 * pa_decode_write -- pa_write_kv(k, v, slot_mapping, num_tokens) followed by
 * pa_decode(...), as one call.
 * (foundry PagedAttention page, "How it works": a decode step stores the new
 * token's key and value in the sequence's current block, and attention then
 * reads the whole context, that token included, through the block table.)
 *
 * Arguments: those of pa_write_kv (k, v, slot_mapping, num_tokens), then
 * those of pa_decode; k_cache and v_cache are written.  The pools after the
 * call and out are those of the two calls in sequence (bitwise), given this
 * precondition: on the balanced path with num_tokens == num_seqs, token i
 * must be sequence i's newest position, slot_mapping[i] being the slot the
 * block table gives for position context_lens[i] - 1 (or < 0 to store
 * nothing, only for a sequence of length 0).  That path is one kernel: the
 * tokens are stored while it runs and the attention reads position
 * context_lens[i] - 1 from k and v themselves.  Otherwise the call runs
 * pa_write_kv, then pa_decode.  Errors: those of the two calls; with
 * num_seqs == 0 only the store is done.
 * ------------------------------------------------------------------------ */
pa_status_t pa_decode_write(const void *k, const void *v, const int64_t *slot_mapping,
                            int32_t num_tokens, const void *q, int32_t num_seqs,
                            int32_t num_q_heads, void *k_cache, void *v_cache,
                            const pa_cache_t *cache, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t max_context_len, float scale, int32_t partition_size,
                            void *workspace, size_t workspace_bytes, void *out,
                            int32_t out_dtype, void *stream);

/* ---------------------------------------------------------------------------
 * pa_decode_write_noalloc -- pa_decode_write without a workspace argument,
 * for callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, result and errors: those of pa_decode_write, minus workspace
 * and workspace_bytes; the same kernels run.  The scratch those kernels need
 * (partial softmax statistics of the cut sequences, the split's header) is a
 * static device array of PA_NOALLOC_SCRATCH_BYTES inside the library: each
 * GPU the library runs on holds its own copy until the process ends.  A call
 * whose scratch need (pa_decode_workspace_bytes of the same arguments)
 * exceeds it returns PA_EINVAL and enqueues nothing.  The call allocates and
 * frees nothing (no hipMalloc / hipFree, no allocating library routine);
 * the first call on a device looks up that device's scratch address once.
 * The scratch starts each call in whatever state the last one left; the
 * kernels write every byte they read before reading it.  Calls that overlap
 * on one GPU (other streams, other threads) share that scratch and race:
 * serialise them.
 * ------------------------------------------------------------------------ */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

pa_status_t pa_decode_write_noalloc(const void *k, const void *v, const int64_t *slot_mapping,
                                    int32_t num_tokens, const void *q, int32_t num_seqs,
                                    int32_t num_q_heads, void *k_cache, void *v_cache,
                                    const pa_cache_t *cache, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                                    int32_t max_context_len, float scale, int32_t partition_size,
                                    void *out, int32_t out_dtype, void *stream);

/* ---------------------------------------------------------------------------
 * pa_prefill -- causal attention of a chunk of new queries per sequence (a
 * prompt, or its next piece), reading keys and values through the block table.
 * (foundry PagedAttention page, Concept and How it works: a sequence's keys
 * and values sit in the blocks its table names, wherever they are, and the
 * attention reads them through the table; a prompt is many tokens at once.)
 *
 *   q             device [num_tokens][num_q_heads][head_dim], bf16; the
 *                 queries of all sequences packed in sequence order.
 *   cu_seqlens    device int32 [num_seqs + 1]: sequence s owns query rows
 *                 cu_seqlens[s] .. cu_seqlens[s + 1] - 1 (n_s of them),
 *                 non-decreasing from 0 to at most num_tokens; n_s <=
 *                 max_query_len (a host bound; rows past it are not
 *                 computed).
 *   context_lens  device int32 [num_seqs]: keys of sequence s after its new
 *                 tokens were stored (pa_write_kv); its n_s queries are its
 *                 last n_s positions: query i sits at position
 *                 context_lens[s] - n_s + i and attends to keys 0 .. that
 *                 position (softmax(q K^T * scale) V).  A query at a
 *                 position below 0 attends to nothing and its row is zero.
 *   block_tables, max_blocks_per_seq, max_context_len: as for pa_decode
 *                 (lengths are clamped to min(max_context_len,
 *                 max_blocks_per_seq * block_size)).
 *   scale         the softmax scale; positive and finite, else PA_EINVAL.
 *   out           device [num_tokens][num_q_heads][head_dim] of out_dtype
 *                 (PA_F32 or PA_BF16).
 * Built for bf16 pools, head_dim 64 or 128, 1, 2, 4 or 8 query heads per KV
 * head, power-of-two block sizes up to 256 and num_kv_heads x block_size
 * below 2^31 (rows per pool block); otherwise PA_EUNSUPPORTED.
 * Scores and the softmax are fp32; the probabilities enter the product with
 * V rounded to bf16.  num_seqs, num_tokens or max_query_len == 0: no-op.
 * ------------------------------------------------------------------------ */
pa_status_t pa_prefill(const void *q, int32_t num_tokens, int32_t num_q_heads,
                       const int32_t *cu_seqlens, int32_t num_seqs, int32_t max_query_len,
                       const void *k_cache, const void *v_cache, const pa_cache_t *cache,
                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                       const int32_t *context_lens, int32_t max_context_len, float scale,
                       void *out, int32_t out_dtype, void *stream);

/* ---------------------------------------------------------------------------
 * pa_prefill_write -- pa_write_kv(k, v, slot_mapping, num_tokens) followed by
 * pa_prefill(...), as one call: a prompt's (or chunk's) keys and values are
 * stored in their blocks and its queries attend.
 * (foundry PagedAttention page, "How it works": new tokens' keys and values
 * go into the sequence's blocks, and attention reads the whole context, the
 * new tokens included, through the block table; a prompt is many tokens.)
 *
 * Arguments: k, v (device [num_tokens][num_kv_heads][head_dim], bf16: row r
 * holds the key and value of query row r) and slot_mapping (device int64
 * [num_tokens]; slots < 0 or outside the pool are skipped), then those of
 * pa_prefill; k_cache and v_cache are written.  The pools after the call and
 * out are those of the two calls in sequence (bitwise), given this
 * precondition: cu_seqlens[num_seqs] == num_tokens, no length above
 * min(max_context_len, max_blocks_per_seq * block_size), and for every row r
 * of sequence s, slot_mapping[r] is the slot the block table gives for the
 * row's position context_lens[s] - n_s + (r - cu_seqlens[s]) (or < 0 only
 * where that position is below 0).  With head_dim 128 and block_size >= 8
 * that is one kernel: the rows are stored while it runs and the attention
 * reads the chunk's keys and values from k and v themselves.  Otherwise the
 * call runs pa_write_kv, then pa_prefill.  Errors: those of the two calls,
 * all found before anything is enqueued, plus PA_EINVAL when k or v is not
 * 16-byte aligned; num_seqs, max_query_len == 0: only the store is done.
 * ------------------------------------------------------------------------ */
pa_status_t pa_prefill_write(const void *k, const void *v, const int64_t *slot_mapping, const void *q,
                             int32_t num_tokens, int32_t num_q_heads, const int32_t *cu_seqlens,
                             int32_t num_seqs, int32_t max_query_len, void *k_cache, void *v_cache,
                             const pa_cache_t *cache, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *context_lens,
                             int32_t max_context_len, float scale, void *out, int32_t out_dtype,
                             void *stream);

/* ---------------------------------------------------------------------------
 * Host block manager (host memory only, no device calls).
 * (foundry PagedAttention page, "Concept", "How it works", "At a glance";
 * aiacademy lesson "Paged Attention", analogy table.)
 *
 * Policy fixed by this library where the pages leave it open:
 *   - the free pool is a stack that starts as free_order (free_order[0] is
 *     handed out first; NULL means 0, 1, 2, ...); released blocks are pushed
 *     on top and handed out next;
 *   - a sequence holds exactly ceil(len / block_size) blocks;
 *   - appending to a block whose reference count is > 1 first moves the
 *     writer to a fresh private copy (the pair (src, dst) is reported for
 *     pa_copy_blocks); the other sharers keep src;
 *   - releasing a sequence walks its table in logical order;
 *   - every failing call leaves the pool unchanged.
 * Sequence ids are arbitrary int64 values chosen by the caller.
 * ------------------------------------------------------------------------ */
typedef struct pa_pool pa_pool;

/* Create a pool; *out receives the handle (owned by the caller until
 * pa_pool_destroy).  free_order: host int32 [num_blocks] permutation or NULL. */
pa_status_t pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order,
                           pa_pool **out);
void pa_pool_destroy(pa_pool *pool);

int32_t pa_pool_num_free(const pa_pool *pool);
/* Reference count of a block, or -1 for an id outside the pool. */
int32_t pa_pool_refcount(const pa_pool *pool, int32_t block);
/* Free blocks in hand-out order into host out[cap]; *n receives the count. */
pa_status_t pa_pool_free_list(const pa_pool *pool, int32_t *out, int32_t cap, int32_t *n);

/* New sequence with num_tokens tokens (ceil(n / block_size) fresh blocks). */
pa_status_t pa_seq_create(pa_pool *pool, int64_t seq, int32_t num_tokens);
/* child shares every block of parent (reference counts + 1). */
pa_status_t pa_seq_fork(pa_pool *pool, int64_t parent, int64_t child);
/* Reserve the slot of one new token of seq.  *slot receives it; cow_pair[2]
 * receives (src, dst) when a shared block had to be copied first, else
 * (-1, -1). */
pa_status_t pa_seq_append(pa_pool *pool, int64_t seq, int64_t *slot, int64_t cow_pair[2]);
/* pa_seq_append for seqs[0..n) in order, all or nothing.  slots: host int64
 * [n]; pairs: host int64 [n][2] receives the copy pairs in order, *num_pairs
 * their count (at most n). */
pa_status_t pa_seq_append_batch(pa_pool *pool, const int64_t *seqs, int32_t n, int64_t *slots,
                                int64_t *pairs, int32_t *num_pairs);
/* Give seq a private copy of logical block lb if it is shared: pair (src,
 * dst), else (-1, -1) and nothing changes. */
pa_status_t pa_seq_cow(pa_pool *pool, int64_t seq, int32_t logical_block, int64_t pair[2]);
/* Release every block of seq (counts - 1; blocks reaching 0 return to the
 * pool) and forget seq. */
pa_status_t pa_seq_free(pa_pool *pool, int64_t seq);
/* Slots of logical positions [start, start + count) of seq into host
 * slots[count]. */
pa_status_t pa_seq_slots(const pa_pool *pool, int64_t seq, int32_t start, int32_t count,
                         int64_t *slots);
/* Table row of seq into host row[max_blocks] (padded with -1), plus its block
 * count and length (host swap block ids while seq is swapped out).
 * PA_EINVAL if the row does not fit. */
pa_status_t pa_seq_table(const pa_pool *pool, int64_t seq, int32_t *row, int32_t max_blocks,
                         int32_t *num_blocks, int32_t *len);
/* Tables and lengths of seqs[0..n) into host tables[n][max_blocks] (padded
 * with -1) and context_lens[n], ready to upload for pa_decode. */
pa_status_t pa_pool_tables(const pa_pool *pool, const int64_t *seqs, int32_t n, int32_t *tables,
                           int32_t max_blocks, int32_t *context_lens);

/* Swap space (foundry page, How it works and Trade-offs: under memory
 * pressure a sequence is preempted and its blocks can move to CPU memory and
 * back).  The pool can own a second stack of num_host_blocks host swap
 * blocks, handed out in host_free_order (NULL: 0, 1, ...), LIFO afterwards;
 * the caller keeps the swap pools themselves (pa_swap_blocks moves the data).
 * A swapped-out sequence may only be swapped in, inspected (pa_seq_table,
 * pa_seq_is_swapped) or freed; other calls on it return PA_ESTATE, and so do
 * pa_seq_slots / pa_pool_tables.  Every call succeeds or changes nothing. */
/* Set up or replace the swap space; PA_ESTATE while a sequence is swapped
 * out. */
pa_status_t pa_pool_set_swap_space(pa_pool *pool, int32_t num_host_blocks, const int32_t *host_free_order);
int32_t pa_pool_num_free_host(const pa_pool *pool);
/* Free host blocks in hand-out order into out[cap]; *n = their count. */
pa_status_t pa_pool_host_free_list(const pa_pool *pool, int32_t *out, int32_t cap, int32_t *n);
/* 1 swapped out, 0 resident, -1 unknown sequence (or NULL pool). */
int32_t pa_seq_is_swapped(const pa_pool *pool, int64_t seq);
/* Swap seq out: each logical block, in order, gets a host block h; the pair
 * (device block, h) is written to pairs[i][2] (cap pairs of room) and the
 * device block loses one reference (it returns to the free pool unless
 * another sequence shares it).  *num_pairs = blocks of seq.  PA_ENOMEM when
 * the swap space has too few free blocks. */
pa_status_t pa_seq_swap_out(pa_pool *pool, int64_t seq, int64_t *pairs, int32_t cap, int32_t *num_pairs);
/* Swap seq back in: each host block, in logical order, gets a fresh device
 * block b; pairs[i] = (host block, b); the host blocks return to the swap
 * space.  PA_ENOMEM when the free pool is too small. */
pa_status_t pa_seq_swap_in(pa_pool *pool, int64_t seq, int64_t *pairs, int32_t cap, int32_t *num_pairs);

/* Prefix caching (aimodelwiki "PagedAttention" glossary entry, the paragraph
 * on prefix caching: prompt prefixes shared across requests reuse KV pages
 * already computed; foundry "PagedAttention" ops page, At a glance: shared
 * blocks are tracked by reference count).
 * Once enabled, a sequence created from its prompt tokens
 * (pa_seq_create_cached) registers each of its full blocks under the exact
 * key (prefix before the block, the block's tokens) -- no hash, so no
 * collision -- and a later prompt shares the longest run of its leading full
 * blocks found that way.  A cached block whose count drops to 0 is not freed:
 * it waits, unreferenced, at the tail of an LRU list, and is found again by
 * later prompts.  Blocks are taken from the free stack first, then by
 * evicting the LRU head (its key is forgotten).  A cached block is
 * immutable: pa_seq_cow copies it even when its count is 1.  Blocks filled
 * by pa_seq_append are never registered.  Every call succeeds or changes
 * nothing. */
pa_status_t pa_pool_enable_prefix_cache(pa_pool *pool);
/* Cached blocks with count 0 (the LRU list), or -1 for a NULL pool. */
int32_t pa_pool_num_cached(const pa_pool *pool);
/* 1 if block is registered in the prefix cache, 0 if not, -1 outside the pool. */
int32_t pa_pool_is_cached(const pa_pool *pool, int32_t block);
/* LRU list, least recently released first, into host out[cap]; *n = count. */
pa_status_t pa_pool_lru_list(const pa_pool *pool, int32_t *out, int32_t cap, int32_t *n);
/* New sequence holding tokens[0..num_tokens) (host int32): the leading full
 * blocks found in the cache are shared (counts + 1), the rest are taken
 * fresh, and the new full blocks are registered.  *num_cached_tokens
 * receives the number of leading tokens whose KV is already in the pool (a
 * multiple of block_size); the caller computes and writes only the rest.
 * PA_ESTATE if caching is off or seq exists, PA_ENOMEM if the fresh blocks
 * do not fit (free + evictable blocks, not counting the hits themselves). */
pa_status_t pa_seq_create_cached(pa_pool *pool, int64_t seq, const int32_t *tokens, int32_t num_tokens,
                                 int32_t *num_cached_tokens);
/* pa_seq_create_cached for n requests in one call, in order: request i is
 * sequence seqs[i] (host int64 [n]) with tokens[offsets[i] .. offsets[i+1])
 * (host int32 tokens, host int64 offsets [n + 1], offsets[0] = 0).  For each
 * admitted request num_cached[i] (host int32 [n]) receives its cached token
 * count and slots (host int64, room for slots_cap >= offsets[n] entries)
 * receives the slots of its uncached tokens, request after request, in
 * position order: where pa_write_kv stores their K/V.  The first request that
 * is refused ends the batch: the call returns its status (PA_ENOMEM when the
 * pool is full), the requests before it stay admitted.  *num_admitted and
 * *num_slots receive the admitted count and the slots written.  Argument
 * errors (PA_EINVAL) admit nothing. */
pa_status_t pa_seq_create_cached_batch(pa_pool *pool, const int64_t *seqs, int32_t n, const int32_t *tokens,
                                       const int64_t *offsets, int32_t *num_cached, int64_t *slots,
                                       int64_t slots_cap, int32_t *num_admitted, int64_t *num_slots);

/* ------------------------------------------------------------------------
 * KV-cache waste of a serving loop (host only).
 *
 * foundry "PagedAttention" ops page, Concept and At a glance: a contiguous
 * slab per request, sized to its maximum length, strands its unfilled slots
 * and leaves gaps too small to reuse; paged blocks, handed out one at a time
 * on demand, waste at most one partly filled block per sequence.  aiacademy
 * "Paged Attention" lesson: the slab is sized for the longest output the
 * request might produce.
 *
 * pa_waste_simulate runs num_requests requests (all queued at step 0, in
 * order) through one pool of capacity KV token slots until all finish.
 * Request i has a prompt of prompt_lens[i] >= 1 tokens, generates
 * output_lens[i] >= 1 tokens and, contiguous, reserves a slab of
 * reserve_lens[i] >= p + o slots (host int32 arrays).  Each step: admit
 * from the head of the queue while it fits (PA_WASTE_CONTIGUOUS: first fit,
 * the lowest-addressed free gap of at least r slots, freed slabs merge with
 * free neighbours; PA_WASTE_PAGED: ceil(p / block_size) blocks of this
 * library's block manager over capacity / block_size blocks); record the
 * counters below; store one token for every running request (paged: a
 * request needing a block when none is free preempts the most recently
 * admitted running request -- its blocks freed, its progress lost, back to
 * the front of the queue -- until a block is free or it preempted itself);
 * retire finished requests.  *out receives the totals.  PA_EINVAL for a
 * request that cannot fit in the pool alone or breaks p >= 1, o >= 1,
 * r >= p + o. */
#define PA_WASTE_CONTIGUOUS 0
#define PA_WASTE_PAGED 1
typedef struct pa_waste_stats {
  int64_t steps;
  int64_t live_slot_steps;    /* sum over steps of tokens stored by running requests */
  int64_t held_slot_steps;    /* sum over steps of slots they hold (slabs, or blocks x block_size) */
  int64_t running_steps;      /* sum over steps of running requests */
  int64_t max_running;
  int64_t preemptions;        /* paged only */
  int64_t frag_blocked_steps; /* contiguous: steps whose queue head was refused although the
                                 free slots added up to its slab */
  int64_t decode_tokens;      /* tokens stored after admission, including ones lost to preemption */
} pa_waste_stats;
pa_status_t pa_waste_simulate(int32_t mode, int64_t capacity, int32_t block_size, const int32_t *prompt_lens,
                              const int32_t *output_lens, const int32_t *reserve_lens, int32_t num_requests,
                              pa_waste_stats *out);

/* ---------------------------------------------------------------------------
 * pa_read_probe -- measurement helper, not a step of the attention path.
 * Streams a device buffer once with 16-byte non-temporal loads, each of
 * PA_READ_PROBE_WORKGROUPS workgroups walking one contiguous run of it; its
 * rate is the practical read ceiling of the device, reported beside the HBM
 * peak when the decode's bandwidth is measured.
 *
 *   buf     device, 16-byte aligned, `bytes` long (a multiple of 16; 0 is
 *           allowed); read only.
 *   sink    device uint32 [PA_READ_PROBE_WORKGROUPS]: workgroup w writes the
 *           XOR of the 32-bit words it read, so the XOR of all of sink is
 *           the XOR of every 32-bit word of buf (a check that every byte was
 *           read).
 * Caller-owned memory; asynchronous on `stream`; PA_EINVAL for a size that
 * is not a multiple of 16, a misaligned buffer or a NULL pointer.
 * ------------------------------------------------------------------------ */
#define PA_READ_PROBE_WORKGROUPS 8192
pa_status_t pa_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PA_H */
