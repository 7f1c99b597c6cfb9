// Host block manager: free pool, reference counts, per-sequence block tables.
//
// foundry "PagedAttention" ops page:
//   * Concept -- blocks are handed out one at a time on demand; freed blocks
//     return to a shared pool; waste is at most one partly filled block per
//     sequence.
//   * How it works -- the new token goes into the current block; a full block
//     means a fresh block from the global free pool and a longer block table;
//     sequences with identical content point at the same physical blocks and
//     copy on write when they diverge; an empty pool is where a scheduler
//     preempts.
//   * At a glance -- sharing is tracked by reference counts; a block is copied
//     only when a sequence writes to it.
// aiacademy lesson "Paged Attention", analogy table -- a block is allocated only
// when decode fills the last one; any free block fits any request.
//
// Policy (the pages leave it open): the free pool is a LIFO stack seeded with
// free_order so that free_order[0] is handed out first; release walks a table
// in logical order; the writer of a shared block gets the private copy.  Every
// call either succeeds or leaves the pool untouched.
//
// Swap (foundry page, How it works and Trade-offs: when the pool runs dry a
// scheduler preempts, and a preempted sequence's blocks can be swapped out to
// CPU memory and back in): an optional host swap space of its own blocks, a
// second LIFO stack.  Swapping a sequence out gives each of its logical
// blocks its own host block (in logical order) and drops one reference to
// the device block, which returns to the free pool when no other sequence
// shares it; swapping in takes a device block per host block and returns the
// host blocks.  A swapped-out sequence can only be swapped in, inspected or
// freed.
//
// Prefix caching (aimodelwiki "PagedAttention" glossary entry, prefix-caching
// paragraph: requests that share a prompt prefix reuse its KV blocks; foundry
// ops page, At a glance: shared blocks are tracked by reference count):
// when enabled, the full blocks of a sequence created from its prompt tokens
// are registered under the key (prefix node of the block before it, the
// block's tokens); lookups go through a 64-bit hash of that key and then
// compare the key itself, so a hash collision can never share wrong KV; node
// ids are never reused.  A later prompt walks its full blocks through the cache and shares
// the longest cached run.  A cached block whose count drops to 0 is kept,
// unreferenced, at the tail of an LRU list; blocks are taken from the free
// stack first and then by evicting the LRU head (which leaves the cache).

#include <cstdint>
#include <cstring>
#include <list>
#include <algorithm>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa.h"
#include "pa_status.h"

namespace {

struct Seq {
  std::vector<int32_t> table;  // device block ids, or host swap blocks while swapped out
  int64_t len = 0;
  bool swapped = false;
};

}  // namespace

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;
  int32_t num_host_blocks = 0;
  std::vector<int32_t> host_free;  // host swap blocks; back() is handed out next
  int32_t swapped_seqs = 0;

  // Prefix cache: key (parent node, tokens of the block) -> (block, node),
  // found by the key's hash and confirmed by comparing the key.
  struct CacheEntry {
    int64_t parent;
    std::vector<int32_t> tokens;
    int32_t block;
    int64_t node;
  };
  bool prefix_cache = false;
  int64_t next_node = 1;  // node 0 is the empty prefix
  std::unordered_multimap<uint64_t, CacheEntry> cache;  // elements keep their address on rehash
  std::vector<const CacheEntry *> block_key;            // entry of a cached block, or nullptr
  std::vector<uint64_t> block_hash;

  static uint64_t key_hash(int64_t parent, const int32_t *tok, int32_t n) {
    // FNV-1a over the parent id and the token ids, then a final avalanche
    uint64_t h = 0xcbf29ce484222325ull ^ (uint64_t)parent;
    h *= 0x100000001b3ull;
    for (int32_t i = 0; i < n; ++i) {
      h ^= (uint32_t)tok[i];
      h *= 0x100000001b3ull;
    }
    h ^= h >> 33;
    h *= 0xff51afd7ed558ccdull;
    h ^= h >> 33;
    return h;
  }
  const CacheEntry *find(uint64_t h, int64_t parent, const int32_t *tok, int32_t n) const {
    auto range = cache.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const CacheEntry &e = it->second;
      if (e.parent == parent && std::equal(e.tokens.begin(), e.tokens.end(), tok, tok + n)) return &e;
    }
    return nullptr;
  }
  void forget(int32_t b) {  // drop a cached block's entry
    auto range = cache.equal_range(block_hash[b]);
    for (auto it = range.first; it != range.second; ++it) {
      if (&it->second == block_key[b]) {
        cache.erase(it);
        break;
      }
    }
    block_key[b] = nullptr;
  }
  std::list<int32_t> lru;                   // cached blocks with count 0, least recent first
  std::vector<std::list<int32_t>::iterator> lru_pos;

  // Blocks a request can still get: free ones and evictable cached ones.
  size_t available() const { return free_stack.size() + lru.size(); }

  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {  // evict the least recently released cached block
      b = lru.front();
      lru.pop_front();
      forget(b);
    }
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) {
      if (block_key[b]) lru_pos[b] = lru.insert(lru.end(), b);
      else free_stack.push_back(b);
    }
  }
  // A cached block gains a reference (leaving the LRU list if it had none).
  void reuse(int32_t b) {
    if (refcount[b]++ == 0) lru.erase(lru_pos[b]);
  }
  // Blocks one append to `s` needs: 1 for a fresh or copied block, else 0.
  int32_t append_need(const Seq &s) const {
    int64_t off = s.len % block_size;
    if (off == 0) return 1;
    return refcount[s.table[s.len / block_size]] > 1 ? 1 : 0;
  }
  // Performs one append; the caller has checked that a block is available.
  void append(Seq &s, int64_t *slot, int64_t pair[2]) {
    int64_t lb = s.len / block_size, off = s.len % block_size;
    pair[0] = pair[1] = -1;
    if (off == 0) {
      s.table.push_back(take());
    } else if (refcount[s.table[lb]] > 1) {
      int32_t src = s.table[lb];
      int32_t dst = take();
      release(src);
      s.table[lb] = dst;
      pair[0] = src;
      pair[1] = dst;
    }
    *slot = (int64_t)s.table[lb] * block_size + off;
    s.len += 1;
  }
};

using pa::fail;

namespace {
// A resident (not swapped-out) sequence, or an error.
pa_status_t resident(pa_pool *pool, int64_t seq, const char *fn, Seq **out) {
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_ESTATE, "%s: unknown sequence %lld", fn, (long long)seq);
  if (it->second.swapped) return fail(PA_ESTATE, "%s: sequence %lld is swapped out", fn, (long long)seq);
  *out = &it->second;
  return PA_OK;
}
}  // namespace

extern "C" {

pa_status_t pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order,
                           pa_pool **out) {
  if (!out) return fail(PA_EINVAL, "pa_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_EINVAL, "pa_pool_create: num_blocks=%d block_size=%d must be > 0", num_blocks,
                block_size);
  pa_pool *p = new (std::nothrow) pa_pool;
  if (!p) return fail(PA_ENOMEM, "pa_pool_create: host allocation failed");
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->refcount.assign(num_blocks, 0);
  p->block_key.assign(num_blocks, nullptr);
  p->block_hash.assign(num_blocks, 0);
  p->lru_pos.resize(num_blocks);
  p->free_stack.resize(num_blocks);
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete p;
      return fail(PA_EINVAL, "pa_pool_create: free_order is not a permutation (entry %d = %d)", i,
                  b);
    }
    seen[b] = 1;
    p->free_stack[num_blocks - 1 - i] = b;
  }
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool *pool) { delete pool; }

int32_t pa_pool_num_free(const pa_pool *pool) {
  return pool ? (int32_t)pool->free_stack.size() : -1;
}

int32_t pa_pool_refcount(const pa_pool *pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->refcount[block];
}

pa_status_t pa_pool_free_list(const pa_pool *pool, int32_t *out, int32_t cap, int32_t *n) {
  if (!pool || !n) return fail(PA_EINVAL, "pa_pool_free_list: NULL argument");
  int32_t total = (int32_t)pool->free_stack.size();
  *n = total;
  if (total > cap || (total > 0 && !out))
    return fail(PA_EINVAL, "pa_pool_free_list: %d free blocks do not fit in %d", total, cap);
  for (int32_t i = 0; i < total; ++i) out[i] = pool->free_stack[total - 1 - i];
  return PA_OK;
}

pa_status_t pa_seq_create(pa_pool *pool, int64_t seq, int32_t num_tokens) {
  if (!pool) return fail(PA_EINVAL, "pa_seq_create: pool is NULL");
  if (num_tokens < 0) return fail(PA_EINVAL, "pa_seq_create: num_tokens=%d < 0", num_tokens);
  if (pool->seqs.count(seq)) return fail(PA_ESTATE, "pa_seq_create: sequence %lld exists", (long long)seq);
  int64_t need = ((int64_t)num_tokens + pool->block_size - 1) / pool->block_size;
  if (need > (int64_t)pool->available())
    return fail(PA_ENOMEM, "pa_seq_create: %lld blocks needed, %zu free", (long long)need,
                pool->available());
  Seq s;
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(pool->take());
  s.len = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status_t pa_seq_fork(pa_pool *pool, int64_t parent, int64_t child) {
  if (!pool) return fail(PA_EINVAL, "pa_seq_fork: pool is NULL");
  Seq *par;
  if (pa_status_t st = resident(pool, parent, "pa_seq_fork", &par)) return st;
  if (pool->seqs.count(child)) return fail(PA_ESTATE, "pa_seq_fork: sequence %lld exists", (long long)child);
  Seq s = *par;
  for (int32_t b : s.table) pool->refcount[b] += 1;
  pool->seqs.emplace(child, std::move(s));
  return PA_OK;
}

pa_status_t pa_seq_append(pa_pool *pool, int64_t seq, int64_t *slot, int64_t cow_pair[2]) {
  if (!pool || !slot || !cow_pair) return fail(PA_EINVAL, "pa_seq_append: NULL argument");
  Seq *sq;
  if (pa_status_t st = resident(pool, seq, "pa_seq_append", &sq)) return st;
  if (pool->append_need(*sq) > (int32_t)pool->available())
    return fail(PA_ENOMEM, "pa_seq_append: free pool is empty");
  pool->append(*sq, slot, cow_pair);
  return PA_OK;
}

pa_status_t pa_seq_append_batch(pa_pool *pool, const int64_t *seqs, int32_t n, int64_t *slots,
                                int64_t *pairs, int32_t *num_pairs) {
  if (!pool || !num_pairs || n < 0 || (n > 0 && (!seqs || !slots || !pairs)))
    return fail(PA_EINVAL, "pa_seq_append_batch: bad argument");
  *num_pairs = 0;
  std::vector<Seq *> refs(n);
  for (int32_t i = 0; i < n; ++i)
    if (pa_status_t st = resident(pool, seqs[i], "pa_seq_append_batch", &refs[i])) return st;
  // Dry run on counts only, so that a shortage is found before anything
  // changes.  A repeated sequence sees its own earlier appends.
  {
    std::unordered_map<int64_t, int64_t> extra_len;   // appends so far per seq
    std::unordered_map<int64_t, char> private_tail;   // tail block already private
    std::unordered_map<int32_t, int32_t> rc_drop;     // shared tails left so far
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      const Seq &s = *refs[i];
      int64_t len = s.len + extra_len[seqs[i]];
      int64_t off = len % pool->block_size;
      if (off == 0) {
        need += 1;
        private_tail[seqs[i]] = 1;
      } else if (!private_tail[seqs[i]]) {
        int32_t b = s.table[len / pool->block_size];
        if (pool->refcount[b] - rc_drop[b] > 1) {
          need += 1;
          rc_drop[b] += 1;
        }
        private_tail[seqs[i]] = 1;
      }
      extra_len[seqs[i]] += 1;
    }
    if (need > (int64_t)pool->available())
      return fail(PA_ENOMEM, "pa_seq_append_batch: %lld blocks needed, %zu free", (long long)need,
                  pool->available());
  }
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int64_t pair[2];
    pool->append(*refs[i], &slots[i], pair);
    if (pair[0] >= 0) {
      pairs[2 * np] = pair[0];
      pairs[2 * np + 1] = pair[1];
      ++np;
    }
  }
  *num_pairs = np;
  return PA_OK;
}

pa_status_t pa_seq_cow(pa_pool *pool, int64_t seq, int32_t logical_block, int64_t pair[2]) {
  if (!pool || !pair) return fail(PA_EINVAL, "pa_seq_cow: NULL argument");
  pair[0] = pair[1] = -1;
  Seq *sq;
  if (pa_status_t st = resident(pool, seq, "pa_seq_cow", &sq)) return st;
  Seq &s = *sq;
  if (logical_block < 0 || logical_block >= (int32_t)s.table.size())
    return fail(PA_ESTATE, "pa_seq_cow: logical block %d outside [0, %zu)", logical_block,
                s.table.size());
  int32_t src = s.table[logical_block];
  // private and not in the prefix cache: written in place, no copy (a
  // cached block is immutable: others may find it by its tokens)
  if (pool->refcount[src] == 1 && !pool->block_key[src]) return PA_OK;
  if (pool->available() == 0) return fail(PA_ENOMEM, "pa_seq_cow: free pool is empty");
  int32_t dst = pool->take();
  pool->release(src);
  s.table[logical_block] = dst;
  pair[0] = src;
  pair[1] = dst;
  return PA_OK;
}

pa_status_t pa_seq_free(pa_pool *pool, int64_t seq) {
  if (!pool) return fail(PA_EINVAL, "pa_seq_free: pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_ESTATE, "pa_seq_free: unknown sequence %lld", (long long)seq);
  if (it->second.swapped) {
    for (int32_t h : it->second.table) pool->host_free.push_back(h);
    pool->swapped_seqs -= 1;
  } else {
    for (int32_t b : it->second.table) pool->release(b);
  }
  pool->seqs.erase(it);
  return PA_OK;
}

pa_status_t pa_seq_slots(const pa_pool *pool, int64_t seq, int32_t start, int32_t count,
                         int64_t *slots) {
  if (!pool || (count > 0 && !slots)) return fail(PA_EINVAL, "pa_seq_slots: NULL argument");
  Seq *sq;
  if (pa_status_t st = resident(const_cast<pa_pool *>(pool), seq, "pa_seq_slots", &sq)) return st;
  const Seq &s = *sq;
  if (start < 0 || count < 0 || (int64_t)start + count > s.len)
    return fail(PA_ESTATE, "pa_seq_slots: positions [%d, %d) outside length %lld", start,
                start + count, (long long)s.len);
  for (int32_t i = 0; i < count; ++i) {
    int64_t pos = (int64_t)start + i;
    slots[i] = (int64_t)s.table[pos / pool->block_size] * pool->block_size + pos % pool->block_size;
  }
  return PA_OK;
}

pa_status_t pa_seq_table(const pa_pool *pool, int64_t seq, int32_t *row, int32_t max_blocks,
                         int32_t *num_blocks, int32_t *len) {
  if (!pool || !num_blocks || !len) return fail(PA_EINVAL, "pa_seq_table: NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_ESTATE, "pa_seq_table: unknown sequence %lld", (long long)seq);
  const Seq &s = it->second;
  *num_blocks = (int32_t)s.table.size();
  *len = (int32_t)s.len;
  if ((int32_t)s.table.size() > max_blocks || (max_blocks > 0 && !row))
    return fail(PA_EINVAL, "pa_seq_table: %zu blocks do not fit in %d", s.table.size(), max_blocks);
  for (int32_t i = 0; i < max_blocks; ++i) row[i] = i < (int32_t)s.table.size() ? s.table[i] : -1;
  return PA_OK;
}

pa_status_t pa_pool_tables(const pa_pool *pool, const int64_t *seqs, int32_t n, int32_t *tables,
                           int32_t max_blocks, int32_t *context_lens) {
  if (!pool || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables || !context_lens)))
    return fail(PA_EINVAL, "pa_pool_tables: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    Seq *sq;
    if (pa_status_t st = resident(const_cast<pa_pool *>(pool), seqs[i], "pa_pool_tables", &sq)) return st;
    auto it = pool->seqs.find(seqs[i]);
    if ((int32_t)it->second.table.size() > max_blocks)
      return fail(PA_EINVAL, "pa_pool_tables: sequence %lld has %zu blocks > %d", (long long)seqs[i],
                  it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq &s = pool->seqs.find(seqs[i])->second;
    int32_t *row = tables + (int64_t)i * max_blocks;
    int32_t nb = (int32_t)s.table.size();
    if (nb) std::memcpy(row, s.table.data(), sizeof(int32_t) * nb);
    for (int32_t j = nb; j < max_blocks; ++j) row[j] = -1;
    context_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

pa_status_t pa_pool_set_swap_space(pa_pool *pool, int32_t num_host_blocks, const int32_t *host_free_order) {
  if (!pool) return fail(PA_EINVAL, "pa_pool_set_swap_space: pool is NULL");
  if (num_host_blocks < 0)
    return fail(PA_EINVAL, "pa_pool_set_swap_space: num_host_blocks=%d < 0", num_host_blocks);
  if (pool->swapped_seqs > 0)
    return fail(PA_ESTATE, "pa_pool_set_swap_space: %d sequences are swapped out", pool->swapped_seqs);
  std::vector<int32_t> stack(num_host_blocks);
  std::vector<char> seen(num_host_blocks, 0);
  for (int32_t i = 0; i < num_host_blocks; ++i) {
    int32_t h = host_free_order ? host_free_order[i] : i;
    if (h < 0 || h >= num_host_blocks || seen[h])
      return fail(PA_EINVAL, "pa_pool_set_swap_space: host_free_order is not a permutation (entry %d = %d)", i,
                  h);
    seen[h] = 1;
    stack[num_host_blocks - 1 - i] = h;
  }
  pool->num_host_blocks = num_host_blocks;
  pool->host_free.swap(stack);
  return PA_OK;
}

int32_t pa_pool_num_free_host(const pa_pool *pool) { return pool ? (int32_t)pool->host_free.size() : -1; }

pa_status_t pa_pool_host_free_list(const pa_pool *pool, int32_t *out, int32_t cap, int32_t *n) {
  if (!pool || !n) return fail(PA_EINVAL, "pa_pool_host_free_list: NULL argument");
  int32_t total = (int32_t)pool->host_free.size();
  *n = total;
  if (total > cap || (total > 0 && !out))
    return fail(PA_EINVAL, "pa_pool_host_free_list: %d free host blocks do not fit in %d", total, cap);
  for (int32_t i = 0; i < total; ++i) out[i] = pool->host_free[total - 1 - i];
  return PA_OK;
}

int32_t pa_seq_is_swapped(const pa_pool *pool, int64_t seq) {
  if (!pool) return -1;
  auto it = pool->seqs.find(seq);
  return it == pool->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

pa_status_t pa_seq_swap_out(pa_pool *pool, int64_t seq, int64_t *pairs, int32_t cap, int32_t *num_pairs) {
  if (!pool || !num_pairs) return fail(PA_EINVAL, "pa_seq_swap_out: NULL argument");
  *num_pairs = 0;
  Seq *sq;
  if (pa_status_t st = resident(pool, seq, "pa_seq_swap_out", &sq)) return st;
  const int32_t nb = (int32_t)sq->table.size();
  if (nb > cap || (nb > 0 && !pairs))
    return fail(PA_EINVAL, "pa_seq_swap_out: %d pairs do not fit in %d", nb, cap);
  if (nb > (int32_t)pool->host_free.size())
    return fail(PA_ENOMEM, "pa_seq_swap_out: %d host blocks needed, %zu free", nb, pool->host_free.size());
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t b = sq->table[i];
    const int32_t h = pool->host_free.back();
    pool->host_free.pop_back();
    pairs[2 * i] = b;
    pairs[2 * i + 1] = h;
    sq->table[i] = h;
    pool->release(b);
  }
  sq->swapped = true;
  pool->swapped_seqs += 1;
  *num_pairs = nb;
  return PA_OK;
}

pa_status_t pa_seq_swap_in(pa_pool *pool, int64_t seq, int64_t *pairs, int32_t cap, int32_t *num_pairs) {
  if (!pool || !num_pairs) return fail(PA_EINVAL, "pa_seq_swap_in: NULL argument");
  *num_pairs = 0;
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_ESTATE, "pa_seq_swap_in: unknown sequence %lld", (long long)seq);
  Seq &s = it->second;
  if (!s.swapped) return fail(PA_ESTATE, "pa_seq_swap_in: sequence %lld is not swapped out", (long long)seq);
  const int32_t nb = (int32_t)s.table.size();
  if (nb > cap || (nb > 0 && !pairs))
    return fail(PA_EINVAL, "pa_seq_swap_in: %d pairs do not fit in %d", nb, cap);
  if (nb > (int32_t)pool->available())
    return fail(PA_ENOMEM, "pa_seq_swap_in: %d blocks needed, %zu free", nb, pool->available());
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t h = s.table[i];
    const int32_t b = pool->take();
    pairs[2 * i] = h;
    pairs[2 * i + 1] = b;
    s.table[i] = b;
    pool->host_free.push_back(h);
  }
  s.swapped = false;
  pool->swapped_seqs -= 1;
  *num_pairs = nb;
  return PA_OK;
}

pa_status_t pa_pool_enable_prefix_cache(pa_pool *pool) {
  if (!pool) return fail(PA_EINVAL, "pa_pool_enable_prefix_cache: pool is NULL");
  pool->prefix_cache = true;
  return PA_OK;
}

int32_t pa_pool_num_cached(const pa_pool *pool) { return pool ? (int32_t)pool->lru.size() : -1; }

int32_t pa_pool_is_cached(const pa_pool *pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->block_key[block] ? 1 : 0;
}

pa_status_t pa_pool_lru_list(const pa_pool *pool, int32_t *out, int32_t cap, int32_t *n) {
  if (!pool || !n) return fail(PA_EINVAL, "pa_pool_lru_list: NULL argument");
  int32_t total = (int32_t)pool->lru.size();
  *n = total;
  if (total > cap || (total > 0 && !out))
    return fail(PA_EINVAL, "pa_pool_lru_list: %d cached blocks do not fit in %d", total, cap);
  int32_t i = 0;
  for (int32_t b : pool->lru) out[i++] = b;
  return PA_OK;
}

pa_status_t pa_seq_create_cached(pa_pool *pool, int64_t seq, const int32_t *tokens, int32_t num_tokens,
                                 int32_t *num_cached_tokens) {
  if (!pool || !num_cached_tokens || num_tokens < 0 || (num_tokens > 0 && !tokens))
    return fail(PA_EINVAL, "pa_seq_create_cached: bad argument");
  *num_cached_tokens = 0;
  if (!pool->prefix_cache) return fail(PA_ESTATE, "pa_seq_create_cached: prefix caching is not enabled");
  if (pool->seqs.count(seq)) return fail(PA_ESTATE, "pa_seq_create_cached: sequence %lld exists", (long long)seq);
  const int32_t bs = pool->block_size;
  const int32_t need = (int32_t)(((int64_t)num_tokens + bs - 1) / bs);
  const int32_t full = num_tokens / bs;
  // Longest cached run of full blocks.
  std::vector<int32_t> hits;
  int64_t parent = 0;
  int32_t idle_hits = 0;  // hits now in the LRU list: they stop being available
  for (int32_t i = 0; i < full; ++i) {
    const int32_t *tok = tokens + (int64_t)i * bs;
    const pa_pool::CacheEntry *e = pool->find(pa_pool::key_hash(parent, tok, bs), parent, tok, bs);
    if (!e) break;
    hits.push_back(e->block);
    idle_hits += pool->refcount[e->block] == 0;
    parent = e->node;
  }
  const int32_t fresh = need - (int32_t)hits.size();
  if ((size_t)fresh + idle_hits > pool->available())
    return fail(PA_ENOMEM, "pa_seq_create_cached: %d blocks needed, %zu free", fresh,
                pool->available() - idle_hits);
  Seq s;
  s.table.reserve(need);
  for (int32_t b : hits) {
    pool->reuse(b);
    s.table.push_back(b);
  }
  for (int32_t i = (int32_t)hits.size(); i < need; ++i) {
    const int32_t b = pool->take();
    s.table.push_back(b);
    if (i < full) {  // a full block of the prompt: register it
      const int32_t *tok = tokens + (int64_t)i * bs;
      const int64_t node = pool->next_node++;
      const uint64_t h = pa_pool::key_hash(parent, tok, bs);
      auto it = pool->cache.emplace(h, pa_pool::CacheEntry{parent, std::vector<int32_t>(tok, tok + bs), b, node});
      pool->block_key[b] = &it->second;
      pool->block_hash[b] = h;
      parent = node;
    }
  }
  s.len = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  *num_cached_tokens = (int32_t)hits.size() * bs;
  return PA_OK;
}

pa_status_t pa_seq_create_cached_batch(pa_pool *pool, const int64_t *seqs, int32_t n, const int32_t *tokens,
                                       const int64_t *offsets, int32_t *num_cached, int64_t *slots,
                                       int64_t slots_cap, int32_t *num_admitted, int64_t *num_slots) {
  if (!pool || n < 0 || !num_admitted || !num_slots || (n > 0 && (!seqs || !offsets || !num_cached)))
    return fail(PA_EINVAL, "pa_seq_create_cached_batch: bad argument");
  *num_admitted = 0;
  *num_slots = 0;
  if (n == 0) return PA_OK;
  if (offsets[0] != 0) return fail(PA_EINVAL, "pa_seq_create_cached_batch: offsets[0] must be 0");
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = offsets[i + 1] - offsets[i];
    if (len < 0 || len > INT32_MAX)
      return fail(PA_EINVAL, "pa_seq_create_cached_batch: bad length %lld of request %d", (long long)len, i);
  }
  if (offsets[n] > 0 && (!tokens || !slots))
    return fail(PA_EINVAL, "pa_seq_create_cached_batch: tokens or slots is NULL");
  if (slots_cap < offsets[n])
    return fail(PA_EINVAL, "pa_seq_create_cached_batch: slots has room for %lld, the batch has %lld tokens",
                (long long)slots_cap, (long long)offsets[n]);
  // Admit in order; the first request that is refused ends the batch.
  int64_t out = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t len = (int32_t)(offsets[i + 1] - offsets[i]);
    int32_t cached = 0;
    if (pa_status_t st = pa_seq_create_cached(pool, seqs[i], tokens + offsets[i], len, &cached)) {
      *num_slots = out;
      return st;
    }
    const Seq &sq = pool->seqs.find(seqs[i])->second;
    const int32_t bs = pool->block_size;
    for (int64_t pos = cached; pos < len; ++pos) slots[out++] = (int64_t)sq.table[pos / bs] * bs + pos % bs;
    num_cached[i] = cached;
    *num_admitted = i + 1;
  }
  *num_slots = out;
  return PA_OK;
}

}  // extern "C"
