// KV-cache memory waste of a serving loop: contiguous per-request slabs
// against paged blocks, over one pool of KV token slots.
//
// Pages: foundry "PagedAttention" ops page, Concept (a slab per request sized
// to its maximum length strands what the request never fills; paging hands
// out one block at a time, so at most one partly filled block per sequence
// is wasted, and freed blocks return to a shared pool) and At a glance
// (slabs strand memory inside, in unfilled reserved slots, and outside, in
// gaps too small to reuse); aiacademy "Paged Attention" lesson (the slab is
// sized for the longest output the request might produce; a block is taken
// only when decode fills the last one; all blocks are freed on completion).
//
// The loop, step by step: admit requests first come first served while the
// head of the queue fits (a slab takes the lowest-addressed free gap that
// holds it; a paged request takes ceil(p / bs) blocks from this library's
// block manager); record the memory map; store one new token for every
// running request (paged: a request that needs a block when none is free
// preempts the most recently admitted running request, which loses its
// progress and goes back to the front of the queue); retire finished
// requests.

#include <cstdint>
#include <deque>
#include <iterator>
#include <map>
#include <vector>

#include "pa.h"
#include "pa_status.h"

using pa::fail;

namespace {

// First-fit allocator over [0, capacity): free gaps by start address.
struct SlabSpace {
  std::map<int64_t, int64_t> gaps;  // start -> length
  int64_t free_total = 0;

  explicit SlabSpace(int64_t capacity) : free_total(capacity) {
    if (capacity > 0) gaps.emplace(0, capacity);
  }
  // Start of a slab of r slots in the lowest-addressed gap that holds it, or -1.
  int64_t take(int64_t r) {
    for (auto it = gaps.begin(); it != gaps.end(); ++it) {
      if (it->second < r) continue;
      const int64_t start = it->first, rest = it->second - r;
      gaps.erase(it);
      if (rest) gaps.emplace(start + r, rest);
      free_total -= r;
      return start;
    }
    return -1;
  }
  // Return [start, start + r), merged with the free gaps on either side.
  void give(int64_t start, int64_t r) {
    free_total += r;
    int64_t len = r;
    auto next = gaps.lower_bound(start);
    if (next != gaps.end() && next->first == start + len) {
      len += next->second;
      next = gaps.erase(next);
    }
    if (next != gaps.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second == start) {
        prev->second += len;
        return;
      }
    }
    gaps.emplace(start, len);
  }
};

struct PoolGuard {
  pa_pool *p = nullptr;
  ~PoolGuard() { pa_pool_destroy(p); }
};

}  // namespace

extern "C" {

pa_status_t pa_waste_simulate(int32_t mode, int64_t capacity, int32_t block_size, const int32_t *prompt_lens,
                              const int32_t *output_lens, const int32_t *reserve_lens, int32_t num_requests,
                              pa_waste_stats *out) {
  if (!out || num_requests < 0 || (num_requests > 0 && (!prompt_lens || !output_lens || !reserve_lens)))
    return fail(PA_EINVAL, "pa_waste_simulate: NULL argument or negative request count");
  if (mode != PA_WASTE_CONTIGUOUS && mode != PA_WASTE_PAGED)
    return fail(PA_EINVAL, "pa_waste_simulate: unknown mode %d", mode);
  if (block_size < 1 || capacity < 0) return fail(PA_EINVAL, "pa_waste_simulate: bad block size or capacity");
  const bool paged = mode == PA_WASTE_PAGED;
  const int64_t num_blocks = capacity / block_size;
  if (paged && num_blocks > INT32_MAX) return fail(PA_EINVAL, "pa_waste_simulate: %lld blocks", (long long)num_blocks);
  for (int32_t i = 0; i < num_requests; ++i) {
    const int64_t p = prompt_lens[i], o = output_lens[i], r = reserve_lens[i];
    if (p < 1 || o < 1 || r < p + o)
      return fail(PA_EINVAL, "pa_waste_simulate: request %d needs p >= 1, o >= 1, r >= p + o", i);
    if (!paged && r > capacity)
      return fail(PA_EINVAL, "pa_waste_simulate: request %d: slab of %lld exceeds the pool", i, (long long)r);
    if (paged && (p + o + block_size - 1) / block_size > num_blocks)
      return fail(PA_EINVAL, "pa_waste_simulate: request %d: %lld tokens exceed the pool", i, (long long)(p + o));
  }

  pa_waste_stats st = {};
  std::deque<int32_t> waiting;
  for (int32_t i = 0; i < num_requests; ++i) waiting.push_back(i);
  std::vector<int32_t> running;          // admission order
  std::vector<int64_t> len(num_requests, 0), slab(num_requests, -1);
  SlabSpace space(paged ? 0 : capacity);
  PoolGuard pool;
  if (paged && num_requests > 0) {  // validation above leaves at least one block
    if (pa_status_t s = pa_pool_create((int32_t)num_blocks, block_size, nullptr, &pool.p)) return s;
  }

  while (!waiting.empty() || !running.empty()) {
    // admission, first come first served
    while (!waiting.empty()) {
      const int32_t i = waiting.front();
      if (!paged) {
        const int64_t start = space.take(reserve_lens[i]);
        if (start < 0) {
          if (space.free_total >= reserve_lens[i]) st.frag_blocked_steps += 1;
          break;
        }
        slab[i] = start;
      } else {
        const pa_status_t s = pa_seq_create(pool.p, i, prompt_lens[i]);
        if (s == PA_ENOMEM) break;
        if (s) return s;
      }
      waiting.pop_front();
      running.push_back(i);
      len[i] = prompt_lens[i];
    }

    // the step's memory map
    st.steps += 1;
    st.running_steps += (int64_t)running.size();
    if ((int64_t)running.size() > st.max_running) st.max_running = (int64_t)running.size();
    for (int32_t i : running) {
      st.live_slot_steps += len[i];
      st.held_slot_steps += paged ? (len[i] + block_size - 1) / block_size * block_size : reserve_lens[i];
    }

    // one new token per running request
    for (size_t k = 0; k < running.size();) {
      const int32_t i = running[k];
      if (paged) {
        bool self_preempted = false;
        for (;;) {
          int64_t slot, pair[2];
          const pa_status_t s = pa_seq_append(pool.p, i, &slot, pair);
          if (s == PA_OK) break;
          if (s != PA_ENOMEM) return s;
          const int32_t victim = running.back();  // most recently admitted
          running.pop_back();
          if (pa_status_t e = pa_seq_free(pool.p, victim)) return e;
          len[victim] = 0;
          waiting.push_front(victim);
          st.preemptions += 1;
          if (victim == i) {
            self_preempted = true;
            break;
          }
        }
        if (self_preempted) continue;  // k == running.size() now
      }
      len[i] += 1;
      st.decode_tokens += 1;
      ++k;
    }

    // finished requests leave
    size_t kept = 0;
    for (size_t k = 0; k < running.size(); ++k) {
      const int32_t i = running[k];
      if (len[i] == (int64_t)prompt_lens[i] + output_lens[i]) {
        if (paged) {
          if (pa_status_t s = pa_seq_free(pool.p, i)) return s;
        } else {
          space.give(slab[i], reserve_lens[i]);
        }
        len[i] = 0;
      } else {
        running[kept++] = i;
      }
    }
    running.resize(kept);
  }
  *out = st;
  return PA_OK;
}

}  // extern "C"
