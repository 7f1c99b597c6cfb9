// KV-slot write and whole-block copy for the paged KV pools (gfx950).
//
// foundry "PagedAttention" ops page, "How it works": each decode step stores
// the new token's key and value into the sequence's current block; shared
// blocks are duplicated (copy-on-write) when a sharer writes.  "At a glance":
// a block is copied only when a sequence writes to it.
//
// Same page, "How it works" and "Trade-offs": a preempted sequence's blocks
// can be swapped out to CPU memory and back; pa_swap_blocks copies whole
// blocks between a device pool and a pool in pinned host memory, which the
// kernel reads or writes directly over the bus.
//
// The kernels move bytes only (16 bytes per lane, coalesced) and are bitwise
// exact.  Pool layout: [num_blocks][num_kv_heads][block_size][head_dim].

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa.h"
#include "pa_status.h"

namespace {

constexpr int kThreads = 256;

// One lane moves 16 bytes of one token row of one KV head, for K and V.
// Rows are head_dim * elt bytes, a multiple of 16.
__global__ __launch_bounds__(kThreads) void write_kv_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, const int64_t *__restrict__ slots,
    int64_t num_chunks, int32_t chunks_per_row, int32_t num_kv_heads, int32_t block_size,
    int64_t num_slots, uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache) {
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= num_chunks) return;
  int64_t row = i / chunks_per_row;          // token * num_kv_heads + head
  int32_t c = (int32_t)(i - row * chunks_per_row);
  int64_t tok = row / num_kv_heads;
  int32_t head = (int32_t)(row - tok * num_kv_heads);
  int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;  // padding / out of pool: skipped
  int64_t blk = slot / block_size;
  int64_t off = slot - blk * block_size;
  int64_t dst = ((blk * num_kv_heads + head) * block_size + off) * chunks_per_row + c;
  k_cache[dst] = k[i];
  v_cache[dst] = v[i];
}

// Workgroup w copies part (w % parts) of pair (w / parts); a block's bytes
// are split over `parts` workgroups of kThreads lanes.  Block src of the
// source pools goes to block dst of the destination pools (the same pools
// for copy-on-write); pairs naming a block outside its pool are skipped.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    const uint4 *src_k, const uint4 *src_v, uint4 *dst_k, uint4 *dst_v, const int64_t *__restrict__ pairs,
    int64_t chunks_per_block, int32_t parts, int32_t src_blocks, int32_t dst_blocks) {
  int64_t pair = blockIdx.x / parts;
  int32_t part = (int32_t)(blockIdx.x - pair * parts);
  int64_t src = pairs[2 * pair];
  int64_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4 *ks = src_k + src * chunks_per_block;
  const uint4 *vs = src_v + src * chunks_per_block;
  uint4 *kd = dst_k + dst * chunks_per_block;
  uint4 *vd = dst_v + dst * chunks_per_block;
  for (int64_t i = (int64_t)part * kThreads + threadIdx.x; i < chunks_per_block;
       i += (int64_t)parts * kThreads) {
    uint4 a = ks[i];
    uint4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

// Measurement helper, not a step of the attention path: reads n 16-byte
// chunks with non-temporal loads and writes the XOR of every 32-bit word a
// workgroup read to sink[workgroup], so that no load can be dropped.  Each
// workgroup walks one contiguous run of the buffer, kProbeUnroll full
// workgroup rows (16 KiB per workgroup) in flight per step; measured on
// MI355X over 1 GiB: 7.03 TB/s with 8192 workgroups, against 5.7 TB/s for a
// grid-strided walk with 4 rows in flight (2048 workgroups).  Its rate is
// the practical ceiling of a pure streaming read, the yardstick next to the
// HBM peak.
constexpr int kProbeUnroll = 8;
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4 *__restrict__ buf, int64_t n,
                                                              uint32_t *__restrict__ sink) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t *b = reinterpret_cast<const u32x4_t *>(buf);
  const int64_t step = (int64_t)kThreads * kProbeUnroll;
  const int64_t per = ((n + gridDim.x - 1) / gridDim.x + step - 1) / step * step;  // chunks per workgroup
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = min(n, lo + per);
  uint32_t x = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kThreads < hi; i += step) {
    u32x4_t a[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) a[u] = __builtin_nontemporal_load(b + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) x ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  for (; i < hi; i += kThreads) {
    const u32x4_t t = __builtin_nontemporal_load(b + i);
    x ^= t.x ^ t.y ^ t.z ^ t.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  __shared__ uint32_t wave_x[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t ^= wave_x[w];
    sink[blockIdx.x] = t;
  }
}

hipError_t launch_copy(const void *src_k, const void *src_v, void *dst_k, void *dst_v, const pa_cache_t *geom,
                       int32_t src_blocks, int32_t dst_blocks, const int64_t *pairs, int32_t num_pairs,
                       void *stream);

int elt_bytes(int32_t dtype) { return dtype == PA_BF16 ? 2 : dtype == PA_F32 ? 4 : 0; }

pa_status_t check_cache(const char *who, const pa_cache_t *c) {
  if (!c) return pa::fail(PA_EINVAL, "%s: cache descriptor is NULL", who);
  if (c->num_blocks <= 0 || c->block_size <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return pa::fail(PA_EINVAL, "%s: cache dimensions must be > 0", who);
  if (!elt_bytes(c->dtype)) return pa::fail(PA_EUNSUPPORTED, "%s: dtype %d", who, c->dtype);
  if ((c->head_dim * elt_bytes(c->dtype)) % 16)
    return pa::fail(PA_EUNSUPPORTED, "%s: a row of head_dim %d is not a multiple of 16 bytes", who,
                    c->head_dim);
  return PA_OK;
}

}  // namespace

extern "C" pa_status_t pa_write_kv(const void *k, const void *v, const int64_t *slot_mapping,
                                   int32_t num_tokens, void *k_cache, void *v_cache,
                                   const pa_cache_t *cache, void *stream) {
  if (pa_status_t st = check_cache("pa_write_kv", cache)) return st;
  if (num_tokens < 0) return pa::fail(PA_EINVAL, "pa_write_kv: num_tokens=%d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return pa::fail(PA_EINVAL, "pa_write_kv: NULL pointer");
  int32_t cpr = cache->head_dim * elt_bytes(cache->dtype) / 16;
  int64_t chunks = (int64_t)num_tokens * cache->num_kv_heads * cpr;
  int64_t grid = (chunks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4 *)k, (const uint4 *)v, slot_mapping, chunks, cpr,
                     cache->num_kv_heads, cache->block_size,
                     (int64_t)cache->num_blocks * cache->block_size, (uint4 *)k_cache,
                     (uint4 *)v_cache);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_EHIP, "pa_write_kv: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" pa_status_t pa_copy_blocks(void *k_cache, void *v_cache, const pa_cache_t *cache,
                                      const int64_t *src_dst_pairs, int32_t num_pairs,
                                      void *stream) {
  if (pa_status_t st = check_cache("pa_copy_blocks", cache)) return st;
  if (num_pairs < 0) return pa::fail(PA_EINVAL, "pa_copy_blocks: num_pairs=%d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return pa::fail(PA_EINVAL, "pa_copy_blocks: NULL pointer");
  hipError_t e = launch_copy(k_cache, v_cache, k_cache, v_cache, cache, cache->num_blocks, cache->num_blocks,
                             src_dst_pairs, num_pairs, stream);
  if (e != hipSuccess) return pa::fail(PA_EHIP, "pa_copy_blocks: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" pa_status_t pa_swap_blocks(const void *src_k, const void *src_v, const pa_cache_t *src_cache,
                                      void *dst_k, void *dst_v, const pa_cache_t *dst_cache,
                                      const int64_t *src_dst_pairs, int32_t num_pairs, void *stream) {
  if (pa_status_t st = check_cache("pa_swap_blocks", src_cache)) return st;
  if (pa_status_t st = check_cache("pa_swap_blocks", dst_cache)) return st;
  if (src_cache->block_size != dst_cache->block_size || src_cache->num_kv_heads != dst_cache->num_kv_heads ||
      src_cache->head_dim != dst_cache->head_dim || src_cache->dtype != dst_cache->dtype)
    return pa::fail(PA_EINVAL, "pa_swap_blocks: source and destination blocks differ in shape or dtype");
  if (num_pairs < 0) return pa::fail(PA_EINVAL, "pa_swap_blocks: num_pairs=%d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !src_dst_pairs)
    return pa::fail(PA_EINVAL, "pa_swap_blocks: NULL pointer");
  if (((uintptr_t)src_k | (uintptr_t)src_v | (uintptr_t)dst_k | (uintptr_t)dst_v) % 16)
    return pa::fail(PA_EINVAL, "pa_swap_blocks: pools must be 16-byte aligned");
  hipError_t e = launch_copy(src_k, src_v, dst_k, dst_v, src_cache, src_cache->num_blocks, dst_cache->num_blocks,
                             src_dst_pairs, num_pairs, stream);
  if (e != hipSuccess) return pa::fail(PA_EHIP, "pa_swap_blocks: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

namespace {

hipError_t launch_copy(const void *src_k, const void *src_v, void *dst_k, void *dst_v, const pa_cache_t *geom,
                       int32_t src_blocks, int32_t dst_blocks, const int64_t *pairs, int32_t num_pairs,
                       void *stream) {
  const int64_t block_bytes = (int64_t)geom->num_kv_heads * geom->block_size * geom->head_dim * elt_bytes(geom->dtype);
  const int64_t chunks = block_bytes / 16;
  int64_t parts = (chunks + kThreads - 1) / kThreads;
  if (parts > 64) parts = 64;
  const int64_t grid = parts * num_pairs;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4 *)src_k, (const uint4 *)src_v, (uint4 *)dst_k, (uint4 *)dst_v, pairs, chunks,
                     (int32_t)parts, src_blocks, dst_blocks);
  return hipGetLastError();
}

}  // namespace

extern "C" pa_status_t pa_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  if (bytes % 16) return pa::fail(PA_EINVAL, "pa_read_probe: %zu bytes is not a multiple of 16", bytes);
  if (!sink || (bytes && !buf)) return pa::fail(PA_EINVAL, "pa_read_probe: NULL pointer");
  if ((uintptr_t)buf % 16) return pa::fail(PA_EINVAL, "pa_read_probe: buffer must be 16-byte aligned");
  hipLaunchKernelGGL(read_probe_kernel, dim3(PA_READ_PROBE_WORKGROUPS), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4 *)buf, (int64_t)(bytes / 16), sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_EHIP, "pa_read_probe: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
