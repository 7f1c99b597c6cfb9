// Paged single-query decode attention for gfx950 (MI355X).
//
// foundry "PagedAttention" ops page, "How it works": the attention kernel
// reads KV through the per-sequence block table, gathering scattered
// physical blocks, so the math is the same as over one contiguous run;
// "Concept": blocks hold a fixed number of tokens and live anywhere in the
// pool.  The math is softmax(scale * q K^T) V per (sequence, query head),
// accumulated in fp32 with an online softmax (Milakov & Gimelshein 2018).
//
// Work decomposition
//   One workgroup of 4 wave64s per (sequence, KV head, context partition).
//   The G = Hq / Hkv query heads of a KV head share that workgroup, so each
//   K/V row is read from HBM once.  A K or V row is head_dim elements; a lane
//   owns 16 bytes of it, so LPR = row_bytes / 16 lanes cover a row and one
//   wave-wide load streams RPW = 64 / LPR consecutive rows (1 KiB).  Lane
//   (r, c) = (lane / LPR, lane % LPR) holds channels [c*VEC, c*VEC + VEC) of
//   row r of each load.
//   The block-table slice of the workgroup's tokens is staged in LDS first;
//   each token's row address is then pool + ((blk * Hkv + kvh) * bs + off) * row.
//   QK: per-lane partial dots, summed over the LPR lanes of a row with DPP
//   row permutations (every lane ends with the identical sum).  Softmax runs
//   in the exp2 domain (logits pre-multiplied by log2 e); each row group keeps
//   its own running (max, sum, acc) and the groups / waves are merged at the
//   end (shuffles, then LDS).
//   Partitioned mode writes per-partition (max, sum, unnormalised acc) to the
//   workspace and a second kernel merges them:
//     M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
//
// Masking: tokens at or past the sequence length are never loaded and their
// logits are -inf (selected, not multiplied), so whatever the tail slots of
// the last block hold cannot reach the output.
//
// This vector-ALU kernel serves fp32 pools and bf16 pools with 1 or 2 query
// heads per KV head; bf16 pools with 4 or 8 go to the matrix-core kernel in
// pa_decode_gqa.hip.  Both write the same partition statistics, merged by
// merge_kernel below.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "pa.h"
#include "pa_decode_common.h"
#include "pa_status.h"

namespace {

using pa::DecodeArgs;
using pa::bf16_hi;
using pa::bf16_lo;
using pa::exp2_fast;
using pa::group_sum;
using pa::kLog2e;
using pa::kMaxTableLds;
using pa::kNegBig;
using pa::kThreads;
using pa::kWaves;
using pa::store_out;
using pa::xcd_work_id;

constexpr int kLoadsPerTile = 4;             // 16-byte loads per lane per K (and V) tile

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename E>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kVec = 4;   // elements per 16 bytes
};
template <>
struct Elt<uint16_t> {
  static constexpr int kVec = 8;
};

// Lane-owned query chunk for G heads, in the form the dot product wants.
template <typename E, int G>
struct QChunk;

template <int G>
struct QChunk<float, G> {
  float v[G][4];
  __device__ __forceinline__ void load(const uint4 *q, int stride_heads_chunks, float qscale) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      uint4 w = q[j * stride_heads_chunks];
      v[j][0] = __uint_as_float(w.x) * qscale;
      v[j][1] = __uint_as_float(w.y) * qscale;
      v[j][2] = __uint_as_float(w.z) * qscale;
      v[j][3] = __uint_as_float(w.w) * qscale;
    }
  }
  // Partial dot of head j with one lane chunk of a K row, already scaled.
  __device__ __forceinline__ float dot(int j, uint4 k) const {
    float s = v[j][0] * __uint_as_float(k.x);
    s = fmaf(v[j][1], __uint_as_float(k.y), s);
    s = fmaf(v[j][2], __uint_as_float(k.z), s);
    s = fmaf(v[j][3], __uint_as_float(k.w), s);
    return s;
  }
  static constexpr bool kPostScale = false;
};

template <int G>
struct QChunk<uint16_t, G> {
  uint4 v[G];
  __device__ __forceinline__ void load(const uint4 *q, int stride_heads_chunks, float) {
#pragma unroll
    for (int j = 0; j < G; ++j) v[j] = q[j * stride_heads_chunks];
  }
  // bf16 pairs: v_dot2_f32_bf16 accumulates both products into fp32.
  __device__ __forceinline__ float dot(int j, uint4 k) const {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                              __builtin_bit_cast(bf16x2_t, v[j].x), 0.0f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                        __builtin_bit_cast(bf16x2_t, v[j].y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                        __builtin_bit_cast(bf16x2_t, v[j].z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                        __builtin_bit_cast(bf16x2_t, v[j].w), s, false);
    return s;
  }
  static constexpr bool kPostScale = true;
};

template <typename E>
__device__ __forceinline__ void widen(uint4 w, float (&f)[Elt<E>::kVec]);

template <>
__device__ __forceinline__ void widen<float>(uint4 w, float (&f)[4]) {
  f[0] = __uint_as_float(w.x);
  f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z);
  f[3] = __uint_as_float(w.w);
}

template <>
__device__ __forceinline__ void widen<uint16_t>(uint4 w, float (&f)[8]) {
  f[0] = bf16_lo(w.x);
  f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y);
  f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z);
  f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w);
  f[7] = bf16_hi(w.w);
}

template <typename E, int D, int G, bool PART>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int VEC = Elt<E>::kVec;
  constexpr int LPR = D / VEC;        // lanes per row
  constexpr int RPW = 64 / LPR;       // rows per wave-wide load
  constexpr int U = kLoadsPerTile;
  constexpr int TILE = RPW * U;       // tokens per wave iteration
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row must map onto a wave");

  extern __shared__ int32_t tbl[];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ float red_acc[kWaves][G][D];

  const int n_work = a.num_seqs * a.num_kv_heads * a.num_parts;
  const int w = xcd_work_id(blockIdx.x, n_work);
  // work order: KV head (slowest), partition, sequence (fastest)
  const int s = w % a.num_seqs;
  const int rest = w / a.num_seqs;
  const int p = rest % a.num_parts;
  const int kvh = rest / a.num_parts;

  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_cap ? a.ctx_cap : ctx);
  const int start = p * a.partition_size;
  const int end = min(ctx, start + a.partition_size);
  if (PART && start >= end) return;  // no tokens: the merge never reads this slot

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int bs = a.block_size;
  const int first_blk = start >> a.log2_bs;
  const int nblk = end > start ? ((end - 1) >> a.log2_bs) - first_blk + 1 : 0;

  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks + first_blk;
  for (int i = tid; i < nblk; i += kThreads) {
    int b = trow[i];
    tbl[i] = (unsigned)b < (unsigned)a.num_blocks ? b : 0;  // stay inside the pool
  }

  QChunk<E, G> qc;
  const int h0 = kvh * G;
  qc.load(a.q + ((size_t)s * a.num_q_heads + h0) * LPR + c, LPR, a.qscale);

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegBig;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[j][e] = 0.0f;
  }
  __syncthreads();

  const size_t head_rows = (size_t)kvh * bs;        // row offset of this head in a block
  const size_t block_rows = (size_t)a.num_kv_heads * bs;
  const uint4 *kbase = a.k_cache + c;
  const uint4 *vbase = a.v_cache + c;

  for (int t0 = start + wave * TILE; t0 < end; t0 += kWaves * TILE) {
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * RPW + r;
      if (t < end) {
        const int blk = tbl[(t >> a.log2_bs) - first_blk];
        const size_t row = (size_t)blk * block_rows + head_rows + (t & (bs - 1));
        kr[u] = pa::load_stream(kbase + row * LPR);
        vr[u] = pa::load_stream(vbase + row * LPR);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float z[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = t0 + u * RPW + r < end;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = group_sum<LPR>(qc.dot(j, kr[u]));
        if (QChunk<E, G>::kPostScale) d *= a.qscale;
        z[u][j] = valid ? d : -INFINITY;
      }
    }
    float vf[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) widen<E>(vr[u], vf[u]);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mt = z[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, z[u][j]);
      const float mn = fmaxf(m[j], mt);
      const float alpha = exp2_fast(m[j] - mn);
      m[j] = mn;
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pr = exp2_fast(z[u][j] - mn);
        l[j] += pr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(pr, vf[u][e], acc[j][e]);
      }
    }
  }

  // Merge the RPW row groups of the wave (lanes c, c + LPR, c + 2 LPR, ...).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = __shfl_xor(m[j], off, 64);
      const float lo = __shfl_xor(l[j], off, 64);
      const float mn = fmaxf(m[j], mo);
      const float a1 = exp2_fast(m[j] - mn);
      const float a2 = exp2_fast(mo - mn);
      l[j] = l[j] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = __shfl_xor(acc[j][e], off, 64);
        acc[j][e] = acc[j][e] * a1 + ao * a2;
      }
      m[j] = mn;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) red_acc[wave][j][c * VEC + e] = acc[j][e];
      if (c == 0) {
        red_m[wave][j] = m[j];
        red_l[wave][j] = l[j];
      }
    }
  }
  __syncthreads();

  // Merge the waves: one output element per thread step.
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int j = idx / D;
    const int ch = idx % D;
    float M = red_m[0][j];
#pragma unroll
    for (int wv = 1; wv < kWaves; ++wv) M = fmaxf(M, red_m[wv][j]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const float f = exp2_fast(red_m[wv][j] - M);
      L = fmaf(red_l[wv][j], f, L);
      A = fmaf(red_acc[wv][j][ch], f, A);
    }
    const int h = h0 + j;
    if (PART) {
      const size_t slot = ((size_t)s * a.num_q_heads + h) * a.num_parts + p;
      a.part_o[slot * D + ch] = A;
      if (ch == 0) {
        a.part_m[slot] = M;
        a.part_l[slot] = L;
      }
    } else {
      const float o = L > 0.0f ? A / L : 0.0f;
      store_out<E>(a.out, ((size_t)s * a.num_q_heads + h) * D + ch, o, a.out_f32);
    }
  }
}

// Merge of partition statistics: one workgroup of D threads per (seq, q head).
template <typename E, int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
  const int s = blockIdx.x / a.num_q_heads;
  const int h = blockIdx.x % a.num_q_heads;
  const int ch = threadIdx.x;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_cap ? a.ctx_cap : ctx);
  int np = (ctx + a.partition_size - 1) / a.partition_size;
  np = np > a.num_parts ? a.num_parts : np;
  const size_t base = ((size_t)s * a.num_q_heads + h) * a.num_parts;
  float M = kNegBig;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_m[base + p]);
  float L = 0.0f, A = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float f = exp2_fast(a.part_m[base + p] - M);
    L = fmaf(a.part_l[base + p], f, L);
    A = fmaf(a.part_o[(base + p) * D + ch], f, A);
  }
  const float o = L > 0.0f ? A / L : 0.0f;
  store_out<E>(a.out, ((size_t)s * a.num_q_heads + h) * D + ch, o, a.out_f32);
}

template <typename E, int D, int G>
hipError_t launch(const DecodeArgs &a, bool part, int nblk_lds, hipStream_t st) {
  const int n_work = a.num_seqs * a.num_kv_heads * a.num_parts;
  const size_t lds = (size_t)nblk_lds * sizeof(int32_t);
  if (part)
    hipLaunchKernelGGL((decode_kernel<E, D, G, true>), dim3(n_work), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<E, D, G, false>), dim3(n_work), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_g(int g, const DecodeArgs &a, bool part, int nblk_lds, hipStream_t st) {
  switch (g) {
    case 1: return launch<E, D, 1>(a, part, nblk_lds, st);
    case 2: return launch<E, D, 2>(a, part, nblk_lds, st);
    case 4: return launch<E, D, 4>(a, part, nblk_lds, st);
    case 8: return launch<E, D, 8>(a, part, nblk_lds, st);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_d(int d, int g, const DecodeArgs &a, bool part, int nblk_lds, hipStream_t st) {
  switch (d) {
    case 64: return launch_g<E, 64>(g, a, part, nblk_lds, st);
    case 128: return launch_g<E, 128>(g, a, part, nblk_lds, st);
    case 256: return launch_g<E, 256>(g, a, part, nblk_lds, st);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_merge(int d, const DecodeArgs &a, hipStream_t st) {
  const dim3 grid(a.num_seqs * a.num_q_heads);
  switch (d) {
    case 64: hipLaunchKernelGGL((merge_kernel<E, 64>), grid, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL((merge_kernel<E, 128>), grid, dim3(128), 0, st, a); break;
    case 256: hipLaunchKernelGGL((merge_kernel<E, 256>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WorkspaceLayout {
  size_t m_off, l_off, o_off, hdr_off, total;
};

// Partitioned: m, l [B][Hq][NP] and acc [B][Hq][NP][d], fp32.
WorkspaceLayout partitioned_layout(int64_t b, int64_t hq, int64_t d, int64_t np) {
  WorkspaceLayout w{};
  const size_t ml = align256((size_t)(b * hq * np) * sizeof(float));
  w.m_off = 0;
  w.l_off = ml;
  w.o_off = 2 * ml;
  w.total = 2 * ml + align256((size_t)(b * hq * np * d) * sizeof(float));
  return w;
}

// Balanced: header + [B + 1] prefix sums, then per slot (one per workgroup
// plus one per (sequence, KV head)) m, l [G] and acc [G][d], fp32.
WorkspaceLayout balanced_layout(int64_t b, int64_t hq, int64_t hkv, int64_t d) {
  WorkspaceLayout w{};
  const int64_t g = hq / hkv;
  const int64_t slots = pa::kBalancedMaxWorkgroups + b * hkv;
  w.hdr_off = 0;
  const size_t hdr = align256((size_t)(pa::kBalancedHdrInts + b + 1) * sizeof(int32_t));
  const size_t ml = align256((size_t)(slots * g) * sizeof(float));
  w.m_off = hdr;
  w.l_off = hdr + ml;
  w.o_off = hdr + 2 * ml;
  w.total = hdr + 2 * ml + align256((size_t)(slots * g * d) * sizeof(float));
  return w;
}

int64_t parts_for(int64_t max_ctx, int64_t part) {
  int64_t np = (max_ctx + part - 1) / part;
  return np < 1 ? 1 : np;
}

// Partition size used when the balanced split is asked for but a grouped-
// query batch's prefix sums would not fit (a multiple of every supported
// block size).
constexpr int kValuBalancedFallbackP = 4096;
// Partition size of the vector-ALU kernel (fp32 pools, 1 or 2 query heads
// per KV head) under PA_PARTITION_BALANCED when a context is longer than
// that: the long sequences of a skewed batch are cut into pieces that spread
// over the GPU instead of leaving a tail of lone long workgroups (measured
// on MI355X, 256 MHA sequences of lognormal lengths up to 8192: 873 us per
// call unpartitioned, 820 / 810 / 821 us with 512 / 1024 / 2048-token
// partitions).  Also within one workgroup's table at every block size.
constexpr int kValuBalancedP = 1024;

bool uses_gqa_kernel(int dtype, int group, int head_dim) {
  return dtype == PA_BF16 && pa::gqa_mfma_supported(group, head_dim);
}

}  // namespace

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t max_context_len,
                                            int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_q_heads % num_kv_heads)
    return 0;
  const int64_t mc = max_context_len < 0 ? 0 : max_context_len;
  if (partition_size > 0)
    return partitioned_layout(num_seqs, num_q_heads, head_dim, parts_for(mc, partition_size)).total;
  if (partition_size == PA_PARTITION_BALANCED) {
    // whichever kernel runs: the balanced split, or partitions (the vector-ALU
    // kernel's are the finer, so their layout covers the other fallback's)
    const size_t bal = balanced_layout(num_seqs, num_q_heads, num_kv_heads, head_dim).total;
    const size_t fb = partitioned_layout(num_seqs, num_q_heads, head_dim, parts_for(mc, kValuBalancedP)).total;
    return bal > fb ? bal : fb;
  }
  return 0;
}

namespace {

// New tokens to store before attending (pa_decode_write), or none.
struct NewTokens {
  const void *k, *v;
  const int64_t *slot_mapping;
  int32_t num_tokens;
  void *k_cache, *v_cache;
};

pa_status_t decode_call(const void *q, int32_t num_seqs, int32_t num_q_heads, const void *k_cache,
                        const void *v_cache, const pa_cache_t *cache, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                        float scale, int32_t partition_size, void *workspace, size_t workspace_bytes,
                        void *out, int32_t out_dtype, void *stream, const NewTokens *nt) {
  using pa::fail;
  if (!cache) return fail(PA_EINVAL, "pa_decode: cache descriptor is NULL");
  const pa_cache_t c = *cache;
  if (num_seqs < 0 || num_q_heads <= 0 || c.num_blocks <= 0 || c.num_kv_heads <= 0 ||
      c.block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return fail(PA_EINVAL, "pa_decode: sizes must be positive (num_seqs may be 0)");
  if (c.dtype != PA_F32 && c.dtype != PA_BF16)
    return fail(PA_EUNSUPPORTED, "pa_decode: cache dtype %d", c.dtype);
  if (out_dtype != PA_F32 && out_dtype != c.dtype)
    return fail(PA_EUNSUPPORTED, "pa_decode: out dtype %d (use PA_F32 or the cache dtype)", out_dtype);
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256)
    return fail(PA_EUNSUPPORTED, "pa_decode: head_dim %d (built: 64, 128, 256)", c.head_dim);
  if (c.block_size > 256 || (c.block_size & (c.block_size - 1)))
    return fail(PA_EUNSUPPORTED, "pa_decode: block_size %d (powers of two up to 256)", c.block_size);
  if (num_q_heads % c.num_kv_heads)
    return fail(PA_EINVAL, "pa_decode: %d query heads not a multiple of %d KV heads", num_q_heads,
                c.num_kv_heads);
  const int g = num_q_heads / c.num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PA_EUNSUPPORTED, "pa_decode: query heads per KV head = %d (built: 1, 2, 4, 8)", g);
  if (partition_size != PA_PARTITION_BALANCED && (partition_size < 0 || (partition_size % c.block_size)))
    return fail(PA_EINVAL,
                "pa_decode: partition_size %d must be 0, PA_PARTITION_BALANCED or a multiple of "
                "block_size %d",
                partition_size, c.block_size);
  if (num_seqs == 0)  // nothing to attend; new tokens are still stored
    return nt ? pa_write_kv(nt->k, nt->v, nt->slot_mapping, nt->num_tokens, nt->k_cache, nt->v_cache,
                            cache, stream)
              : PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PA_EINVAL, "pa_decode: NULL pointer");
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16)
    return fail(PA_EINVAL, "pa_decode: q and the pools must be 16-byte aligned");

  int log2_bs = 0;
  while ((1 << log2_bs) < c.block_size) ++log2_bs;
  const int64_t cap64 = (int64_t)max_blocks_per_seq * c.block_size;
  const int32_t ctx_cap = (int32_t)(cap64 < max_context_len ? cap64 : max_context_len);
  const int64_t ctx_blocks = ((int64_t)ctx_cap + c.block_size - 1) / c.block_size;
  const bool gqa = uses_gqa_kernel(c.dtype, g, c.head_dim);

  DecodeArgs a{};
  a.q = (const uint4 *)q;
  a.k_cache = (const uint4 *)k_cache;
  a.v_cache = (const uint4 *)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c.num_kv_heads;
  a.block_size = c.block_size;
  a.log2_bs = log2_bs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = c.num_blocks;
  a.ctx_cap = ctx_cap;
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  a.qscale = scale * kLog2e;

  // How the contexts are cut into workgroup ranges.
  int mode = pa::kModeUnpartitioned;
  int32_t part = 0;
  if (partition_size > 0) {
    mode = pa::kModePartitioned;
    part = partition_size;
  } else if (partition_size == PA_PARTITION_BALANCED) {
    // the balanced split keeps the sequences' prefix sums (padded lengths
    // plus a per-sequence cost of at most 256 positions) in int32 and in LDS
    const bool fits = num_seqs <= pa::kBalancedMaxSeqs &&
                      (int64_t)num_seqs * ((((int64_t)ctx_cap + 15) & ~(int64_t)15) + 256) <= 0x7fffffff;
    if (gqa && fits) {
      mode = pa::kModeBalanced;
    } else if (gqa && ctx_cap > kValuBalancedFallbackP) {
      mode = pa::kModePartitioned;
      part = kValuBalancedFallbackP;
    } else if (!gqa && ctx_cap > kValuBalancedP) {
      mode = pa::kModePartitioned;
      part = kValuBalancedP;
    }
  }
  if (!gqa && mode == pa::kModePartitioned && part / c.block_size > kMaxTableLds)
    return fail(PA_EUNSUPPORTED, "pa_decode: partition of %d blocks exceeds %d for this head configuration",
                part / c.block_size, kMaxTableLds);
  if (!gqa && mode == pa::kModeUnpartitioned && ctx_blocks > kMaxTableLds)
    return fail(PA_EUNSUPPORTED,
                "pa_decode: %lld blocks per sequence exceed %d for this head configuration; use a "
                "partition_size",
                (long long)ctx_blocks, kMaxTableLds);

  const int64_t tbl_need = ctx_blocks < 1 ? 1 : ctx_blocks;
  int nblk_lds = 0;  // vector-ALU kernel: table entries per workgroup
  if (mode == pa::kModePartitioned) {
    const int64_t np = parts_for(ctx_cap, part);
    const WorkspaceLayout wl = partitioned_layout(num_seqs, num_q_heads, c.head_dim, np);
    if (!workspace || workspace_bytes < wl.total)
      return fail(PA_EINVAL, "pa_decode: workspace of %zu bytes < %zu needed", workspace_bytes,
                  wl.total);
    a.partition_size = part;
    a.num_parts = (int32_t)np;
    a.part_m = (float *)((char *)workspace + wl.m_off);
    a.part_l = (float *)((char *)workspace + wl.l_off);
    a.part_o = (float *)((char *)workspace + wl.o_off);
    nblk_lds = part / c.block_size;
    const int64_t per_part = part / c.block_size;
    a.tbl_cap = (int32_t)(per_part < kMaxTableLds ? per_part : kMaxTableLds);
  } else if (mode == pa::kModeBalanced) {
    const WorkspaceLayout wl = balanced_layout(num_seqs, num_q_heads, c.num_kv_heads, c.head_dim);
    if (!workspace || workspace_bytes < wl.total)
      return fail(PA_EINVAL, "pa_decode: workspace of %zu bytes < %zu needed", workspace_bytes,
                  wl.total);
    a.partition_size = ctx_cap > 0 ? ctx_cap : 1;
    a.num_parts = 1;
    a.bal_hdr = (int32_t *)((char *)workspace + wl.hdr_off);
    a.part_m = (float *)((char *)workspace + wl.m_off);
    a.part_l = (float *)((char *)workspace + wl.l_off);
    a.part_o = (float *)((char *)workspace + wl.o_off);
    a.tbl_cap = (int32_t)(tbl_need < kMaxTableLds ? tbl_need : kMaxTableLds);
  } else {
    a.partition_size = ctx_cap > 0 ? ctx_cap : 1;
    a.num_parts = 1;
    nblk_lds = (int)ctx_blocks;
    a.tbl_cap = (int32_t)(tbl_need < kMaxTableLds ? tbl_need : kMaxTableLds);
  }
  if (workspace && (uintptr_t)workspace % 256)
    return fail(PA_EINVAL, "pa_decode: workspace must be 256-byte aligned");
  const int64_t n_work = (int64_t)num_seqs * c.num_kv_heads * a.num_parts;
  if (n_work > 0x7fffffff)
    return fail(PA_EINVAL, "pa_decode: grid of %lld workgroups too large", (long long)n_work);

  // New tokens: stored by the balanced kernel itself when there is one per
  // sequence, else by pa_write_kv before the attention.
  if (nt) {
    if (mode == pa::kModeBalanced && nt->num_tokens == num_seqs) {
      if (((uintptr_t)nt->k | (uintptr_t)nt->v) % 16)
        return fail(PA_EINVAL, "pa_decode_write: k and v must be 16-byte aligned");
      a.k_new = (const uint4 *)nt->k;
      a.v_new = (const uint4 *)nt->v;
      a.slot_mapping = nt->slot_mapping;
      a.num_slots = (int64_t)c.num_blocks * c.block_size;
    } else if (pa_status_t ws = pa_write_kv(nt->k, nt->v, nt->slot_mapping, nt->num_tokens, nt->k_cache,
                                            nt->v_cache, cache, stream)) {
      return ws;
    }
  }

  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (gqa)
    e = pa::launch_decode_gqa(c.head_dim, g, a, mode, st);
  else if (c.dtype == PA_BF16)
    e = launch_d<uint16_t>(c.head_dim, g, a, mode == pa::kModePartitioned, nblk_lds, st);
  else
    e = launch_d<float>(c.head_dim, g, a, mode == pa::kModePartitioned, nblk_lds, st);
  if (e == hipSuccess && mode == pa::kModePartitioned)
    e = c.dtype == PA_BF16 ? launch_merge<uint16_t>(c.head_dim, a, st) : launch_merge<float>(c.head_dim, a, st);
  if (e != hipSuccess) return fail(PA_EHIP, "pa_decode: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" pa_status_t pa_decode(const void *q, int32_t num_seqs, int32_t num_q_heads,
                                 const void *k_cache, const void *v_cache, const pa_cache_t *cache,
                                 const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *context_lens, int32_t max_context_len, float scale,
                                 int32_t partition_size, void *workspace, size_t workspace_bytes,
                                 void *out, int32_t out_dtype, void *stream) {
  return decode_call(q, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, scale, partition_size, workspace, workspace_bytes, out,
                     out_dtype, stream, nullptr);
}

extern "C" pa_status_t pa_decode_write(const void *k, const void *v, const int64_t *slot_mapping,
                                       int32_t num_tokens, const void *q, int32_t num_seqs,
                                       int32_t num_q_heads, void *k_cache, void *v_cache,
                                       const pa_cache_t *cache, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *context_lens,
                                       int32_t max_context_len, float scale, int32_t partition_size,
                                       void *workspace, size_t workspace_bytes, void *out,
                                       int32_t out_dtype, void *stream) {
  if (num_tokens < 0) return pa::fail(PA_EINVAL, "pa_decode_write: num_tokens=%d < 0", num_tokens);
  if (num_tokens > 0 && (!k || !v || !slot_mapping))
    return pa::fail(PA_EINVAL, "pa_decode_write: NULL pointer");
  const NewTokens nt{k, v, slot_mapping, num_tokens, k_cache, v_cache};
  return decode_call(q, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, scale, partition_size, workspace, workspace_bytes, out,
                     out_dtype, stream, num_tokens > 0 ? &nt : nullptr);
}

// Scratch of pa_decode_write_noalloc: a static array in the code object, one
// copy per GPU, so that entry point allocates nothing.  Host code never uses
// the name itself as an address (on the host it is only a stand-in): each
// device's address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];

// Address of the current device's scratch array, or NULL (status in *err).
void *scratch_address(pa_status_t *err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = pa::fail(PA_EHIP, "pa_decode_write_noalloc: no usable current device (%d)", dev);
    return nullptr;
  }
  void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    *err = pa::fail(PA_EHIP, "pa_decode_write_noalloc: scratch address on device %d: %s", dev,
                    hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_addr[dev].store(p, std::memory_order_release);  // same value if two threads race here
  return p;
}

}  // namespace

extern "C" pa_status_t pa_decode_write_noalloc(const void *k, const void *v, const int64_t *slot_mapping,
                                               int32_t num_tokens, const void *q, int32_t num_seqs,
                                               int32_t num_q_heads, void *k_cache, void *v_cache,
                                               const pa_cache_t *cache, const int32_t *block_tables,
                                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                                               int32_t max_context_len, float scale, int32_t partition_size,
                                               void *out, int32_t out_dtype, void *stream) {
  if (!cache) return pa::fail(PA_EINVAL, "pa_decode_write_noalloc: cache descriptor is NULL");
  if (partition_size != 0 && num_seqs > 0) {
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                                  max_context_len, partition_size);
    if (need > PA_NOALLOC_SCRATCH_BYTES)
      return pa::fail(PA_EINVAL,
                      "pa_decode_write_noalloc: this call needs %zu bytes of scratch, more than the %zu of "
                      "the library's static array (use pa_decode_write with a workspace)",
                      need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  }
  void *ws = nullptr;
  size_t ws_bytes = 0;
  if (partition_size != 0 && num_seqs > 0) {
    pa_status_t err = PA_OK;
    ws = scratch_address(&err);
    if (!ws) return err;
    ws_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  return pa_decode_write(k, v, slot_mapping, num_tokens, q, num_seqs, num_q_heads, k_cache, v_cache, cache,
                         block_tables, max_blocks_per_seq, context_lens, max_context_len, scale, partition_size,
                         ws, ws_bytes, out, out_dtype, stream);
}
