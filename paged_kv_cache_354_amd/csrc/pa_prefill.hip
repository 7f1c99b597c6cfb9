// pa_prefill: causal attention of a chunk of new queries per sequence (a
// prompt, or its next piece) over the keys and values read through the
// block table, on gfx950.
//
// (foundry PagedAttention page, Concept and How it works: every token's key
// and value sit in the blocks the sequence's table names, and attention reads
// them through the table; a prompt is many tokens at once.  The attention is
// the textbook causal softmax: the query at position p sees keys 0..p.)
//
// One workgroup (4 wave64s) takes 32 query tokens of GW = min(G, 4) query
// heads of one KV head (for G < 4, 4 / G blocks of 32 tokens), so that the
// key/value tiles it stages in LDS serve 128 (token, head) rows.  A wave
// owns 32 rows of one head, as two blocks of 16, and every K or V^T operand
// it reads from LDS feeds both blocks.  Per tile of 32 keys each block
// computes, on the matrix cores (v_mfma_f32_16x16x32_bf16):
//
//   S^T = K Q^T       keys in M, the block's 16 query rows in N, channels in
//                     K.  Lane (g, n) ends up with the scores of row n for
//                     keys 4g..4g+3 of each 16-key half.
//   O^T += V^T P^T    channels in M (16 per block), rows in N, the 32 keys in
//                     K.  The lane's 8 probabilities (keys 4g..4g+3 and
//                     16+4g..16+4g+3, its own S^T entries rounded to bf16)
//                     are exactly its B operand, so no value crosses lanes.
//                     V stays in LDS as key rows; the A operand (V^T) comes
//                     from two transposing LDS reads (ds_read_b64_tr_b16):
//                     in each 16-lane group, lane i names 4 channels of one
//                     key row and lane 4a + e receives channel e of the rows
//                     named by lanes a, a + 4, a + 8, a + 12, so lane n gets
//                     channel n of 4 key rows.
//
// Every O^T value a lane holds belongs to its own row n, so the online
// softmax rescale is lane-local; only the row max and the final row sum are
// combined over the 4 lanes that share a row (lanes n, n+16, n+32, n+48).
// The probabilities enter the PV product in bf16 (the usual flash-attention
// trade: relative error up to 2^-9 per weight), the rest is fp32.
//
// Two kernels share that tile math and differ in how the key/value tiles
// reach LDS.  prefill_ring_kernel (head_dim 128, blocks of 8 tokens or more)
// loads them straight from HBM into a ring of three LDS slots, two tiles
// ahead; prefill_kernel (the other shapes) loads the next tile into
// registers during the current tile's math and stores it to LDS after.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "pa.h"
#include "pa_decode_common.h"
#include "pa_status.h"

namespace {

using pa::exp2_fast;
using pa::kLog2e;
using pa::kNegBig;
using pa::to_bf16;
using pa::wave_incl_scan;
using pa::xcd_work_id;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;  // 4 wave64s
constexpr int kKeys = 32;      // keys per tile
constexpr int kRB = 2;         // 16-row blocks per wave
constexpr int kTblLds = 2048;  // block ids of a workgroup's keys staged in LDS (else read from HBM)
constexpr int kRankSeqs = 32; // batches up to this many sequences run longest first
constexpr int kCompactSeqs = 64;  // and up to this many get a grid of only the query blocks that exist
constexpr int kTailSeqs = 8;   // at most this many shortest ones merged by key count
constexpr float kLazyW = 256.0f;  // headroom of the running max: weights up to 2^8 (8 in log2 units)
// s_waitcnt operand: vmcnt(0) (expcnt and lgkmcnt at their maxima: no wait)
constexpr int kWaitVmem = 0x0F70;

struct PrefillArgs {
  const uint4 *q;               // [T][Hq][D]
  const uint4 *k_cache;         // [NB][Hkv][bs][D]
  const uint4 *v_cache;
  const int32_t *block_tables;  // [B][max_blocks]
  const int32_t *context_lens;  // [B]
  const int32_t *cu_seqlens;    // [B + 1]
  void *out;                    // [T][Hq][D]
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t log2_bs;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t ctx_cap;   // lengths are clamped to this
  int32_t q_blocks;  // query blocks (of the workgroup's tokens) per sequence, at most
  int32_t q_items;   // grid slots per (KV head, head group): one per query block
  int32_t tail_keys; // ranked batches: context tokens the merged tail may hold per KV head
  int32_t out_f32;   // 1: fp32 output, 0: bf16
  float qscale;      // scale * log2(e)
  // Fused store (pa_prefill_write; k_new NULL otherwise): query row r's key
  // and value rows, [T][Hkv][D], go to pool slot slot_mapping[r], and the
  // attention reads the chunk's keys from these rows.
  const uint4 *k_new;
  const uint4 *v_new;
  const int64_t *slot_mapping;
  int64_t num_slots;  // num_blocks * block_size
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8_t;

template <int D>
struct PrefillShared {
  uint4 k[2][kKeys][D / 8 + 1];        // K rows of the tile (double buffer), 16 B of padding per row
  uint4 v[2][kKeys][D / 8 + 2];        // V rows of the tile, 32 B of padding per row: the 4 rows a
                                       // transposing read spans start in different bank groups
  int32_t tbl[kTblLds];                // block ids of keys [0, kend)
};


// Which (sequence, query block, head group, KV head) workgroup blockIdx.x
// serves, and the sequence's query offset, query count and context length.
//
// Work order: query block (last first: causal blocks near the end see the
// most keys), sequence (longest context first), head group, KV head;
// contiguous ranges per XCD.  With the KV head slowest, XCD x takes the
// same KV head(s) of every sequence: the XCDs get equal shares however
// unequal the sequences are, and an XCD's L2 holds the keys and values of
// its own heads only.  Longest first within an XCD keeps a long
// sequence's workgroups from starting last and running alone at the end.
// In a batch of 2 to kCompactSeqs sequences the grid holds only the query
// blocks that exist: a sequence of n rows has ceil(n / TQ) of them, so the
// grid is sized from the token count instead of every sequence taking as
// many as the longest (measured on MI355X, 8 prompts of U{512..4096}: 8,192
// workgroups of which 3,392 had no rows, each still dispatched and staging
// the lengths before it exited).  Wave 0 finds the sequence of query slot
// `item` from the block counts in rank order (index order past kRankSeqs
// sequences: ranking 64 prefix-cached suffixes cost more than it gained).
// The shortest contexts, up to kTailSeqs of them whose keys and values fit
// half an XCD's L2 per KV head, are merged: their query blocks are taken by
// key count, most first, so the costliest blocks of the last sequences do
// not start after the cheap ones of the sequences before them (measured on
// MI355X, 8 prompts of U{512..4096}: 1.8% faster per call; merging all of
// them, 9% slower: one XCD's L2 no longer holds the keys in use).
struct WorkItem {
  int s, lo, n, ctx;  // sequence, its first query row, its query rows, its context length
  int qb, hg, kvh;    // query block, head group, KV head
};

template <int HG, int TQ>
__device__ __forceinline__ WorkItem find_work(const PrefillArgs &a, int32_t *scratch) {
  WorkItem w;
  const int n_work = a.q_items * a.num_kv_heads * HG;
  int r = xcd_work_id(blockIdx.x, n_work);
  const int item = r % a.q_items;
  r /= a.q_items;
  w.hg = r % HG;
  w.kvh = r / HG;
  w.qb = a.q_blocks - 1 - item % a.q_blocks;
  const int rank = item / a.q_blocks;
  if (a.num_seqs > 1 && a.num_seqs <= kCompactSeqs) {
    // Ranks: by context length, longest first, ties by index (a
    // permutation, so exactly one sequence has each), or the index itself
    // past kRankSeqs sequences.  The lengths and the query offsets are
    // staged together, so this costs no extra round trip; the scratch is
    // LDS the caller reuses afterwards.
    __shared__ int chosen, chosen_qb;
    __shared__ int by_rank[kCompactSeqs], blocks_by_rank[kCompactSeqs];
    __shared__ int first_by_rank[kCompactSeqs], rows_by_rank[kCompactSeqs];
    int32_t *len = scratch;
    int32_t *cu = scratch + kCompactSeqs;
    for (int i = threadIdx.x; i <= a.num_seqs; i += kThreads) {
      cu[i] = a.cu_seqlens[i];
      if (i < a.num_seqs) {
        const int c = a.context_lens[i];
        len[i] = c < 0 ? 0 : (c > a.ctx_cap ? a.ctx_cap : c);
      }
    }
    __syncthreads();
    const bool ranked = a.num_seqs <= kRankSeqs;
    for (int t = threadIdx.x; t < a.num_seqs; t += kThreads) {
      const int lt = len[t];
      int rk = ranked ? 0 : t;
      if (ranked)
        for (int j = 0; j < a.num_seqs; ++j) {
          const int lj = len[j];
          rk += lj > lt || (lj == lt && j < t);
        }
      const int rows = cu[t + 1] - cu[t];
      by_rank[rk] = t;
      blocks_by_rank[rk] = min((rows + TQ - 1) / TQ, a.q_blocks);
      first_by_rank[rk] = lt - rows;
      rows_by_rank[rk] = rows;
    }
    __syncthreads();
    if (threadIdx.x < 64) {  // the sequence and query block of slot `item`
      const int lane = threadIdx.x;
      const int B = a.num_seqs;
      const int nb = lane < B ? blocks_by_rank[lane] : 0;
      const int upto = wave_incl_scan(nb);
      const int total = __builtin_amdgcn_readlane(upto, B - 1);
      // The tail: the last ranks, at most kTailSeqs, whose contexts sum to
      // at most tail_keys (lane l adds the context of rank B - 1 - l).
      const int back = lane < B ? len[by_rank[B - 1 - lane]] : 0;
      const int upto_back = wave_incl_scan(back);
      int k = __popcll(__ballot(lane < B && lane < kTailSeqs && upto_back <= a.tail_keys));
      if (k < 2 || !ranked) k = 0;
      const int t0 = k == 0 ? total : (k == B ? 0 : __builtin_amdgcn_readlane(upto, B - 1 - k));
      if (lane == 0) {
        chosen = -1;  // a slot past the last block
        chosen_qb = 0;
      }
      if (item < t0) {  // rank by rank, each one's blocks last first
        const uint64_t at = __ballot(item >= upto - nb && item < upto);
        const int rk = at ? __builtin_ctzll(at) : -1;
        if (lane == 0 && rk >= 0) {
          chosen = by_rank[rk];
          chosen_qb = __builtin_amdgcn_readlane(upto, rk) - 1 - item;
        }
      } else if (item < total) {
        // The tail's blocks merged by key count, most first (ties by rank):
        // a block's place is the number of blocks before it, counted per
        // rank in closed form since a rank's keys grow with its block.
        // Exactly one (rank, block) has place `item - t0`.
        const int j = item - t0;
        const int f = lane < B ? first_by_rank[lane] : 0;
        const int nr = lane < B ? rows_by_rank[lane] : 0;
        for (int r1 = B - k; r1 < B; ++r1) {
          const int nb1 = __builtin_amdgcn_readlane(nb, r1);
          const int f1 = __builtin_amdgcn_readlane(f, r1);
          const int n1 = __builtin_amdgcn_readlane(nr, r1);
          for (int qb = lane; qb < nb1; qb += 64) {
            const int key = f1 + min((qb + 1) * TQ, n1);
            int place = nb1 - 1 - qb;
            for (int r2 = B - k; r2 < B; ++r2) {
              if (r2 == r1) continue;
              const int nb2 = __builtin_amdgcn_readlane(nb, r2);
              const int f2 = __builtin_amdgcn_readlane(f, r2);
              const int n2 = __builtin_amdgcn_readlane(nr, r2);
              // blocks of r2 with key above `key`, or equal to it when r2 < r1
              const int below = key - (r2 > r1 ? 0 : 1);  // their keys <= below come after
              const int d = below - f2;
              const int after = below >= f2 + n2 ? nb2 : (d < TQ ? 0 : min(d / TQ, nb2));
              place += nb2 - after;
            }
            if (place == j) {
              chosen = by_rank[r1];
              chosen_qb = qb;
            }
          }
        }
      }
    }
    __syncthreads();
    const int cs = __builtin_amdgcn_readfirstlane(chosen);
    if (cs < 0) {
      w.s = 0;
      w.lo = 0;
      w.n = 0;  // nothing to do: the caller returns
      w.ctx = 0;
      w.qb = 0;
      __syncthreads();
      return w;
    }
    w.s = cs;
    w.qb = __builtin_amdgcn_readfirstlane(chosen_qb);
    w.lo = __builtin_amdgcn_readfirstlane(cu[w.s]);
    w.n = __builtin_amdgcn_readfirstlane(cu[w.s + 1]) - w.lo;
    w.ctx = __builtin_amdgcn_readfirstlane(len[w.s]);
    __syncthreads();  // every thread has read the scratch before it is overwritten
  } else {
    w.s = rank;
    w.lo = a.cu_seqlens[w.s];
    w.n = a.cu_seqlens[w.s + 1] - w.lo;
    const int c = a.context_lens[w.s];
    w.ctx = c < 0 ? 0 : (c > a.ctx_cap ? a.ctx_cap : c);
  }
  return w;
}

// One tile of 32 keys for the wave's 2 x 16 rows: scores, online softmax,
// and the product with V, on the matrix cores.  kop_at(hh, i) returns the A
// operand of S^T for keys 16hh.. (channels [8(4i + g), +8) of key row
// 16hh + nl); vop_at(j) returns the V^T operand of channel block j (see the
// file comment).  row0 is the position of the wave's first row; prow[rb]
// the position of this lane's row of block rb (-1 for no row).  The V^T
// operands of the first VEARLY channel blocks are read before the softmax.
template <int D, int VEARLY, typename KOp, typename VOp>
__device__ __forceinline__ void attend_tile(KOp kop_at, VOp vop_at, const uint4 (&qop)[kRB][D / 32],
                                            f32x4_t (&o)[kRB][D / 16], float (&m)[kRB], float (&l)[kRB],
                                            const int (&prow)[kRB], int kt0, int row0, int g, float qscale,
                                            int xor16, int xor32) {
  constexpr int KSTEPS = D / 32;
  constexpr int OB = D / 16;
  __builtin_amdgcn_s_setprio(0);
  // The scheduler's interleaving of matrix ops with LDS reads (strategy 1)
  // for this region (measured on MI355X, alternating passes: with it here
  // and in the P V^T region, whole prompts 416.2 -> 408.7 us per fused
  // call, chunks 605.4 -> 595.8 us; here only, a further 0.4-0.5%; in the
  // P V^T region only, slower; strategy 0 about half the gain, 2 and 3
  // slower).
  __builtin_amdgcn_iglp_opt(1);
  // S^T for the two 16-key halves of both row blocks; each K operand
  // read from LDS feeds both blocks.  A half's K operands are read just
  // before its products and the V^T operands just before theirs (below):
  // holding all of a tile's operands at once took 200 VGPRs and two
  // workgroups per CU; read this way the kernel fits three (164 VGPRs),
  // whose waves hide the LDS latency instead (measured on MI355X: 8 whole
  // prompts 519 -> 483 us, 512-token chunks 783 -> 769 us).
  f32x4_t st[kRB][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    bf16x8_t kop[KSTEPS];
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) kop[i] = kop_at(hh, i);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) st[rb][hh] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        st[rb][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[i], __builtin_bit_cast(bf16x8_t, qop[rb][i]),
                                                             st[rb][hh], 0, 0, 0);
  }
  // V^T operands read now, into the registers the K operands held, arrive
  // during the softmax.
  bf16x8_t vop_early[VEARLY > 0 ? VEARLY : 1];
#pragma unroll
  for (int j = 0; j < VEARLY; ++j) vop_early[j] = vop_at(j);
  // Waves share each SIMD: a wave in its softmax (a chain of vector
  // instructions) runs at a higher priority than one issuing matrix ops,
  // so it gets through and reaches its own matrix ops sooner while the
  // other's are in the pipeline (measured on MI355X: 1.3-1.5% faster;
  // the opposite, or raising it already at the V^T reads, was not).
  __builtin_amdgcn_s_setprio(2);
  // Per row block: causal mask (only where the tile reaches past the
  // block's first row), reference max, probabilities.
  bf16x8_t pb[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const bool diag = kt0 + kKeys - 1 > row0 + 16 * rb;  // wave-uniform
    // raw scores; the scale (positive) enters through the max and the
    // exponent's fma
    float z[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 4; ++e) z[4 * hh + e] = st[rb][hh][e];
    if (__builtin_expect(diag, 0)) {  // rare: laid out off the common path
      // A real branch: most tiles lie wholly below the block's first row,
      // and the compiler would otherwise turn the mask into selects that
      // every tile pays for (an empty volatile asm cannot be speculated).
      asm volatile("");
      // key kt0 + 16hh + 4g + e lies past the row when 16hh + e > lim.
      // kt0 passes through an empty asm so that lim is formed here, not
      // stepped on every tile as an induction variable.
      int kt = kt0;
      asm("" : "+s"(kt));
      const int lim = prow[rb] - 4 * g - kt;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * hh + e > lim) z[4 * hh + e] = -INFINITY;
    }
    // Weights against the current reference max m, and their sum.  m moves
    // only when some lane's sum of its 8 weights comes out above kLazyW =
    // 2^8, which every weight above 2^8 (a score past m by more than 8, log2
    // units; +inf included) causes and a NaN does not (a NaN score stays NaN
    // either way): then the row max over its 4 lanes becomes m and the
    // weights are recomputed.  So the rescale of O^T is rare after the first
    // tiles, and the common path spends no instruction on the max's scale
    // or on a max of the weights: the sum it needs anyway is the test
    // (measured on MI355X: 1.8-2.4% faster than a separate max over the
    // weights).  The result does not depend on m.
    f32x8_t p;
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = exp2_fast(fmaf(z[e], qscale, -m[rb]));
    float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    if (__builtin_expect(__any(ps > kLazyW), 0)) {  // rare, as the mask above
      // (measured on MI355X, both marked: 0.5-0.7% faster on both workloads)
      float mx = z[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = __builtin_elementwise_maximum(mx, z[e]);
      mx *= qscale;
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(xor16, __float_as_int(mx))));
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(xor32, __float_as_int(mx))));
      const float mn = fmaxf(m[rb], mx);
      const float alpha = exp2_fast(m[rb] - mn);
      m[rb] = mn;
      l[rb] *= alpha;
#pragma unroll
      for (int j = 0; j < OB; ++j) o[rb][j] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = exp2_fast(fmaf(z[e], qscale, -mn));
      ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    l[rb] += ps;
    pb[rb] = __builtin_convertvector(p, bf16x8_t);
  }
  __builtin_amdgcn_s_setprio(0);
  // O^T += V^T P^T, keys in the lane's order (4g..4g+3, 16+4g..16+4g+3).
#pragma unroll
  for (int j = 0; j < OB; ++j) {
    const bf16x8_t vop = j < VEARLY ? vop_early[j < VEARLY ? j : 0] : vop_at(j);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) o[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[rb], o[rb][j], 0, 0, 0);
  }
}

// Row sums over each row's 4 lanes; the normalised rows of the wave.
template <int D>
__device__ __forceinline__ void store_rows(const PrefillArgs &a, const f32x4_t (&o)[kRB][D / 16],
                                           const float (&l)[kRB], const bool (&row_ok)[kRB], int lo, int tok0,
                                           int h, int nl, int g) {
  constexpr int OB = D / 16;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float lr = l[rb];
    lr += __shfl_xor(lr, 16, 64);
    lr += __shfl_xor(lr, 32, 64);
    if (row_ok[rb]) {
      const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
      const size_t base = ((size_t)(lo + tok0 + 16 * rb + nl) * a.num_q_heads + h) * D + 4 * g;
#pragma unroll
      for (int j = 0; j < OB; ++j) {
        const f32x4_t v = o[rb][j] * inv;
        if (a.out_f32) {
          *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + base + 16 * j) =
              make_float4(v[0], v[1], v[2], v[3]);
        } else {
          const uint32_t w0 = (uint32_t)to_bf16(v[0]) | ((uint32_t)to_bf16(v[1]) << 16);
          const uint32_t w1 = (uint32_t)to_bf16(v[2]) | ((uint32_t)to_bf16(v[3]) << 16);
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + base + 16 * j) = make_uint2(w0, w1);
        }
      }
    }
  }
}

// The wave's rows, their positions, and their query operands.
template <int D>
struct WaveRows {
  int prow[kRB];       // position of the lane's row of block rb (-1: no row)
  bool row_ok[kRB];
  uint4 qop[kRB][D / 32];  // B operands of S^T: channels [8(4i + g), +8) of each row's query

  __device__ __forceinline__ void load(const PrefillArgs &a, int lo, int n, int first_pos, int tok0, int h,
                                       int nl, int g) {
    constexpr int C = D / 8;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int tok = tok0 + 16 * rb + nl;
      row_ok[rb] = tok < n;
      prow[rb] = row_ok[rb] ? first_pos + tok : -1;
      const uint4 *qrow = a.q + ((size_t)(lo + (row_ok[rb] ? tok : 0)) * a.num_q_heads + h) * C + g;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) qop[rb][i] = row_ok[rb] ? qrow[4 * i] : make_uint4(0, 0, 0, 0);
    }
  }
};

template <int D, int G>
// Three workgroups per CU (see the operand reads in the tile loop).
__global__ __launch_bounds__(kThreads, 3) void prefill_kernel(PrefillArgs a) {
  constexpr int GW = G < 4 ? G : 4;   // query heads per workgroup
  constexpr int TQ = 16 * kRB * (4 / GW);  // query tokens per workgroup
  constexpr int HG = G / GW;          // workgroups per (KV head, query block)
  constexpr int C = D / 8;            // 16-byte chunks per row
  constexpr int OB = D / 16;          // 16-channel blocks of the output
  __shared__ PrefillShared<D> sh;

  const WorkItem wk = find_work<HG, TQ>(a, sh.tbl);
  const int s = wk.s, lo = wk.lo, n = wk.n, ctx = wk.ctx, kvh = wk.kvh;
  const int q0 = wk.qb * TQ;
  if (q0 >= n) return;
  const int first_pos = ctx - n;  // position of query 0 of the sequence

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int nl = lane & 15;
  // byte addresses of the lanes 16 and 32 away (the 4 lanes of a row)
  const int xor16 = (lane ^ 16) << 2;
  const int xor32 = (lane ^ 32) << 2;
  const int h = kvh * G + wk.hg * GW + wave % GW;
  const int tok0 = q0 + (wave / GW) * 16 * kRB;  // the wave's first query
  // keys the workgroup needs, and the ones this wave needs
  const int kend = max(0, min(ctx, first_pos + min(q0 + TQ, n)));
  const int wkend = tok0 < n ? max(0, min(ctx, first_pos + min(tok0 + 16 * kRB, n))) : 0;

  WaveRows<D> rows;
  rows.load(a, lo, n, first_pos, tok0, h, nl, g);

  f32x4_t o[kRB][OB];  // O^T: channel 16j + 4g + e of row nl of block rb
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int j = 0; j < OB; ++j) o[rb][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // running max per row (shared by the row's 4 lanes) and this lane's sum
  float m[kRB], l[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m[rb] = kNegBig;
    l[rb] = 0.0f;
  }

  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks;
  // rows per block; the host keeps it below 2^31, and block ids are
  // clamped into the pool (non-negative), so one 32 x 32 -> 64-bit multiply
  // places a block
  const uint32_t block_rows = (uint32_t)(a.num_kv_heads * a.block_size);
  const size_t head_rows = (size_t)kvh * a.block_size;

  // The block ids of keys [0, kend), staged once when they fit.
  const int nblk = (kend + a.block_size - 1) >> a.log2_bs;
  const bool tbl_lds = nblk <= kTblLds;
  if (tbl_lds)
    for (int i = tid; i < nblk; i += kThreads) {
      const int blk = trow[i];
      sh.tbl[i] = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;  // stay inside the pool
    }
  __syncthreads();

  // Staging: item i (thread tid, tid + 256, ...) moves 16-byte chunk ch of
  // keys 2kp and 2kp + 1 (ch = i % C, kp = i / C), so that each load
  // instruction reads whole rows; with D = 64 the last two waves have no
  // item.  Loads are not predicated per lane, so that nothing serialises
  // them: a key at or past kend reads key kend - 1 and is stored as zeros (it
  // is never visible).
  constexpr int ITEMS = kKeys / 2 * C;
  constexpr int NCH = (ITEMS + kThreads - 1) / kThreads;
  static_assert(ITEMS % 64 == 0, "items must cover whole waves");
  uint4 kreg[NCH][2], vreg[NCH][2];

  // The tile loop, with the block ids read from LDS (STAGED) or from HBM.
  auto run = [&](auto staged_tag) {
  constexpr bool STAGED = decltype(staged_tag)::value;
  auto key_row = [&](int kk) -> size_t {
    int blk;
    if constexpr (STAGED) blk = sh.tbl[kk >> a.log2_bs];
    else blk = max(0, min(trow[kk >> a.log2_bs], a.num_blocks - 1));
    return (uint64_t)(uint32_t)blk * block_rows + head_rows + (kk & (a.block_size - 1));
  };
  // A tile below kend needs neither the clamp nor the zero fill; the two
  // keys of a pair share a block (and sit in consecutive rows) unless the
  // block size is 1.
  const bool pair_rows = a.block_size >= 2;
  auto load_tile = [&](int kt0) {
    const bool full = kt0 + kKeys <= kend;  // uniform
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int item = tid + u * kThreads;
      if (item >= ITEMS) break;  // uniform per wave
      const int ch = item % C;
      const int kp = item / C;
      const int k0 = kt0 + 2 * kp;
      size_t o0, o1;  // uint4 offsets of the two keys' chunks
      if (full) {
        o0 = key_row(k0) * C + ch;
        o1 = pair_rows ? o0 + C : key_row(k0 + 1) * C + ch;
      } else {
        o0 = key_row(min(k0, kend - 1)) * C + ch;
        o1 = key_row(min(k0 + 1, kend - 1)) * C + ch;
      }
      // Ordinary (cached) loads for K and V alike: every later query block
      // of the same (sequence, KV head) reads these tiles again, mostly
      // from L2 (measured on MI355X: streaming V past the caches was 2-4%
      // slower on whole prompts, chunks and prefix-cached suffixes).
      kreg[u][0] = a.k_cache[o0];
      kreg[u][1] = a.k_cache[o1];
      vreg[u][0] = a.v_cache[o0];
      vreg[u][1] = a.v_cache[o1];
    }
  };
  auto store_tile = [&](int b, int kt0) {
    if (kt0 + kKeys <= kend) {  // uniform: a full tile, stored as loaded
#pragma unroll
      for (int u = 0; u < NCH; ++u) {
        const int item = tid + u * kThreads;
        if (item >= ITEMS) break;  // uniform per wave
        const int ch = item % C;
        const int kp = item / C;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          sh.k[b][2 * kp + e][ch] = kreg[u][e];
          sh.v[b][2 * kp + e][ch] = vreg[u][e];
        }
      }
    } else {
      // the last, partial tile: keys at or past kend are stored as zeros (a
      // real branch, so that full tiles do not pay for the selects)
      asm volatile("");
#pragma unroll
      for (int u = 0; u < NCH; ++u) {
        const int item = tid + u * kThreads;
        if (item >= ITEMS) break;  // uniform per wave
        const int ch = item % C;
        const int kp = item / C;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bool past = kt0 + 2 * kp + e >= kend;
          sh.k[b][2 * kp + e][ch] = past ? make_uint4(0, 0, 0, 0) : kreg[u][e];
          sh.v[b][2 * kp + e][ch] = past ? make_uint4(0, 0, 0, 0) : vreg[u][e];
        }
      }
    }
  };

  const int ntiles = (kend + kKeys - 1) / kKeys;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0, 0);
  }
  // Nothing in flight from here on (the query loads included), so the waits
  // in the loop only cover the next tile's loads.
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    const int kt0 = t * kKeys;
    if (t + 1 < ntiles) load_tile(kt0 + kKeys);  // in flight during this tile's math
    if (kt0 < wkend) {
      // V^T operand of channel block j: lane (g, n) names key rows 4g + n / 4
      // and 16 + 4g + n / 4 at channels 16j + 4 (n % 4) .. + 3, and receives
      // channel 16j + n of keys 4g..4g+3 and 16+4g..16+4g+3.
      constexpr int VS = D + 16;  // elements per V row in LDS
      const uint16_t *vb = reinterpret_cast<const uint16_t *>(&sh.v[b][0][0]);
      const int off0 = (4 * g + (nl >> 2)) * VS + 4 * (nl & 3);
      attend_tile<D, 0>(
          [&](int hh, int i) { return __builtin_bit_cast(bf16x8_t, sh.k[b][16 * hh + nl][4 * i + g]); },
          [&](int j) {
            const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vb + off0 + 16 * j));
            const s16x4_t hi4 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vb + off0 + 16 * VS + 16 * j));
            return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          },
          rows.qop, o, m, l, rows.prow, kt0, first_pos + tok0, g, a.qscale, xor16, xor32);
    }
    __builtin_amdgcn_s_setprio(0);
    if (t + 1 < ntiles) store_tile(b ^ 1, kt0 + kKeys);
    __syncthreads();
  }
  };
  if (tbl_lds) run(std::true_type{});
  else run(std::false_type{});

  store_rows<D>(a, o, l, rows.row_ok, lo, tok0, h, nl, g);
}

// ---- The ring pipeline (head_dim 128, block size >= 8) ----
//
// Tiles reach LDS without passing through registers: each wave issues
// global_load_lds_dwordx4 (64 lanes x 16 bytes straight into LDS at M0 +
// 16 x lane) for 8 key rows of K and of V per tile, two tiles ahead, into a
// ring of three tile slots.  Compared with loading the next tile into
// registers and storing it after the math, this frees the 16 staging VGPRs
// and the per-tile address arithmetic, and gives each load two tiles of
// math to arrive in (measured on MI355X: a build that skipped the loads
// altogether ran 10-17% faster, the bound of what hiding them can win).
//
// The compiler does not follow these loads: they are issued from inline
// assembly, which writes no register, and the waits on them are explicit
// (vmcnt counts this wave's loads in the order it issued them; nothing else
// the compiler tracks is in flight inside the tile loop).  The block ids
// come from scalar loads through the constant address space (the table is
// not written during the call), so they use the scalar counter and keep
// the vector count to the tiles alone.
//
// LDS image of a tile: K and V as 8 groups of 4 key rows each.  A group is
// one load instruction.  Each quad of lanes (4 consecutive lanes, which the
// vector memory path serves together) brings 64 contiguous bytes of one
// row: quad 4s + r loads segment s (bytes 64s..64s+63) of row r, so a group
// is stored segment-major (segment s of row r at 256 s + 64 r), and groups
// sit 1056 bytes apart (32 bytes of padding).  A quad that spans 4 rows
// instead touched 4 cache lines per quad: 2.9x the vector L1 accesses and
// 11% slower.  Laid out this way, the K operand reads (rows nl, chunk
// 4i + g) of the lanes the LDS serves together (0-7 with 16-23) and the V^T
// transposing reads of lanes 0-31 fall in 64 different banks, and every
// read of the tile math is a lane constant plus an immediate.
constexpr int kRing = 3;         // tile slots: the one in use and the next two
constexpr int kGrp = 1056;       // bytes from one group to the next
constexpr int kSlotK = 8 * kGrp;
constexpr int kSlot = 2 * kSlotK;  // bytes per tile slot (K, then V)
constexpr int kRowBytes = 256;   // one bf16 row of 128 channels
// s_waitcnt operand: vmcnt(4) (one tile of this wave's loads may stay in flight)
constexpr int kWaitVmem4 = 0x0F74;

typedef __attribute__((address_space(4))) const int32_t const_i32;

// 16 bytes per lane from base + voff into LDS at lds + 16 * lane.  M0 holds
// the LDS address (the compiler uses M0 for nothing in these kernels; it is
// declared clobbered all the same, which clang notes as a reserved register).
// One wait state between the M0 write and the load that reads it.
// load_lds16_at: the same from a 64-bit address per lane.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(uint64_t base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "m0");
}
__device__ __forceinline__ void load_lds16_at(uint64_t addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(addr) : "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32);
}

// WRITE: the fused store of pa_prefill_write.  The workgroups of head group
// 0 store their query tokens' key and value rows of their KV head (so every
// new row is stored once), and every workgroup reads the chunk's keys (its
// last n positions) from those input rows, not from the pools: no workgroup
// waits for another's stores.
template <int G, bool WRITE>
// Three workgroups per CU: 3 x 50,688 bytes of ring fit the 160 KiB of LDS.
__global__ __launch_bounds__(kThreads, 3) void prefill_ring_kernel(PrefillArgs a) {
  constexpr int D = 128;
  constexpr int GW = G < 4 ? G : 4;   // query heads per workgroup
  constexpr int TQ = 16 * kRB * (4 / GW);  // query tokens per workgroup
  constexpr int HG = G / GW;          // workgroups per (KV head, query block)
  constexpr int OB = D / 16;          // 16-channel blocks of the output
  __shared__ uint4 ring[kRing * kSlot / 16];

  const WorkItem wk = find_work<HG, TQ>(a, reinterpret_cast<int32_t *>(ring));
  const int s = wk.s, lo = wk.lo, n = wk.n, ctx = wk.ctx, kvh = wk.kvh;
  const int q0 = wk.qb * TQ;
  if (q0 >= n) return;
  const int first_pos = ctx - n;  // position of query 0 of the sequence

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int nl = lane & 15;
  const int xor16 = (lane ^ 16) << 2;
  const int xor32 = (lane ^ 32) << 2;
  const int h = kvh * G + wk.hg * GW + wave % GW;
  const int tok0 = q0 + (wave / GW) * 16 * kRB;  // the wave's first query
  // keys the workgroup needs, and the ones this wave needs
  const int kend = max(0, min(ctx, first_pos + min(q0 + TQ, n)));
  const int wkend = tok0 < n ? max(0, min(ctx, first_pos + min(tok0 + 16 * kRB, n))) : 0;

  // WRITE, head group 0: rows q0 .. q0 + TQ - 1 of the chunk (those that
  // exist), KV head kvh, 16 bytes of K and of V per item.
  // - 32 tokens per workgroup (4 or 8 query heads per KV head): the rows
  //   are the workgroup's last keys, so after the tile loop they sit in the
  //   last two ring slots (brought from the input rows); they are stored from
  //   there, and only their slots are loaded up front.  No wait covers these
  //   stores (measured on MI355X: the stores and row loads at the start cost
  //   ~19 us per call on whole prompts).
  // - more tokens per workgroup: the rows are loaded with the queries (one
  //   round trip for both) and stored just before the first tile loads;
  //   vmcnt counts stores too, in issue order, so the tile loop's first wait
  //   covers them along with the first tile's loads, and no later wait does.
  constexpr bool kStoreFromLds = TQ == kKeys;
  constexpr int kStoreItems = TQ * (D / 8);
  constexpr int NST = WRITE ? (kStoreItems + kThreads - 1) / kThreads : 1;
  const bool storing = WRITE && wk.hg == 0;
  const int items = storing ? min(TQ, n - q0) * (D / 8) : 0;
  // a vector type, not uint4: a uint4 copied from memory becomes a memcpy
  // that leaves these arrays on the stack
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t st_k[NST], st_v[NST];
  int64_t st_slot[NST];
  if constexpr (WRITE) {
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int i = tid + j * kThreads;
      st_slot[j] = -1;
      if (i < items) {
        const int r = lo + q0 + i / (D / 8);
        const size_t src = ((size_t)r * a.num_kv_heads + kvh) * (D / 8) + i % (D / 8);
        st_slot[j] = a.slot_mapping[r];
        if constexpr (!kStoreFromLds) {
          st_k[j] = reinterpret_cast<const u32x4_t *>(a.k_new)[src];
          st_v[j] = reinterpret_cast<const u32x4_t *>(a.v_new)[src];
        }
      }
    }
  }

  WaveRows<D> rows;
  rows.load(a, lo, n, first_pos, tok0, h, nl, g);

  // The query rows (and the rows to store) have arrived before any tile
  // load is issued: from here on, vmcnt counts the stores and then this
  // wave's tile loads only.
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  if constexpr (WRITE && !kStoreFromLds) {
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int i = tid + j * kThreads;
      const int64_t slot = st_slot[j];
      if (i < items && slot >= 0 && slot < a.num_slots) {  // slots < 0 or outside the pool are skipped
        const size_t dst = (((size_t)(slot >> a.log2_bs) * a.num_kv_heads + kvh) * a.block_size +
                            (slot & (a.block_size - 1))) * (D / 8) + i % (D / 8);
        reinterpret_cast<u32x4_t *>(const_cast<uint4 *>(a.k_cache))[dst] = st_k[j];
        reinterpret_cast<u32x4_t *>(const_cast<uint4 *>(a.v_cache))[dst] = st_v[j];
      }
    }
  }

  f32x4_t o[kRB][OB];  // O^T: channel 16j + 4g + e of row nl of block rb
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int j = 0; j < OB; ++j) o[rb][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m[kRB], l[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m[rb] = kNegBig;
    l[rb] = 0.0f;
  }

  const_i32 *trow = (const_i32 *)(a.block_tables + (size_t)s * a.max_blocks);
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)ring;
  const uint64_t block_bytes = (uint64_t)(uint32_t)(a.num_kv_heads * a.block_size) * kRowBytes;
  const uint64_t head_bytes = (uint64_t)kvh * a.block_size * kRowBytes;
  const uint64_t kbase = (uint64_t)(uintptr_t)a.k_cache + head_bytes;
  const uint64_t vbase = (uint64_t)(uintptr_t)a.v_cache + head_bytes;
  const uint32_t lane_seg = (lane >> 4) * 64 + (lane & 3) * 16;  // segment and chunk of the lane's 16 bytes
  const uint32_t lane_off = ((lane >> 2) & 3) * kRowBytes + lane_seg;
  const int bmask = a.block_size - 1;
  // the chunk's rows (WRITE): position p >= first_pos is row lo + p - first_pos
  const uint32_t new_row_bytes = (uint32_t)a.num_kv_heads * kRowBytes;
  const uint64_t knew = (uint64_t)(uintptr_t)a.k_new + (uint64_t)kvh * kRowBytes;
  const uint64_t vnew = (uint64_t)(uintptr_t)a.v_new + (uint64_t)kvh * kRowBytes;
  auto new_row_at = [&](int p) -> uint64_t { return (uint64_t)(uint32_t)(lo + p - first_pos) * new_row_bytes; };
  const uint32_t lane_new_off = ((lane >> 2) & 3) * new_row_bytes + lane_seg;

  // The table entry of group grp (keys 32u + 8 wave + 4 grp ..) of tile u.
  // A group's 4 keys share a block (block size >= 8, groups 4-aligned).
  // The entry is clamped into the pool where it is used, so that the wait
  // for the scalar load falls there, a tile later.
  auto block_of = [&](int u, int grp) -> int {
    const int key0 = min(u * kKeys + 8 * wave + 4 * grp, kend - 1);
    return trow[key0 >> a.log2_bs];
  };
  // This wave's loads of tile u (4 instructions): its two groups of K and V.
  // Keys at or past kend read key kend - 1 instead (a real key, finite; the
  // causal mask gives every such key weight 0).
  auto load_tile = [&](int u, int slot_idx, int blk0, int blk1) {  // slot_idx = u % kRing
    const uint32_t slot = ring0 + (uint32_t)slot_idx * kSlot;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const int qg = 2 * wave + grp;
      const int kt = u * kKeys + 4 * qg;
      if (WRITE && min(kt + 3, kend - 1) >= first_pos) {  // uniform: the group holds keys of the chunk
        const uint32_t kdst = __builtin_amdgcn_readfirstlane(slot + qg * kGrp);
        const uint32_t vdst = __builtin_amdgcn_readfirstlane(slot + kSlotK + qg * kGrp);
        if (kt >= first_pos) {  // all from the chunk's rows
          const int key0 = min(kt, kend - 1);
          // the lane's row offset is a lane constant unless the group
          // reaches kend (uniform; a real branch, as for the causal mask)
          uint32_t voff = lane_new_off;
          if (kt + 3 >= kend) {
            asm volatile("");
            const int p = min(kt + ((lane >> 2) & 3), kend - 1);  // the lane's key
            voff = (uint32_t)(p - key0) * new_row_bytes + lane_seg;
          }
          load_lds16(uniform64(knew + new_row_at(key0)), voff, kdst);
          load_lds16(uniform64(vnew + new_row_at(key0)), voff, vdst);
        } else {  // keys before first_pos from the pool (block of kt), the rest from the chunk's rows
          const int p = min(kt + ((lane >> 2) & 3), kend - 1);  // the lane's key
          const int blk = grp ? blk1 : blk0;
          const uint32_t pb = (unsigned)blk < (unsigned)a.num_blocks ? (uint32_t)blk : 0u;
          const uint64_t pool = (uint64_t)pb * block_bytes + (uint64_t)(p & bmask) * kRowBytes + lane_seg;
          const bool fresh = p >= first_pos;
          const uint64_t nrow = fresh ? new_row_at(p) + lane_seg : 0;
          load_lds16_at(fresh ? knew + nrow : kbase + pool, kdst);
          load_lds16_at(fresh ? vnew + nrow : vbase + pool, vdst);
        }
        continue;
      }
      int key0 = kt;
      uint32_t voff = lane_off;
      if (kt + 3 >= kend) {  // uniform: the group reaches kend (a real branch)
        asm volatile("");
        key0 = min(kt, kend - 1);
        voff = (uint32_t)(min(kt + ((lane >> 2) & 3), kend - 1) - key0) * kRowBytes + (lane >> 4) * 64 + (lane & 3) * 16;
      }
      const int blk = grp ? blk1 : blk0;
      const uint32_t pb = (unsigned)blk < (unsigned)a.num_blocks ? (uint32_t)blk : 0u;  // stay inside the pool
      const uint64_t off = (uint64_t)pb * block_bytes + (uint64_t)(key0 & bmask) * kRowBytes;
      load_lds16(uniform64(kbase + off), voff, __builtin_amdgcn_readfirstlane(slot + qg * kGrp));
      load_lds16(uniform64(vbase + off), voff, __builtin_amdgcn_readfirstlane(slot + kSlotK + qg * kGrp));
    }
  };

  // Lane constants of the tile math's LDS reads (bytes from the slot).
  // K operand (hh, i): key row 16hh + nl = group 4hh + nl / 4, row nl % 4,
  // segment i, chunk g of the segment.  V^T operand j: lane names key row
  // 4g + nl / 4 (and 16 + that: group g + 4) at channels 16j + 4 (nl % 4)
  // .. + 3: segment j / 2, chunk 2 (j % 2) + (nl / 2) % 2, half nl % 2.
  const uint32_t k_lane = (nl >> 2) * kGrp + (nl & 3) * 64 + g * 16;
  const uint32_t v_lane = g * kGrp + (nl >> 2) * 64 + ((nl >> 1) & 1) * 16 + (nl & 1) * 8;

  const uint32_t k_at = ring0 + k_lane, v_at = ring0 + kSlotK + v_lane;

  const int ntiles = (kend + kKeys - 1) / kKeys;
  int nb0 = 0, nb1 = 0;  // block ids of the tile loaded next
  // (t % kRing) * kSlot, stepped in a scalar register: one vector add per
  // read address and tile (the compiler had rebuilt it from t * kSlot and
  // t / 3 with two)
  if (ntiles > 0) load_tile(0, 0, block_of(0, 0), block_of(0, 1));
  if (ntiles > 1) load_tile(1, 1, block_of(1, 0), block_of(1, 1));
  if (ntiles > 2) {
    nb0 = block_of(2, 0);
    nb1 = block_of(2, 1);
  }
  // The tile loop, unrolled by the ring's three slots so that each copy's
  // slot is a constant.
  auto tile_step = [&](int t, auto slot_tag) {
    constexpr uint32_t SLOT = decltype(slot_tag)::value;
    // this wave's loads of tile t have landed (those of t + 1 may not), then
    // every wave's have
    if (t + 1 < ntiles) __builtin_amdgcn_s_waitcnt(kWaitVmem4);
    else __builtin_amdgcn_s_waitcnt(kWaitVmem);
    __syncthreads();
    // tile t + 2 goes to the slot of tile t - 1, which every wave finished
    // reading before the barrier
    if (t + 2 < ntiles) load_tile(t + 2, (SLOT + 2) % kRing, nb0, nb1);
    const int kt0 = t * kKeys;
    if (kt0 < wkend) {
      // The tile's K and V^T reads: a loop-invariant lane base plus an
      // immediate offset (the slot is a constant of this copy of the body,
      // and every offset stays below 64 KiB), no per-tile address work.
      const uint32_t ka = k_at + SLOT * kSlot, va = v_at + SLOT * kSlot;
      // half the V^T operands read before the softmax (measured on MI355X:
      // 1-1.5% faster on whole prompts, 0.6% on chunks; all of them do not
      // fit three workgroups per CU)
      attend_tile<D, OB / 2>(
          [&](int hh, int i) { return *(const lds_bf16x8_t *)(uintptr_t)(ka + hh * 4 * kGrp + i * 256); },
          [&](int j) {
            const uint32_t v = va + (j >> 1) * 256 + (j & 1) * 32;
            const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)v);
            const s16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(uintptr_t)(v + 4 * kGrp));
            return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          },
          rows.qop, o, m, l, rows.prow, kt0, first_pos + tok0, g, a.qscale, xor16, xor32);
    }
    // The table entries of tile t + 3, read after the tile's LDS reads: the
    // scalar loads share the LDS wait counter, and here they are waited for
    // only at the next barrier.
    if (t + 3 < ntiles) {
      nb0 = block_of(t + 3, 0);
      nb1 = block_of(t + 3, 1);
    }
  };
  for (int t = 0; t < ntiles; t += kRing) {
    tile_step(t, std::integral_constant<uint32_t, 0>{});
    if (t + 1 >= ntiles) break;
    tile_step(t + 1, std::integral_constant<uint32_t, 1>{});
    if (t + 2 >= ntiles) break;
    tile_step(t + 2, std::integral_constant<uint32_t, 2>{});
  }
  if constexpr (WRITE && kStoreFromLds) {
    // Row i of the workgroup's tokens (position first_pos + q0 + i) is key
    // p of tile p / 32, in ring slot (p / 32) % 3: group (p % 32) / 4, row
    // p % 4 of it, segment c / 4, chunk c % 4 (c the 16-byte chunk).  The
    // last two tiles hold all of them, and no tile load came after them.
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int i = tid + j * kThreads;
      const int64_t slot = st_slot[j];
      const int p = first_pos + q0 + i / (D / 8), c = i % (D / 8);
      // slots < 0 or outside the pool are skipped, and so are positions
      // below 0 (which no tile holds; their slots are < 0)
      if (i < items && p >= 0 && slot >= 0 && slot < a.num_slots) {
        const uint32_t at = (uint32_t)((p / kKeys) % kRing) * kSlot + ((p % kKeys) >> 2) * kGrp + (c >> 2) * 256 +
                            (p & 3) * 64 + (c & 3) * 16;
        const u32x4_t kv = *(const __attribute__((address_space(3))) u32x4_t *)(uintptr_t)(ring0 + at);
        const u32x4_t vv = *(const __attribute__((address_space(3))) u32x4_t *)(uintptr_t)(ring0 + at + kSlotK);
        const size_t dst = (((size_t)(slot >> a.log2_bs) * a.num_kv_heads + kvh) * a.block_size +
                            (slot & (a.block_size - 1))) * (D / 8) + c;
        reinterpret_cast<u32x4_t *>(const_cast<uint4 *>(a.k_cache))[dst] = kv;
        reinterpret_cast<u32x4_t *>(const_cast<uint4 *>(a.v_cache))[dst] = vv;
      }
    }
  }
  store_rows<D>(a, o, l, rows.row_ok, lo, tok0, h, nl, g);
}

template <int D, int G>
hipError_t launch_dg(const PrefillArgs &a, int n_work, hipStream_t st) {
  if (D == 128 && a.block_size >= 8) {
    if (a.k_new)
      hipLaunchKernelGGL((prefill_ring_kernel<G, true>), dim3(n_work), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_ring_kernel<G, false>), dim3(n_work), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<D, G>), dim3(n_work), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int group, const PrefillArgs &a, int n_work, hipStream_t st) {
  switch (group) {
    case 1: return launch_dg<D, 1>(a, n_work, st);
    case 2: return launch_dg<D, 2>(a, n_work, st);
    case 4: return launch_dg<D, 4>(a, n_work, st);
    case 8: return launch_dg<D, 8>(a, n_work, st);
  }
  return hipErrorInvalidValue;
}

// pa_prefill and pa_prefill_write.  Every argument is checked before
// anything is enqueued.  With k_new set the chunk's rows are stored too: in
// the attention kernel itself where it loads tiles straight into LDS, else
// by pa_write_kv ahead of the attention.
pa_status_t prefill_impl(const char *who, const void *q, int32_t num_tokens, int32_t num_q_heads,
                         const int32_t *cu_seqlens, int32_t num_seqs, int32_t max_query_len, const void *k_cache,
                         const void *v_cache, const pa_cache_t *cache, const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                         float scale, void *out, int32_t out_dtype, void *stream, const void *k_new,
                         const void *v_new, const int64_t *slot_mapping) {
  using pa::fail;
  if (!cache) return fail(PA_EINVAL, "%s: cache descriptor is NULL", who);
  const pa_cache_t c = *cache;
  if (num_tokens < 0 || num_seqs < 0 || max_query_len < 0 || max_context_len < 0 || num_q_heads <= 0 ||
      c.num_blocks <= 0 || c.num_kv_heads <= 0 || c.block_size <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_EINVAL, "%s: sizes must be positive (counts may be 0)", who);
  if (c.dtype != PA_BF16) return fail(PA_EUNSUPPORTED, "%s: cache dtype %d (built: bf16)", who, c.dtype);
  if (out_dtype != PA_F32 && out_dtype != PA_BF16)
    return fail(PA_EUNSUPPORTED, "%s: out dtype %d (use PA_F32 or PA_BF16)", who, out_dtype);
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(PA_EUNSUPPORTED, "%s: head_dim %d (built: 64, 128)", who, c.head_dim);
  if (c.block_size > 256 || (c.block_size & (c.block_size - 1)))
    return fail(PA_EUNSUPPORTED, "%s: block_size %d (powers of two up to 256)", who, c.block_size);
  if ((int64_t)c.num_kv_heads * c.block_size > INT32_MAX)
    return fail(PA_EUNSUPPORTED, "%s: %d KV heads x block size %d: over 2^31 rows per block", who,
                c.num_kv_heads, c.block_size);
  if (num_q_heads % c.num_kv_heads)
    return fail(PA_EINVAL, "%s: %d query heads not a multiple of %d KV heads", who, num_q_heads,
                c.num_kv_heads);
  if (!(scale > 0.0f) || !(scale < INFINITY))
    return fail(PA_EINVAL, "%s: scale %g must be positive and finite", who, (double)scale);
  const int g = num_q_heads / c.num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PA_EUNSUPPORTED, "%s: query heads per KV head = %d (built: 1, 2, 4, 8)", who, g);
  const bool store = k_new != nullptr || v_new != nullptr || slot_mapping != nullptr;
  if (store && num_tokens > 0 && (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache))
    return fail(PA_EINVAL, "%s: NULL pointer", who);
  const bool attend = num_seqs > 0 && num_tokens > 0 && max_query_len > 0;
  if (attend && (!q || !cu_seqlens || !k_cache || !v_cache || !block_tables || !context_lens || !out))
    return fail(PA_EINVAL, "%s: NULL pointer", who);
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out | (uintptr_t)k_new |
       (uintptr_t)v_new) % 16)
    return fail(PA_EINVAL, "%s: q, out, the pools and the stored rows must be 16-byte aligned", who);

  int log2_bs = 0;
  while ((1 << log2_bs) < c.block_size) ++log2_bs;
  const int64_t cap64 = (int64_t)max_blocks_per_seq * c.block_size;
  const int gw = g < 4 ? g : 4;
  const int tq = 16 * kRB * (4 / gw);
  PrefillArgs a{};
  a.q = (const uint4 *)q;
  a.k_cache = (const uint4 *)k_cache;
  a.v_cache = (const uint4 *)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_seqlens = cu_seqlens;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c.num_kv_heads;
  a.block_size = c.block_size;
  a.log2_bs = log2_bs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = c.num_blocks;
  a.ctx_cap = (int32_t)(cap64 < max_context_len ? cap64 : max_context_len);
  a.q_blocks = attend ? (max_query_len + tq - 1) / tq : 0;
  // A batch of 2 to kCompactSeqs sequences gets a grid of the query blocks
  // that exist: sum over s of ceil(n_s / tq) <= ceil(num_tokens / tq) +
  // num_seqs (the rows are packed).
  const int64_t all_slots = (int64_t)num_seqs * a.q_blocks;
  const bool compact = num_seqs > 1 && num_seqs <= kCompactSeqs;
  const int64_t packed = ((int64_t)num_tokens + tq - 1) / tq + num_seqs;
  a.q_items = (int32_t)(compact && packed < all_slots ? packed : all_slots);
  // The merged tail's keys and values (2 bytes each of K and V per channel
  // and token) stay within 2 MiB per KV head, half an XCD's L2.
  a.tail_keys = (2 << 20) / (4 * c.head_dim);
  a.out_f32 = out_dtype == PA_F32 ? 1 : 0;
  a.qscale = scale * kLog2e;
  const int64_t n_work = (int64_t)a.q_items * c.num_kv_heads * (g / gw);
  if (n_work > 0x7fffffff)
    return fail(PA_EINVAL, "%s: grid of %lld workgroups too large", who, (long long)n_work);

  const bool fused = store && attend && c.head_dim == 128 && c.block_size >= 8;
  if (store && num_tokens > 0 && !fused)
    if (pa_status_t st = pa_write_kv(k_new, v_new, slot_mapping, num_tokens, const_cast<void *>(k_cache),
                                     const_cast<void *>(v_cache), cache, stream))
      return st;
  if (!attend) return PA_OK;
  if (fused) {
    a.k_new = (const uint4 *)k_new;
    a.v_new = (const uint4 *)v_new;
    a.slot_mapping = slot_mapping;
    a.num_slots = (int64_t)c.num_blocks * c.block_size;
  }
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = c.head_dim == 64 ? launch_d<64>(g, a, (int)n_work, st) : launch_d<128>(g, a, (int)n_work, st);
  if (e != hipSuccess) return fail(PA_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" pa_status_t pa_prefill(const void *q, int32_t num_tokens, int32_t num_q_heads,
                                  const int32_t *cu_seqlens, int32_t num_seqs, int32_t max_query_len,
                                  const void *k_cache, const void *v_cache, const pa_cache_t *cache,
                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, int32_t max_context_len, float scale,
                                  void *out, int32_t out_dtype, void *stream) {
  return prefill_impl("pa_prefill", q, num_tokens, num_q_heads, cu_seqlens, num_seqs, max_query_len, k_cache,
                      v_cache, cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale, out,
                      out_dtype, stream, nullptr, nullptr, nullptr);
}

extern "C" pa_status_t pa_prefill_write(const void *k, const void *v, const int64_t *slot_mapping, const void *q,
                                        int32_t num_tokens, int32_t num_q_heads, const int32_t *cu_seqlens,
                                        int32_t num_seqs, int32_t max_query_len, void *k_cache, void *v_cache,
                                        const pa_cache_t *cache, const int32_t *block_tables,
                                        int32_t max_blocks_per_seq, const int32_t *context_lens,
                                        int32_t max_context_len, float scale, void *out, int32_t out_dtype,
                                        void *stream) {
  if (num_tokens > 0 && (!k || !v || !slot_mapping)) return pa::fail(PA_EINVAL, "pa_prefill_write: NULL pointer");
  return prefill_impl("pa_prefill_write", q, num_tokens, num_q_heads, cu_seqlens, num_seqs, max_query_len, k_cache,
                      v_cache, cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale, out,
                      out_dtype, stream, k, v, slot_mapping);
}
