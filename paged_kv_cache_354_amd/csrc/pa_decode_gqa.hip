// Grouped-query paged decode attention on the gfx950 matrix cores (bf16 pools).
//
// foundry "PagedAttention" ops page, "How it works": attention reads K/V
// through the per-sequence block table, gathering scattered physical blocks,
// and the math is that of one contiguous run: per (sequence, query head)
// out = softmax(scale * q K^T) V, accumulated here in fp32 with an online
// softmax (Milakov & Gimelshein 2018) in the exp2 domain.
//
// When G = Hq / Hkv query heads share one KV head, the logits of a 16-token
// tile form a dense [G x d] x [d x 16] product; v_mfma_f32_16x16x32_bf16
// computes it with the G heads in the M dimension (rows G..15 are zero) and
// the 16 tokens in N.  That takes the dot products and their cross-lane sums
// off the vector ALUs, which then only run the softmax and the P.V update.
//
// A workgroup (4 wave64s) runs one token range of one (sequence, KV head):
// wave w takes tiles w, w + 4, ... of the range, two per loop iteration (the
// loads of both are issued first, so the second tile's loads are in flight
// while the first is computed; no load is in flight across the loop's back
// edge, which keeps the compiler's waits exact).  The range's slice of the
// block-table row is staged in LDS (in sub-ranges of at most tbl_cap
// blocks).  Two ways of cutting the work into ranges:
//   - grid: one workgroup per (sequence, KV head, partition of P tokens);
//   - balanced: a grid of one resident workgroup per slot of the GPU, each
//     taking an equal share of all (KV head, sequence, token) work in that
//     order (lengths rounded up to 16, plus a fixed cost per sequence), so
//     no tail of lone long workgroups is left; the shares of one XCD are
//     contiguous.  A workgroup that holds a whole sequence writes its
//     output directly; sequences cut between workgroups are combined by
//     merge_balanced_kernel.
//
// Lane layouts (lane l, 64 per wave):
//   QK operands   g = l / 16, n = l % 16.  For k-step i, lane l holds 8 bf16
//                 channels [8(4i + g), 8(4i + g) + 8) of token n's K row (one
//                 16-byte load) and of query head n's q row (zero for n >= G).
//                 The same (lane, slot) -> channel map on both operands makes
//                 every output a full dot product.
//   QK output     lane l, register j: head 4g + j, token n.
//   PV            a V row is d bf16 = LPR lanes x 16 bytes; lane (r, c) =
//                 (l / LPR, l % LPR) holds channels [8c, 8c + 8) of row r of
//                 each load, RPW = 64 / LPR rows per load.  The tile's p
//                 values go through a small per-wave LDS array to these lanes.
//
// The running max of every head is uniform across the wave (a row-wide max
// after each tile), so the accumulator rescale factors are read into scalar
// registers and skipped when no max moved.  Tokens at or past the end of the
// range read a valid token's row instead (never outside the sequence's
// blocks) and their logits are -inf by select, so tail slots cannot reach the
// output.  K and V rows are streamed with non-temporal loads.  Each K load
// covers half of a 128-byte line of 16 rows; the line's other half is read
// by the next load, issued right after it, and still comes from L2 (the
// measured HBM bytes stay within 3% of the algorithmic ones).  Marking K
// non-temporal as well took ~1 us off a 100 us call on the Llama-3-8B-shaped
// batch (MI355X, median of 185 dispatches).

#include <atomic>
#include <type_traits>

#include "pa_decode_common.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;        // tokens per MFMA tile
constexpr int kTilesPerIter = 2;

template <int D, int G>
struct GqaTile {
  static constexpr int KSTEPS = D / 32;
  static constexpr int LPR = D / 8;
  static constexpr int RPW = 64 / LPR;
  static constexpr int NV = kTile / RPW;
  uint4 k[KSTEPS];
  uint4 v[NV];
};

template <int D, int G, int NW>
struct GqaShared {
  float4 p[NW][kTile][G / 4];
  float red_m[NW][G];
  float red_l[NW][G];
  float red_acc[NW][G][D];
};

// Wave priority from the workgroup's progress through its share.  With equal
// shares the SIMD arbiter, which prefers older waves at equal priority, lets
// the first workgroup placed on a CU run well ahead of the last one
// (measured on MI355X: with equal shares the first finished in 0.69x the
// time of the third, leaving the end of the kernel to a few workgroups).
// Giving the waves of workgroups that are behind a higher priority
// (s_setprio 3 below 55% done, 2 below 75%, 1 below 90%, then 0) keeps them
// together: the spread of finish times fell from 50-98 us to 75-92 us on
// the Llama-3-8B-shaped batch.  Results do not depend on it.
__device__ __forceinline__ void set_progress_priority(float progress) {
  if (progress < 0.55f) __builtin_amdgcn_s_setprio(3);
  else if (progress < 0.75f) __builtin_amdgcn_s_setprio(2);
  else if (progress < 0.9f) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Attention of query heads [kvh G, kvh G + G) of sequence s over the tokens
// [start, end) (0 <= start <= end <= the sequence's length, start a multiple
// of 16): leaves every wave's (max, sum, acc) in sh.red_* and returns after a
// barrier.  tbl has room for tbl_cap >= 1 block ids, staged here; tbl_cap = 0
// means the caller already staged the range's block ids in tbl (entry 0 for
// the block holding token start) and made them visible with a barrier.
// BIG: block_size >= 16, so a tile (16 tokens starting at a multiple of 16)
// lies inside one block and needs one table lookup.  NW: waves per
// workgroup; wave w takes tiles w, w + NW, ... (TPI of them per step), so the
// summation order depends only on token positions.
// share_done >= 0 turns on progress-driven wave priority: share_done is how
// much of the workgroup's share (in tokens) came before this range and
// share_inv the reciprocal of the share's size (see set_progress_priority).
// newpos >= 0: the K and V rows of token newpos (in the range) are read from
// a.k_new / a.v_new (row s, head kvh) instead of the pools.
template <int D, int G, bool BIG, int NW, int TPI = kTilesPerIter>
__device__ __forceinline__ void gqa_range(const DecodeArgs &a, GqaShared<D, G, NW> &sh, int32_t *tbl,
                                          int tbl_cap, int s, int kvh, int start, int end,
                                          int share_done = -1, float share_inv = 0.0f, int newpos = -1) {
  using Tile = GqaTile<D, G>;
  constexpr int KSTEPS = Tile::KSTEPS;
  constexpr int LPR = Tile::LPR;
  constexpr int RPW = Tile::RPW;
  constexpr int NV = Tile::NV;
  constexpr int HR = G / 4;  // 16-lane rows of the QK output that hold real heads
  static_assert(G % 4 == 0 && G <= 16, "heads per KV head must be 4, 8, 12 or 16");
  static_assert(NV * RPW == kTile, "a tile must be a whole number of V loads");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int bs = a.block_size;
  const int log2_bs = a.log2_bs;

  // q operand: head n of this KV head's group, channel chunks 4i + g.
  const int h0 = kvh * G;
  uint4 qop[KSTEPS];
  {
    const uint4 *qrow = a.q + ((size_t)s * a.num_q_heads + h0 + (n < G ? n : 0)) * LPR + g;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) qop[i] = n < G ? qrow[4 * i] : make_uint4(0, 0, 0, 0);
  }

  float m[4], l[4];  // running max / partial sum of head 4g + j (this lane's tokens)
  float acc[G][8];   // PV accumulators: head h, channels [8c, 8c + 8) of the row group
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = kNegBig;
    l[j] = 0.0f;
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;

  const size_t block_rows = (size_t)a.num_kv_heads * bs;  // rows per physical block
  const size_t head_rows = (size_t)kvh * bs;
  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks;
  int first_blk = 0;
  int sub_end = start;

  // Row index (in K/V rows of D elements) of a token of the staged sub-range.
  auto token_row = [&](int t) -> size_t {
    const int blk = tbl[(t >> log2_bs) - first_blk];
    return (size_t)blk * block_rows + head_rows + (t & (bs - 1));
  };

  auto load_tile = [&](Tile &T, int t0) {
    const int last = min(kTile, sub_end - t0) - 1;  // >= 0: t0 < sub_end
    if constexpr (BIG) {
      // t0 is a multiple of 16 and so is bs: the tile lies inside one block.
      const int blk = __builtin_amdgcn_readfirstlane(tbl[(t0 >> log2_bs) - first_blk]);
      const size_t row0 = (size_t)blk * block_rows + head_rows + (t0 & (bs - 1));
      const uint4 *kt = a.k_cache + row0 * LPR;
      const uint4 *vt = a.v_cache + row0 * LPR;
      const int kofs = min(n, last) * LPR + g;
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i) T.k[i] = load_stream(kt + kofs + 4 * i);
#pragma unroll
      for (int u = 0; u < NV; ++u) T.v[u] = load_stream(vt + min(u * RPW + r, last) * LPR + c);
    } else {
      const uint4 *kt = a.k_cache + token_row(t0 + min(n, last)) * LPR + g;
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i) T.k[i] = load_stream(kt + 4 * i);
#pragma unroll
      for (int u = 0; u < NV; ++u)
        T.v[u] = load_stream(a.v_cache + token_row(t0 + min(u * RPW + r, last)) * LPR + c);
    }
  };

  // The tile holding token newpos, whose K and V rows come from the input
  // rows (row s, head kvh of a.k_new / a.v_new) instead of the pools.
  auto load_tile_new = [&](Tile &T, int t0) {
    const int last = min(kTile, sub_end - t0) - 1;
    const size_t new_row = ((size_t)s * a.num_kv_heads + kvh) * LPR;
    const int kt = t0 + min(n, last);
    const uint4 *kp = kt == newpos ? a.k_new + new_row + g : a.k_cache + token_row(kt) * LPR + g;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) T.k[i] = kp[4 * i];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int vt = t0 + min(u * RPW + r, last);
      T.v[u] = load_stream(vt == newpos ? a.v_new + new_row + c : a.v_cache + token_row(vt) * LPR + c);
    }
  };

  auto compute_tile = [&](const Tile &T, int t0) {
    const int nvalid = min(kTile, sub_end - t0);
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qop[i]),
                                                   __builtin_bit_cast(bf16x8_t, T.k[i]), sc, 0, 0, 0);
    const bool valid = n < nvalid;
    float pj[4], alpha[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float z = valid ? sc[j] * a.qscale : -INFINITY;
      const float mn = fmaxf(m[j], row16_max(z));
      alpha[j] = exp2_fast(m[j] - mn);
      m[j] = mn;
      pj[j] = exp2_fast(z - mn);
      l[j] = fmaf(l[j], alpha[j], pj[j]);
    }
    if (g < HR) sh.p[wave][n][g] = make_float4(pj[0], pj[1], pj[2], pj[3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Rescale the accumulators by each head's factor (uniform across the wave).
    float sa[G];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sa[h] = readlane_f(alpha[h & 3], 16 * (h >> 2));
      moved |= sa[h] != 1.0f;
    }
    if (moved) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= sa[h];
    }

#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float4 pp[HR];
#pragma unroll
      for (int q4 = 0; q4 < HR; ++q4) pp[q4] = sh.p[wave][u * RPW + r][q4];
      const uint4 w4 = T.v[u];
      const float vf[8] = {bf16_lo(w4.x), bf16_hi(w4.x), bf16_lo(w4.y), bf16_hi(w4.y),
                           bf16_lo(w4.z), bf16_hi(w4.z), bf16_lo(w4.w), bf16_hi(w4.w)};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 &q4 = pp[h >> 2];
        const float ph = (h & 3) == 0 ? q4.x : (h & 3) == 1 ? q4.y : (h & 3) == 2 ? q4.z : q4.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
      }
    }
    // the next tile's p must not overwrite this tile's before it is read
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  constexpr int kThr = 64 * NW;
  constexpr int kStride = NW * kTile;
  for (int sub = start; sub < end; sub = sub_end) {
    first_blk = sub >> log2_bs;
    if (tbl_cap > 0) {
      // at most tbl_cap whole blocks; later sub-ranges start on a block boundary
      sub_end = (int)min((int64_t)end, ((int64_t)first_blk + tbl_cap) << log2_bs);
      const int nblk = ((sub_end - 1) >> log2_bs) - first_blk + 1;
      for (int i = tid; i < nblk; i += kThr) {
        const int b = trow[first_blk + i];
        tbl[i] = (unsigned)b < (unsigned)a.num_blocks ? b : 0;  // stay inside the pool
      }
      __syncthreads();
    } else {
      sub_end = end;
    }
    // The tile holding newpos (the range's last: newpos = end - 1) is left
    // out of the loop and done after it by the wave whose turn it is; it is
    // that wave's last tile, so every wave's order is unchanged.
    const int new_tile = newpos >= sub && newpos < sub_end ? newpos & ~(kTile - 1) : sub_end;
    for (int t0 = sub + wave * kTile; t0 < new_tile; t0 += TPI * kStride) {
      if (share_done >= 0) set_progress_priority((float)(share_done + (t0 - start)) * share_inv);
      Tile T[TPI];
#pragma unroll
      for (int k = 0; k < TPI; ++k) {
        const int tk = t0 + k * kStride;
        load_tile(T[k], tk < new_tile ? tk : t0);  // always a valid tile; unused past the end
      }
#pragma unroll
      for (int k = 0; k < TPI; ++k) {
        const int tk = t0 + k * kStride;
        if (k == 0 || tk < new_tile) compute_tile(T[k], tk);
      }
    }
    if (new_tile < sub_end && ((new_tile - sub) / kTile) % NW == wave) {
      Tile T;
      load_tile_new(T, new_tile);
      compute_tile(T, new_tile);
    }
    if (tbl_cap > 0) __syncthreads();  // the table may be restaged next
  }

  // Wave totals: l over the 16 token lanes of each row, acc over the row groups.
#pragma unroll
  for (int j = 0; j < 4; ++j) l[j] = group_sum<16>(l[j]);
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) sh.red_acc[wave][h][c * 8 + e] = acc[h][e];
  }
  if (g < HR && n == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sh.red_m[wave][4 * g + j] = m[j];
      sh.red_l[wave][4 * g + j] = l[j];
    }
  }
  __syncthreads();
}

// Combines the waves' statistics of the range and writes, for each of the
// G query heads j: the normalised output (final: element (j, ch) at out
// index out_row + j * D + ch), or the unnormalised partial (max at
// pm[j * sm], sum at pl[j * sm], acc at po[j * so + ch]).
template <int D, int G, int NW>
__device__ __forceinline__ void gqa_finish(const DecodeArgs &a, const GqaShared<D, G, NW> &sh, size_t out_row,
                                           bool final, float *pm, float *pl, float *po, int sm, int so) {
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
    const int j = idx / D;
    const int ch = idx % D;
    float M = sh.red_m[0][j];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) M = fmaxf(M, sh.red_m[wv][j]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      const float f = exp2_fast(sh.red_m[wv][j] - M);
      L = fmaf(sh.red_l[wv][j], f, L);
      A = fmaf(sh.red_acc[wv][j][ch], f, A);
    }
    if (final) {
      const float o = L > 0.0f ? A / L : 0.0f;
      store_out<uint16_t>(a.out, out_row + (size_t)j * D + ch, o, a.out_f32);
    } else {
      po[(size_t)j * so + ch] = A;
      if (ch == 0) {
        pm[(size_t)j * sm] = M;
        pl[(size_t)j * sm] = L;
      }
    }
  }
}

// One workgroup per (sequence, KV head, partition).
template <int D, int G, bool PART, bool BIG>
__global__ __launch_bounds__(kThreads) void decode_gqa_kernel(DecodeArgs a) {
  extern __shared__ int32_t tbl[];
  __shared__ GqaShared<D, G, kWaves> sh;

  const int n_work = a.num_seqs * a.num_kv_heads * a.num_parts;
  const int w = xcd_work_id(blockIdx.x, n_work);
  const int s = w % a.num_seqs;
  const int rest = w / a.num_seqs;
  const int p = rest % a.num_parts;
  const int kvh = rest / a.num_parts;

  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_cap ? a.ctx_cap : ctx);
  const int start = p * a.partition_size;
  const int end = min(ctx, start + a.partition_size);
  if (PART && start >= end) return;  // no tokens: the merge never reads this slot

  gqa_range<D, G, BIG, kWaves>(a, sh, tbl, a.tbl_cap, s, kvh, start, end);
  const size_t head0 = (size_t)s * a.num_q_heads + (size_t)kvh * G;
  const size_t slot = head0 * a.num_parts + p;
  gqa_finish<D, G, kWaves>(a, sh, head0 * D, !PART, a.part_m + slot, a.part_l + slot, a.part_o + slot * D,
                   a.num_parts, a.num_parts * D);
}

// Every segment a workgroup takes on costs it a fixed time (its first loads
// and the reduction at its end), so each nonempty sequence's flattened length
// carries this many extra positions (no tokens) beyond its padding: shares
// with more segments hold fewer tokens.  The cost is 24 KiB of K/V (48
// positions at head size 128, 96 at 64, 32 at 256).  Measured on MI355X,
// Llama-3-8B-shaped batch, 0 / 16 / 32 / 48 / 64 / 80 / 96 positions:
// 102.7 / 102.2 / 101.5 / 100.9 / 101.1 / 101.3 / 101.6 us per call; 8 x 32k
// tokens 174.6 -> 171.7 us at 48 against 96; 256 sequences sharing a prefix
// unchanged.  (96 was best while each segment waited for its own table
// round trip and the walk over a share's segments cost more.)
template <int D>
constexpr int kSegmentCost = (24 * 1024 / (4 * D) + 15) & ~15;
static_assert(kSegmentCost<128> == 48 && kSegmentCost<64> == 96 && kSegmentCost<256> == 32, "segment cost");
// The LDS byte per sequence holds padding + cost in bits 0..6 and, in bit 7,
// whether its length was clamped (its newest token is then not attended).
constexpr int kClampedBit = 0x80;
static_assert(kSegmentCost<64> + 15 < kClampedBit, "padding must fit 7 bits");

// A piece of a balanced share: tokens [t, e) of sequence s for KV head kvh
// (e clipped to the sequence's length), seg flattened positions including
// the padding, lp the padded length, nblk the blocks holding [t, e).
struct BalSegment {
  int kvh, s, t, e, seg, lp, nblk;
};
constexpr int kMaxListedSegs = 16;

// Index of the sequence holding flattened token r: the largest s < B with
// cum[s] <= r (cum is non-decreasing, cum[0] = 0 <= r < cum[B]).
__device__ __forceinline__ int find_seq(const int32_t *cum, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The same index found by one whole wave at once: lane l tests whether
// sequence base + l is the one (cum[s] <= r < cum[s + 1]; exactly one s
// passes), 64 sequences per step.  Every lane of the wave must be active.
__device__ __forceinline__ int find_seq_wave(const int32_t *cum, int B, int r) {
  const int lane = threadIdx.x & 63;
  for (int base = 0;; base += 64) {
    const int s = base + lane;
    const uint64_t hit = __ballot(s < B && cum[s] <= r && r < cum[s + 1]);
    if (hit) return base + __builtin_ctzll(hit);
    if (base + 64 >= B) return B - 1;  // not reached while r < cum[B]
  }
}

// Balanced split: share w is flattened tokens [w chunk, (w + 1) chunk)
// of (KV head, sequence, token), every nonempty length rounded up to 16 plus
// kSegmentCost, with chunk = total / (grid size) rounded up to 16.  The grid is one wave of resident
// workgroups, one share each.  A workgroup that holds a whole sequence writes its output; the
// others write a partial (max, sum, acc) at slot w + (kvh B + s), distinct for
// every (share, sequence) pair because shares and sequences both advance
// with the flattened position.  Workgroup 0 also leaves the
// split (chunk, padded-length sum, prefix sums) in the workspace header for
// merge_balanced_kernel.
template <int D, int G, bool BIG>
__global__ __launch_bounds__(kThreads) void decode_gqa_balanced(DecodeArgs a) {
  extern __shared__ int32_t dyn[];
  __shared__ GqaShared<D, G, kWaves> sh;
  __shared__ int32_t wave_tot[kWaves];
  __shared__ int32_t carry;
  const int B = a.num_seqs;
  int32_t *cum = dyn;                         // [B + 1] prefix sums of padded lengths
  int32_t *tbl = dyn + ((B + 1 + 3) & ~3);    // [a.tbl_cap]
  uint8_t *pad = (uint8_t *)(tbl + a.tbl_cap);  // [B] padded minus clamped length, kClampedBit
  const int tid = threadIdx.x;
  // Until its tiles start, a workgroup is at 0% of its share: top priority,
  // or the waves of workgroups already streaming on the CU starve this
  // prologue (measured: 3-4x longer for workgroups with several segments).
  __builtin_amdgcn_s_setprio(3);

  // Fused write (a.k_new set): token s, the newest of sequence s, goes to
  // pool slot slot_mapping[s] for every KV head (slots < 0 or outside the
  // pool are skipped), tokens spread over the grid.  The attention below
  // reads that token from k_new / v_new, never from the pools, so nothing in
  // this kernel waits for these stores; their loads go out next to the
  // first lengths' load.
  const int ctx_first = tid < B ? a.context_lens[tid] : 0;
  if (a.k_new) {
    constexpr int kChunks = D / 8;  // 16-byte chunks per row
    const int per_tok = a.num_kv_heads * kChunks;
    for (int tok = blockIdx.x; tok < B; tok += a.num_wg) {
      const int64_t slot = a.slot_mapping[tok];
      for (int ch = tid; ch < per_tok; ch += kThreads) {
        const uint4 kv = a.k_new[(size_t)tok * per_tok + ch];
        const uint4 vv = a.v_new[(size_t)tok * per_tok + ch];
        if (slot >= 0 && slot < a.num_slots) {
          const int64_t blk = slot >> a.log2_bs;
          const int64_t off = slot & (a.block_size - 1);
          const size_t dst = ((size_t)(blk * a.num_kv_heads + ch / kChunks) * a.block_size + off) * kChunks +
                             ch % kChunks;
          const_cast<uint4 *>(a.k_cache)[dst] = kv;
          const_cast<uint4 *>(a.v_cache)[dst] = vv;
        }
      }
    }
  }

  // Lengths and the prefix sums of the padded lengths.  Up to 64 sequences
  // wave 0 scans them alone, in registers it keeps for the walk below;
  // larger batches kThreads sequences at a time.
  const bool one_wave = B <= 64;
  int my_len = 0, my_end = 0, my_pad = 0;  // one_wave, lane s of wave 0: sequence s's padded length, cum[s + 1], pad[s]
  if (one_wave) {
    if (tid < 64) {
      const int raw = ctx_first;
      const int ctx = raw < 0 ? 0 : (raw > a.ctx_cap ? a.ctx_cap : raw);
      const int v = ctx > 0 ? ((ctx + 15) & ~15) + kSegmentCost<D> : 0;
      my_pad = (v - ctx) | (raw > a.ctx_cap ? kClampedBit : 0);
      const int c = wave_incl_scan(v);
      my_len = v;
      my_end = c;
      if (tid < B) {
        pad[tid] = (uint8_t)my_pad;
        cum[tid + 1] = c;
      }
      if (tid == 0) cum[0] = 0;
    }
    __syncthreads();
  } else {
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < B; base += kThreads) {
      const int s = base + tid;
      const int raw = base == 0 ? ctx_first : (s < B ? a.context_lens[s] : 0);
      const int ctx = raw < 0 ? 0 : (raw > a.ctx_cap ? a.ctx_cap : raw);
      int v = ctx > 0 ? ((ctx + 15) & ~15) + kSegmentCost<D> : 0;
      if (s < B) pad[s] = (uint8_t)((v - ctx) | (raw > a.ctx_cap ? kClampedBit : 0));
      v = wave_incl_scan(v);  // within the wave
      if ((tid & 63) == 63) wave_tot[tid >> 6] = v;
      __syncthreads();
      int add = carry;
      for (int wv = 0; wv < (tid >> 6); ++wv) add += wave_tot[wv];
      if (s < B) cum[s + 1] = v + add;
      __syncthreads();
      if (tid == kThreads - 1) carry = v + add;
      __syncthreads();
    }
    if (tid == 0) cum[0] = 0;
    __syncthreads();
  }

  const int sigma = cum[B];
  const int64_t total = (int64_t)a.num_kv_heads * sigma;
  const int64_t chunk = ((total + a.num_wg - 1) / a.num_wg + 15) & ~(int64_t)15;
  if (blockIdx.x == 0) {
    if (tid == 0) {
      a.bal_hdr[0] = (int32_t)chunk;
      a.bal_hdr[1] = sigma;
    }
    for (int i = tid; i <= B; i += kThreads) a.bal_hdr[kBalancedHdrInts + i] = cum[i];
  }
  if (total == 0) return;

  // Workgroup L runs on XCD L % 8; it takes share xcd_work_id(L), so the
  // shares of one XCD are one contiguous range: with 8 KV heads, one XCD
  // works on one KV head's sequences.  Blocks that several sequences share
  // (a common prefix) are then read by the workgroups of one XCD at about the
  // same time and come from its L2.  Measured on MI355X, 256 sequences
  // sharing a 2048-token prefix: 250 us per copy-on-write step against 398
  // us with share L on workgroup L; unshared batches are unaffected.
  const int share = xcd_work_id(blockIdx.x, a.num_wg);
  const int64_t f0 = (int64_t)share * chunk;
  const int64_t f1 = min(total, f0 + chunk);
  // only steers wave priority: the hardware reciprocal of the share's size (< 2^31) will do
  const float share_inv = f1 > f0 ? __builtin_amdgcn_rcpf((float)(int)(f1 - f0)) : 0.0f;
  const int log2_bs = a.log2_bs;

  // The share [f0, f1) falls into segments, one per (KV head, sequence):
  // tokens [t, e) of the sequence (e clipped to its length), seg flattened
  // positions including the padding.
  const bool small = total <= 0x7fffffff;  // 32-bit division suffices
  // the segment of sequence s at flattened position f, rr = f - kvh sigma
  auto segment_of = [&](int kvh, int s, int rr, int64_t f) {
    BalSegment g;
    g.kvh = kvh;
    g.s = s;
    g.t = rr - cum[s];
    g.lp = cum[s + 1] - cum[s];
    g.seg = (int)min((int64_t)(g.lp - g.t), f1 - f);
    g.e = max(g.t, min(g.lp - (pad[s] & (kClampedBit - 1)), g.t + g.seg));
    g.nblk = g.e > g.t ? ((g.e - 1) >> log2_bs) - (g.t >> log2_bs) + 1 : 0;
    return g;
  };
  auto segment_at = [&](int64_t f, bool whole_wave) {
    const int kvh = small ? (int)f / sigma : (int)(f / sigma);
    const int rr = (int)(f - (int64_t)kvh * sigma);
    return segment_of(kvh, whole_wave ? find_seq_wave(cum, B, rr) : find_seq(cum, B, rr), rr, f);
  };
  // The segment after g, which ended with its sequence: the next sequence
  // of the same KV head, or the first of the next one.  Only a run of empty
  // sequences needs the search (the same segment as segment_at(f) either
  // way; measured on MI355X, Llama-3-8B-shaped batch: the walk over a share
  // took 1.76 us of the ~3.6 us before the first tile with a division and a
  // 6-step search in LDS per segment).
  auto segment_after = [&](const BalSegment &g, int64_t f) {
    int kvh = g.kvh, cand = g.s + 1;
    int rr = (int)(f - (int64_t)kvh * sigma);
    if (rr >= sigma) {
      kvh += 1;
      rr -= sigma;
      cand = 0;
    }
    const int s = cand < B && cum[cand] <= rr && rr < cum[cand + 1] ? cand : find_seq(cum, B, rr);
    return segment_of(kvh, s, rr, f);
  };

  // One walk over the share lists its segments (the first kMaxListedSegs)
  // and counts the block ids they need.  When the share has no more
  // segments than that and their block ids fit in tbl together, they are all
  // staged now in one pass, so that no segment after the first waits for a
  // table load; otherwise each segment is found again and stages its own.
  // Wave 0 walks alone and leaves the counts in LDS: the walk is scalar
  // work, and the CU's waves share one scalar unit while every workgroup on
  // it is in its prologue (measured on MI355X, Llama-3-8B-shaped batch: the
  // walk took 1.48 us with all four waves walking).
  __shared__ BalSegment segs[kMaxListedSegs];
  __shared__ int seg_off[kMaxListedSegs + 1];  // staged position of each listed segment's first block id
  __shared__ int walk_count[2];                // segments, block ids
  if (tid < 64) {
    bool walked = false;
    if (one_wave) {
      // Every segment at once: lane j takes the j-th (KV head, sequence)
      // pair from the share's first on, in the flattened order; the
      // nonempty pairs that start before f1 are the share's segments, in
      // lane order, the same as the walk below finds one after another.  A
      // share that reaches past 64 pairs walks instead.
      const int kvh0 = small ? (int)f0 / sigma : (int)(f0 / sigma);
      const int rr0 = (int)(f0 - (int64_t)kvh0 * sigma);
      // exactly one sequence holds rr0 (0 <= rr0 < sigma); the guard only keeps ctz defined
      const uint64_t at0 = __ballot(tid < B && my_end - my_len <= rr0 && rr0 < my_end);
      const int s0 = at0 ? __builtin_ctzll(at0) : 0;
      const int q = s0 + tid, qk = q / B, sq = q - qk * B;
      const int kvh = kvh0 + qk;
      const int lp = __shfl(my_len, sq, 64);
      const int c0 = __shfl(my_end - my_len, sq, 64);
      const int pd = __shfl(my_pad, sq, 64);
      const int t = tid == 0 ? rr0 - c0 : 0;
      const int64_t fpos = (int64_t)kvh * sigma + c0 + t;
      const bool valid = lp > 0 && fpos < f1;
      if (!(__ballot(fpos < f1) >> 63)) {  // lane 63's pair starts at or past f1
        BalSegment g;
        g.kvh = kvh;
        g.s = sq;
        g.t = t;
        g.lp = lp;
        g.seg = (int)min((int64_t)(lp - t), f1 - fpos);
        g.e = max(t, min(lp - (pd & (kClampedBit - 1)), t + g.seg));
        g.nblk = valid && g.e > t ? ((g.e - 1) >> log2_bs) - (t >> log2_bs) + 1 : 0;
        const uint64_t vb = __ballot(valid);
        const int idx = __popcll(vb & ((1ull << tid) - 1));
        const int upto = wave_incl_scan(g.nblk);  // block ids of this lane's segment and the ones before it
        if (valid && idx < kMaxListedSegs) {
          segs[idx] = g;
          seg_off[idx] = upto - g.nblk;
        }
        const int nseg = __popcll(vb), need = __shfl(upto, 63, 64);
        if (tid == 0) {
          walk_count[0] = nseg;
          walk_count[1] = need;
          if (nseg <= kMaxListedSegs) seg_off[nseg] = need;
        }
        walked = true;
      }
    }
    if (!walked) {
      int nseg = 0, need = 0;
      BalSegment g;
      for (int64_t f = f0; f < f1; ++nseg) {
        g = nseg == 0 ? segment_at(f, true) : segment_after(g, f);
        if (tid == 0 && nseg < kMaxListedSegs) {
          segs[nseg] = g;
          seg_off[nseg] = need;
        }
        need += g.nblk;
        f += g.seg;
      }
      if (tid == 0) {
        walk_count[0] = nseg;
        walk_count[1] = need;
        if (nseg <= kMaxListedSegs) seg_off[nseg] = need;
      }
    }
  }
  __syncthreads();
  const int nseg = walk_count[0], need = walk_count[1];
  const bool listed = nseg <= kMaxListedSegs;
  const bool staged = listed && need <= a.tbl_cap;
  if (staged) {
    // Every listed segment's block ids in one pass: each thread issues the
    // loads of up to kStageBatch ids (of any segments) before storing any,
    // so the whole share costs one table round trip, not one per segment
    // (measured on MI355X, Llama-3-8B-shaped batch: a workgroup placed on a
    // CU whose other workgroups already stream waited up to ~25 us for its
    // first tile with one round trip per segment, ~12 us with one in all).
    constexpr int kStageBatch = 4;
    for (int base = 0; base < need; base += kThreads * kStageBatch) {
      int ids[kStageBatch];
#pragma unroll
      for (int k = 0; k < kStageBatch; ++k) {
        const int fi = base + tid + k * kThreads;
        ids[k] = 0;
        if (fi < need) {
          int i = 0;
          while (fi >= seg_off[i + 1]) ++i;
          const BalSegment &g = segs[i];
          ids[k] = a.block_tables[(size_t)g.s * a.max_blocks + (g.t >> log2_bs) + (fi - seg_off[i])];
        }
      }
#pragma unroll
      for (int k = 0; k < kStageBatch; ++k) {
        const int fi = base + tid + k * kThreads;
        if (fi < need) tbl[fi] = (unsigned)ids[k] < (unsigned)a.num_blocks ? ids[k] : 0;  // stay inside the pool
      }
    }
    __syncthreads();
  }

  int off = 0;
  int64_t f = f0;
  for (int i = 0; f < f1; ++i) {
    const BalSegment g = listed ? segs[i] : segment_at(f, false);
    const int s = g.s, kvh = g.kvh, t = g.t, e = g.e, seg = g.seg;
    f += seg;
    const int ctx = g.lp - (pad[s] & (kClampedBit - 1));
    if (t >= ctx) continue;  // padding and segment cost only: no piece
    // with the fused write, the newest token (position ctx - 1 unless the
    // length was clamped) comes from the input rows
    const int newpos = a.k_new && e == ctx && !(pad[s] & kClampedBit) ? ctx - 1 : -1;
    gqa_range<D, G, BIG, kWaves>(a, sh, staged ? tbl + off : tbl, staged ? 0 : a.tbl_cap, s, kvh, t, e,
                                 (int)(f - seg - f0), share_inv, newpos);
    off += g.nblk;
    const bool final = t == 0 && e == ctx;
    const size_t slot = ((size_t)share + (size_t)kvh * B + s) * G;
    const size_t head0 = (size_t)s * a.num_q_heads + (size_t)kvh * G;
    gqa_finish<D, G, kWaves>(a, sh, head0 * D, final, a.part_m + slot, a.part_l + slot, a.part_o + slot * D,
                             1, D);
    __syncthreads();  // sh is reused by the next segment
  }
}

// Combines the pieces of each sequence that the balanced split cut between
// workgroups; one workgroup per (sequence, KV head).  The holders are the
// workgroups whose shares meet the sequence's tokens (not its padding).
template <int D, int G>
__global__ __launch_bounds__(kThreads) void merge_balanced_kernel(DecodeArgs a) {
  const int B = a.num_seqs;
  const int s = blockIdx.x % B;
  const int kvh = blockIdx.x / B;
  const int32_t *cum = a.bal_hdr + kBalancedHdrInts;
  const int64_t chunk = a.bal_hdr[0];
  const int sigma = a.bal_hdr[1];
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_cap ? a.ctx_cap : ctx);
  const size_t head0 = (size_t)s * a.num_q_heads + (size_t)kvh * G;
  if (ctx == 0) {  // empty sequence: zeros
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
      store_out<uint16_t>(a.out, head0 * D + idx, 0.0f, a.out_f32);
    return;
  }
  const int64_t first = (int64_t)kvh * sigma + cum[s];
  const int64_t w1 = first / chunk;
  const int64_t w2 = (first + ctx - 1) / chunk;
  if (w1 == w2) return;  // one workgroup held the whole sequence and wrote it
  const size_t pair = (size_t)kvh * B + s;
  // A thread owns E of the G * D outputs (elements tid + k kThreads).  The
  // loads of kBatch pieces for all E elements are issued together, then
  // folded into running (max, sum, acc) in piece order: one round trip per
  // kBatch pieces, whatever E is.  kBatch is 16 when a sequence has more than
  // 8 pieces, else 4 (loads of 16 for a sequence of few pieces cost more than
  // the round trips they save; measured on MI355X, 8 x 32k tokens, ~12
  // pieces each: 177.9 -> 175.7 us per call).  The fold order, and so the
  // result, is the same for both.
  constexpr int E = (G * D + kThreads - 1) / kThreads;
  float M[E], L[E], A[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    M[k] = kNegBig;
    L[k] = 0.0f;
    A[k] = 0.0f;
  }
  auto fold_all = [&](auto batch_tag) {
    constexpr int kBatch = decltype(batch_tag)::value;
    for (int64_t w0 = w1; w0 <= w2; w0 += kBatch) {
      float pm[kBatch][E], pl_[kBatch][E], po[kBatch][E];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t w = w0 + u <= w2 ? w0 + u : w2;  // repeats are masked below
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const int idx = min((int)threadIdx.x + k * kThreads, G * D - 1);  // past the end: unused
          const size_t slot = (w + pair) * G + idx / D;
          pm[u][k] = a.part_m[slot];
          pl_[u][k] = a.part_l[slot];
          po[u][k] = a.part_o[slot * D + idx % D];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (w0 + u <= w2) {
#pragma unroll
          for (int k = 0; k < E; ++k) {
            const float mn = fmaxf(M[k], pm[u][k]);
            const float f0 = exp2_fast(M[k] - mn), f1 = exp2_fast(pm[u][k] - mn);
            L[k] = L[k] * f0 + pl_[u][k] * f1;
            A[k] = A[k] * f0 + po[u][k] * f1;
            M[k] = mn;
          }
        }
      }
    }
  };
  if (w2 - w1 >= 8)
    fold_all(std::integral_constant<int, 16>{});
  else
    fold_all(std::integral_constant<int, 4>{});
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int idx = threadIdx.x + k * kThreads;
    if (idx < G * D) store_out<uint16_t>(a.out, head0 * D + idx, L[k] > 0.0f ? A[k] / L[k] : 0.0f, a.out_f32);
  }
}

// Launch limits of one balanced-kernel instance on the current device: the
// workgroups that fit on it at once for a given dynamic LDS size, and the
// dynamic LDS a workgroup may take.  Queried once per (instance, device, LDS
// size) and kept, each device's entry in one atomic word (callers on several
// threads see either no entry or a whole one).
template <int D, int G, bool BIG>
struct BalancedLimits {
  static int resident(int dev, size_t dyn_lds) {
    static std::atomic<uint64_t> cache[64];  // [device] -> (dyn_lds + 1) << 32 | workgroups
    const uint64_t key = (uint64_t)(dyn_lds + 1) << 32;
    const uint64_t hit = cache[dev].load(std::memory_order_relaxed);
    if ((hit & ~0xffffffffull) == key) return (int)(hit & 0xffffffffull);
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_gqa_balanced<D, G, BIG>, kThreads,
                                                     dyn_lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return kBalancedMaxWorkgroups;
    int n = per_cu * cus;
    n = n < 1 ? 1 : (n > kBalancedMaxWorkgroups ? kBalancedMaxWorkgroups : n);
    cache[dev].store(key | (uint32_t)n, std::memory_order_relaxed);
    return n;
  }
  static size_t max_dyn_lds(int dev) {
    static std::atomic<size_t> cache[64];
    const size_t hit = cache[dev].load(std::memory_order_relaxed);
    if (hit) return hit;
    int max_lds = 0;
    hipFuncAttributes fa{};
    if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(decode_gqa_balanced<D, G, BIG>)) !=
            hipSuccess)
      return 64 * 1024 - 36 * 1024;  // the 64 KiB floor minus the largest static share
    const size_t v = max_lds > (int)fa.sharedSizeBytes ? (size_t)max_lds - fa.sharedSizeBytes : 1;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
  }
};

template <int D, int G, bool BIG>
hipError_t launch_dgb(const DecodeArgs &a0, int mode, hipStream_t st) {
  DecodeArgs a = a0;
  if (mode == kModeBalanced) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    // dynamic LDS: prefix sums [B + 1] and block ids [tbl_cap] (int32), then
    // one padding byte per sequence.  Fewer staged block ids when that would
    // not fit, kept a multiple of 16 so that sub-ranges end on a tile.
    const size_t fixed = (size_t)((a.num_seqs + 1 + 3) & ~3) * sizeof(int32_t) + ((a.num_seqs + 3) & ~3);
    const size_t cap = BalancedLimits<D, G, BIG>::max_dyn_lds(dev);
    if (fixed + kTile * sizeof(int32_t) > cap) return hipErrorInvalidConfiguration;
    const size_t fit = ((cap - fixed) / sizeof(int32_t)) & ~(size_t)(kTile - 1);
    if ((size_t)a.tbl_cap > fit) a.tbl_cap = (int32_t)fit;
    const size_t lds = fixed + (size_t)a.tbl_cap * sizeof(int32_t);
    a.num_wg = BalancedLimits<D, G, BIG>::resident(dev, lds);
    hipLaunchKernelGGL((decode_gqa_balanced<D, G, BIG>), dim3(a.num_wg), dim3(kThreads), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((merge_balanced_kernel<D, G>), dim3(a.num_seqs * a.num_kv_heads), dim3(kThreads), 0,
                       st, a);
    return hipGetLastError();
  }
  const int n_work = a.num_seqs * a.num_kv_heads * a.num_parts;
  const size_t lds = (size_t)a.tbl_cap * sizeof(int32_t);
  if (mode == kModePartitioned)
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, true, BIG>), dim3(n_work), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, false, BIG>), dim3(n_work), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs &a, int mode, hipStream_t st) {
  return a.block_size >= kTile ? launch_dgb<D, G, true>(a, mode, st) : launch_dgb<D, G, false>(a, mode, st);
}

template <int D>
hipError_t launch_d(int group, const DecodeArgs &a, int mode, hipStream_t st) {
  switch (group) {
    case 4: return launch_dg<D, 4>(a, mode, st);
    case 8: return launch_dg<D, 8>(a, mode, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_gqa(int head_dim, int group, const DecodeArgs &a, int mode, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_d<64>(group, a, mode, st);
    case 128: return launch_d<128>(group, a, mode, st);
    case 256: return launch_d<256>(group, a, mode, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
