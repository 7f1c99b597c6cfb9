// Shared pieces of the two decode kernels (gfx950): launch arguments and
// small device helpers.  Internal to libpagedkv.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

constexpr int kWaves = 4;                    // wave64s per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;          // running-max start; finite keeps exp2 defined
constexpr int kMaxTableLds = 4096;           // staged block ids per workgroup (16 KiB)

// How pa_decode cuts each (sequence, KV head) context into workgroup ranges.
constexpr int kModeUnpartitioned = 0;        // one range per (sequence, KV head)
constexpr int kModePartitioned = 1;          // ranges of partition_size tokens, then a merge
constexpr int kModeBalanced = 2;             // equal shares of all work, then a merge
constexpr int kBalancedHdrInts = 64;         // workspace header ints before the prefix sums
constexpr int kBalancedMaxWorkgroups = 2048; // grid bound of the balanced split
constexpr int kBalancedMaxSeqs = 8192;       // sequences whose prefix sums fit in LDS

struct DecodeArgs {
  const uint4 *q;
  const uint4 *k_cache;
  const uint4 *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  void *out;
  float *part_m;   // partitioned: [B][Hq][NP]; balanced: [slots][G]
  float *part_l;   // same shape as part_m
  float *part_o;   // partitioned: [B][Hq][NP][D]; balanced: [slots][G][D]
  int32_t *bal_hdr;  // balanced: {chunk, sum of padded lengths, ...}, then [B + 1] prefix sums
  const uint4 *k_new;           // fused write: [B][Hkv][D] newest token of each sequence (or NULL)
  const uint4 *v_new;           // fused write: same shape as k_new
  const int64_t *slot_mapping;  // fused write: [B] pool slot of each sequence's newest token
  int64_t num_slots;            // fused write: num_blocks * block_size
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t log2_bs;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t partition_size;  // tokens per partition (unpartitioned: >= every length)
  int32_t num_parts;       // partitions per (sequence, KV head) in the grid
  int32_t ctx_cap;         // lengths are clamped to this
  int32_t tbl_cap;         // block ids a workgroup stages in LDS at a time
  int32_t num_wg;          // balanced: grid size
  int32_t out_f32;         // 1: fp32 output, 0: cache element type
  float qscale;            // scale * log2(e)
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 pattern, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load marked non-temporal: K/V rows are read once per call, so they
// are streamed instead of being kept in L2 / the Infinity Cache (measured on
// MI355X: ~7.1 TB/s for streaming reads this way vs ~6.2 TB/s cached).
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (the other quad of an 8-lane half row), row_mirror (the
// other half of a 16-lane row).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of LPR lanes; every lane of a group gets the same
// value (each step adds a partner's value; a + b == b + a exactly).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPR >= 2) x += dpp_mov<kDppXor1>(x);
  if constexpr (LPR >= 4) x += dpp_mov<kDppXor2>(x);
  if constexpr (LPR >= 8) x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp_mov<kDppRowMirror>(x);
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (LPR >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Maximum over each 16-lane row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<kDppXor1>(x));
  x = fmaxf(x, dpp_mov<kDppXor2>(x));
  x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_mov<kDppRowMirror>(x));
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave, all lanes active: within
// each 16-lane row by shifts of 1, 2, 4 and 8 (lanes shifted in from outside
// the row add 0), then row 0's total into rows 1 and 3 and rows 0-1's into
// rows 2 and 3 (row_bcast:15 and row_bcast:31).  Six DPP adds, no LDS
// round trip (checked lane by lane against a host prefix sum on MI355X).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup L runs on
// XCD L % 8).  Renumber so that every XCD receives one contiguous range of
// work ids: neighbouring work (same KV head, same partition) shares an L2.
__device__ __forceinline__ int xcd_work_id(int L, int N) {
  int xcd = L & 7, idx = L >> 3;
  int q = N >> 3, r = N & 7;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

template <typename E>
__device__ __forceinline__ void store_out(void *out, size_t idx, float x, int out_f32) {
  if (out_f32 || sizeof(E) == 4)
    static_cast<float *>(out)[idx] = x;
  else
    static_cast<uint16_t *>(out)[idx] = to_bf16(x);
}

// Query heads per KV head served by the MFMA kernel (bf16 caches only).
__host__ __device__ constexpr bool gqa_mfma_supported(int group, int head_dim) {
  return (group == 4 || group == 8) && (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

// Launches the grouped-query MFMA kernels of pa_decode for bf16 pools (mode:
// kMode*; in the partitioned mode the caller then launches the merge);
// defined in pa_decode_gqa.hip.
hipError_t launch_decode_gqa(int head_dim, int group, const DecodeArgs &a, int mode, hipStream_t st);

}  // namespace pa
