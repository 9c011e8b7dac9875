// q4v_select.h -- device helpers of top-k selection shared by the sampling
// epilogue and the LM-head GEMM's fused epilogue (internal, not ABI).
//
// Candidate order: larger logit first, equal logits by smaller token index,
// folded into one 64-bit key, larger = better:
//   key = orderable(logit bits) << 32 | (0xFFFFFFFF - token)
// where orderable() maps IEEE order onto unsigned order (-0 is keyed as +0,
// so the two zeros tie).  Key 0 means "no candidate".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4v {
namespace {

__device__ __forceinline__ uint64_t make_key(float v, uint32_t token) {
  // -0 and +0 are equal logits: both take the key of +0, so that they tie
  // and the smaller token index comes first
  uint32_t b = v == 0.0f ? 0u : __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(b) << 32) | (0xFFFFFFFFu - token);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t b = static_cast<uint32_t>(key >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return __uint_as_float(b);
}

__device__ __forceinline__ uint32_t key_token(uint64_t key) {
  return 0xFFFFFFFFu - static_cast<uint32_t>(key);
}

// Cross-lane exchange with the lane l ^ J, without LDS: DPP for J <= 8
// (quad permutes and row mirrors: J = 4 is a half-row mirror followed by a
// quad reversal, J = 8 a row mirror followed by a half-row mirror), the
// gfx950 permlane swaps for J = 16 and 32.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
  constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kQuadRev = 0x1B;
  constexpr int kRowMirror = 0x140, kRowHalfMirror = 0x141;
  if constexpr (J == 1) {
    return __builtin_amdgcn_update_dpp(0u, v, kQuadXor1, 0xF, 0xF, false);
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_update_dpp(0u, v, kQuadXor2, 0xF, 0xF, false);
  } else if constexpr (J == 4) {
    const uint32_t t = __builtin_amdgcn_update_dpp(0u, v, kRowHalfMirror, 0xF, 0xF, false);
    return __builtin_amdgcn_update_dpp(0u, t, kQuadRev, 0xF, 0xF, false);
  } else if constexpr (J == 8) {
    const uint32_t t = __builtin_amdgcn_update_dpp(0u, v, kRowMirror, 0xF, 0xF, false);
    return __builtin_amdgcn_update_dpp(0u, t, kRowHalfMirror, 0xF, 0xF, false);
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "xor distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int lane) {
  const uint32_t lo = xor_lane<J>(static_cast<uint32_t>(v), lane);
  const uint32_t hi = xor_lane<J>(static_cast<uint32_t>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One compare-exchange stage of a bitonic network: lanes keep the larger
// key when keep_max, else the smaller.
template <int J>
__device__ __forceinline__ uint64_t cx_stage(uint64_t key, bool keep_max, int lane) {
  const uint64_t other = xor_lane64<J>(key, lane);
  const uint64_t hi = key > other ? key : other;
  const uint64_t lo = key > other ? other : key;
  return keep_max ? hi : lo;
}

template <int J>
__device__ __forceinline__ uint32_t cx_stage32(uint32_t v, bool keep_max, int lane) {
  const uint32_t other = xor_lane<J>(v, lane);
  return keep_max ? (v > other ? v : other) : (v > other ? other : v);
}

__device__ __forceinline__ uint32_t half_cleaner_desc32(uint32_t v, int lane) {
  v = cx_stage32<32>(v, (lane & 32) == 0, lane);
  v = cx_stage32<16>(v, (lane & 16) == 0, lane);
  v = cx_stage32<8>(v, (lane & 8) == 0, lane);
  v = cx_stage32<4>(v, (lane & 4) == 0, lane);
  v = cx_stage32<2>(v, (lane & 2) == 0, lane);
  v = cx_stage32<1>(v, (lane & 1) == 0, lane);
  return v;
}

template <int K, int J>
__device__ __forceinline__ uint32_t sort_stages32(uint32_t v, int lane) {
  const bool desc_block = K == 64 || (lane & K) == 0;
  v = cx_stage32<J>(v, ((lane & J) == 0) == desc_block, lane);
  if constexpr (J > 1) v = sort_stages32<K, J / 2>(v, lane);
  return v;
}

// Sort 64 values (one per lane) descending.
__device__ __forceinline__ uint32_t sort64_desc32(uint32_t v, int lane) {
  v = sort_stages32<2, 1>(v, lane);
  v = sort_stages32<4, 2>(v, lane);
  v = sort_stages32<8, 4>(v, lane);
  v = sort_stages32<16, 8>(v, lane);
  v = sort_stages32<32, 16>(v, lane);
  v = sort_stages32<64, 32>(v, lane);
  return v;
}

// Sort a bitonic sequence of 64 keys (one per lane) descending.
__device__ __forceinline__ uint64_t half_cleaner_desc(uint64_t key, int lane) {
  key = cx_stage<32>(key, (lane & 32) == 0, lane);
  key = cx_stage<16>(key, (lane & 16) == 0, lane);
  key = cx_stage<8>(key, (lane & 8) == 0, lane);
  key = cx_stage<4>(key, (lane & 4) == 0, lane);
  key = cx_stage<2>(key, (lane & 2) == 0, lane);
  key = cx_stage<1>(key, (lane & 1) == 0, lane);
  return key;
}

// Stages j = J, J/2, .., 1 of the merge of blocks of size K.
template <int K, int J>
__device__ __forceinline__ uint64_t sort_stages(uint64_t key, int lane) {
  const bool desc_block = K == 64 || (lane & K) == 0;
  key = cx_stage<J>(key, ((lane & J) == 0) == desc_block, lane);
  if constexpr (J > 1) key = sort_stages<K, J / 2>(key, lane);
  return key;
}

// Sort 64 keys (one per lane) descending: a bitonic network of 21 stages.
__device__ __forceinline__ uint64_t sort64_desc(uint64_t key, int lane) {
  key = sort_stages<2, 1>(key, lane);
  key = sort_stages<4, 2>(key, lane);
  key = sort_stages<8, 4>(key, lane);
  key = sort_stages<16, 8>(key, lane);
  key = sort_stages<32, 16>(key, lane);
  key = sort_stages<64, 32>(key, lane);
  return key;
}

}  // namespace
}  // namespace q4v

namespace q4v {
namespace {

// The k-th largest (1 <= k <= 64) of the wave's 64 keys v (one per lane):
// the largest T with at least k lanes at or above it, found bit by bit
// (ballots, no cross-lane data movement), on the upper halves first and on
// the lower halves only when several lanes tie on the upper half at the
// bound.  Wave-uniform result.
__device__ __forceinline__ uint64_t wave_kth_largest(uint64_t v, int k) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32);
  const uint32_t lo = static_cast<uint32_t>(v);
  uint32_t th = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = th | (1u << b);
    if (__builtin_popcountll(__ballot(hi >= c)) >= k) th = c;
  }
  const uint64_t eq = __ballot(hi == th);
  if (__builtin_popcountll(eq) == 1)  // the bound is that lane's key
    return (static_cast<uint64_t>(th) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(
               static_cast<int>(lo), __builtin_ctzll(eq)));
  const int r = k - __builtin_popcountll(__ballot(hi > th));
  uint32_t tl = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = tl | (1u << b);
    if (__builtin_popcountll(__ballot(hi == th && lo >= c)) >= r) tl = c;
  }
  return (static_cast<uint64_t>(th) << 32) | tl;
}

// Append the keys with keep set to area[*n ..] (in lane order) and advance
// *n (wave-uniform), with no branch around the store: lanes without a key
// write *dummy, or, when dummy is NULL, the slots after the kept keys,
// area[*n + kept .. *n + 64) (the caller's area then has room for 64 slots
// past any count it can reach; later appends overwrite them).
__device__ __forceinline__ void wave_append(uint64_t key, bool keep,
                                            uint64_t *area, uint32_t *n,
                                            uint64_t *dummy) {
  const uint64_t b = __ballot(keep);
  const uint32_t below = __builtin_amdgcn_mbcnt_hi(
      static_cast<uint32_t>(b >> 32),
      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u));
  const uint32_t kept = static_cast<uint32_t>(__builtin_popcountll(b));
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  uint64_t *dst = keep ? area + *n + below
                       : (dummy != nullptr ? dummy : area + *n + kept + (lane - below));
  *dst = key;
  *n += kept;
}

// Best 32 of the n keys at area[0..n) (lanes 0..31 of the result,
// descending): sorted 64 at a time with bitonic networks, each block merged
// into the running list.
__device__ __forceinline__ uint64_t wave_best32_of(const uint64_t *area,
                                                   uint32_t n, int lane) {
  uint64_t list = 0;
  for (uint32_t b0 = 0; b0 < n; b0 += 64) {
    const uint64_t k = sort64_desc(b0 + lane < n ? area[b0 + lane] : 0, lane);
    if (b0 == 0) {
      list = k;
    } else {
      const uint64_t rev = __shfl(k, 63 - lane, 64);
      list = half_cleaner_desc(lane < 32 ? list : rev, lane);
    }
  }
  return list;
}

// The best 32 of the n <= 64 distinct keys at area[0..n) by rank: lane l
// holds key l and counts the keys above it, reading 8 keys per step (every
// lane the same addresses); the key of rank r < 32 goes to out[r], and
// slots n .. 31 of out are zeroed when n < 32.  area must have 8 slots past
// n (they are zeroed here).
__device__ __forceinline__ void wave_rank_top32(uint64_t *area, uint32_t n,
                                                uint64_t *out, int lane) {
  if (lane < 8) area[n + lane] = 0;  // zero keys rank below every key
  const uint64_t mine = static_cast<uint32_t>(lane) < n ? area[lane] : 0;
  uint32_t rank = 0;
  for (uint32_t j = 0; j < n; j += 8) {
    uint64_t k[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = area[j + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) rank += k[i] > mine ? 1u : 0u;
  }
  if (static_cast<uint32_t>(lane) < n && rank < 32) out[rank] = mine;
  if (static_cast<uint32_t>(lane) >= n && lane < 32) out[lane] = 0;
}

// The best 32 of n keys at area[0..n) into out[0..32), descending: by rank
// when n <= 64 (area then needs 8 slots past n), else with bitonic
// networks.
__device__ __forceinline__ void wave_top32(uint64_t *area, uint32_t n,
                                           uint64_t *out, int lane) {
  if (n <= 64) {
    wave_rank_top32(area, n, out, lane);
  } else {
    const uint64_t list = wave_best32_of(area, n, lane);
    if (lane < 32) out[lane] = list;
  }
}

}  // namespace
}  // namespace q4v
