// q4verify_sample.hip -- gfx950 kernels of the verify step's sampling
// epilogue and its C-ABI entry point.
//
// After the LM head has produced the logits of the M verify rows, each row
// needs its top_k (<= 32) candidates, the target probabilities over them
// (temperature, top-p prefix, renormalised), the accept test u q(d) < p(d)
// of the drafted token and, on rejection, a draw from the residual
// max(p - q, 0) (Splash engine article, section "Exact, up to top-32";
// qwen-spec page, the fused sampling kernel and the sampling paragraph).
//
// Candidate order: larger logit first, equal logits by smaller token index.
// Both are folded into one 64-bit key, larger = better:
//   key = orderable(logit bits) << 32 | (0xFFFFFFFF - token)
// where orderable() maps IEEE order onto unsigned order (-0 is keyed as +0,
// so the two zeros tie; a candidate's reported logit is then +0).  Two kernels:
//  1. topk_slices_kernel: workgroup (slice of 16384 columns, row) of 16
//     waves, 16 keys per lane in registers.  A wave sorts its 64 lane maxima;
//     the 32nd of them, kw, is at most the wave's 32nd best key (32 distinct
//     keys are >= it), so only keys >= kw can be among its best 32 (usually
//     a few more than 32 are): they are packed into LDS and sorted.  The 16
//     waves' lists are merged pairwise through LDS (a list and another
//     reversed form a bitonic sequence that one half-cleaner cascade sorts)
//     and the slice's best 32 written out.  Every compare-exchange stage
//     swaps lanes with DPP or the gfx950 permlane swaps, not through LDS.
//  2. sample_rows_kernel: one workgroup per row merges the slices' lists the
//     same way and writes the top_k candidates; then lane i of wave 0 takes
//     candidate i and the probabilities, the accept test and the residual
//     draw are evaluated in fp32 with wave reductions, lane scans and
//     ballots over the candidates in order.

#include <hip/hip_runtime.h>

#include "q4v_internal.h"

namespace q4v {
namespace {

constexpr int kTopMax = 32;
constexpr int kDraftMax = 16;
constexpr int kSliceCols = 16384;  // columns per workgroup of kernel 1

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

// Sum over the wave (a fixed butterfly order, so repeatable).
__device__ __forceinline__ float wave_sum(float x) {
  const int lane = threadIdx.x & 63;
  x += __uint_as_float(xor_lane<32>(__float_as_uint(x), lane));
  x += __uint_as_float(xor_lane<16>(__float_as_uint(x), lane));
  x += __uint_as_float(xor_lane<8>(__float_as_uint(x), lane));
  x += __uint_as_float(xor_lane<4>(__float_as_uint(x), lane));
  x += __uint_as_float(xor_lane<2>(__float_as_uint(x), lane));
  x += __uint_as_float(xor_lane<1>(__float_as_uint(x), lane));
  return x;
}

// Inclusive prefix sum over lanes 0..l.
__device__ __forceinline__ float lane_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 1; j < 64; j <<= 1) {
    const float y = __shfl_up(x, j, 64);
    if (lane >= j) x += y;
  }
  return x;
}

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kColsPerThread = kSliceCols / kThreads;  // 16
// survivor pool of a workgroup: every key it holds (kernel 1: its slice;
// the row kernel: the 32 candidates of each of up to 512 slices)
constexpr int kPoolKeys = kColsPerThread * kThreads;
static_assert(static_cast<int64_t>(Q4_SAMPLE_MAX_VOCAB) <=
                  static_cast<int64_t>(kPoolKeys / kTopMax) * kSliceCols,
              "the row kernel's pool holds every slice's candidates");

// Lanes 0..31: a descending list; merge the descending list `other` (lanes
// 0..31, read through get(i)) into it: the list and the other list reversed
// form a bitonic sequence of 64, which one half-cleaner cascade sorts.
template <typename Get>
__device__ __forceinline__ uint64_t merge_list(uint64_t list, Get get, int lane) {
  const uint64_t key = lane < kTopMax ? list : get(63 - lane);
  return half_cleaner_desc(key, lane);
}

// Merge the waves' lists (lanes 0..31) pairwise through LDS; wave 0
// returns with the best 32.
__device__ __forceinline__ uint64_t block_merge(uint64_t list,
                                                uint64_t (*lists)[kTopMax],
                                                int wave, int lane) {
#pragma unroll
  for (int stride = 1; stride < kWaves; stride <<= 1) {
    if (lane < kTopMax) lists[wave][lane] = list;
    __syncthreads();
    if ((wave & (2 * stride - 1)) == 0) {
      const uint64_t *o = lists[wave + stride];
      list = merge_list(list, [&](int i) { return o[i]; }, lane);
    }
    __syncthreads();
  }
  return list;
}

// LDS of block_best32.
struct SelectLds {
  uint32_t vals[kWaves][kTopMax];  // the waves' best 32 thread maxima
  uint64_t lists[kWaves][kTopMax];
  uint32_t threshold, count;
};

// Best 32 of the keys a workgroup holds, descending in lanes 0..31 of wave
// 0 (the other waves return 0).  for_each(f) calls f(key) for every key of
// the calling thread (0 = none), in a fixed order, twice.  The 32nd largest
// upper half T among the 1024 thread maxima bounds the 32nd best key from
// below (32 distinct keys reach it), so only keys with an upper half >= T
// can be in the answer -- usually a few more than 32.  T comes from one
// 32-bit sort per wave and a merge of the waves' lists; the survivors are
// packed into `pool` (room for every key) and sorted 64 at a time: by wave 0
// alone when at most 64 survive, else by all waves, merged through LDS.
template <typename ForEach>
__device__ __forceinline__ uint64_t block_best32(ForEach for_each, uint64_t *pool,
                                                 SelectLds &sh, int wave, int lane) {
  uint64_t tmax = 0;
  for_each([&](uint64_t k) { tmax = k > tmax ? k : tmax; });
  uint32_t v = sort64_desc32(static_cast<uint32_t>(tmax >> 32), lane);
  if (threadIdx.x == 0) sh.count = 0;
#pragma unroll
  for (int stride = 1; stride < kWaves; stride <<= 1) {
    if (lane < kTopMax) sh.vals[wave][lane] = v;
    __syncthreads();
    if ((wave & (2 * stride - 1)) == 0)
      v = half_cleaner_desc32(lane < kTopMax ? v : sh.vals[wave + stride][63 - lane], lane);
    __syncthreads();
  }
  if (threadIdx.x == kTopMax - 1) sh.threshold = v;
  __syncthreads();
  const uint32_t T = sh.threshold;
  for_each([&](uint64_t k) {
    if (k != 0 && static_cast<uint32_t>(k >> 32) >= T) pool[atomicAdd(&sh.count, 1u)] = k;
  });
  __syncthreads();
  const uint32_t n = sh.count;
  if (n <= 64) {
    if (wave != 0) return 0;
    return sort64_desc(lane < static_cast<int>(n) ? pool[lane] : 0, lane);
  }
  uint64_t list = 0;
  for (uint32_t b = 64 * wave; b < n; b += 64 * kWaves) {
    const uint64_t k = sort64_desc(b + lane < n ? pool[b + lane] : 0, lane);
    const uint64_t rev = __shfl(k, 63 - lane, 64);
    list = half_cleaner_desc(lane < kTopMax ? list : rev, lane);
  }
  list = block_merge(list, sh.lists, wave, lane);
  return wave == 0 ? list : 0;
}

// Kernel 1: workgroup (s, m) takes columns [V s / S, V (s+1) / S) of row m,
// at most 16384: 16 per thread, in registers.
__global__ __launch_bounds__(kThreads) void topk_slices_kernel(
    const float *__restrict__ logits, int64_t V, int S,
    uint64_t *__restrict__ cand) {
  __shared__ uint64_t pool[kColsPerThread * kThreads];
  __shared__ SelectLds sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int s = blockIdx.x;
  const int m = blockIdx.y;
  const int64_t c0 = V * s / S;
  const int64_t c1 = V * (s + 1) / S;
  const float *row = logits + static_cast<uint64_t>(m) * V;
  uint64_t key[kColsPerThread];
#pragma unroll
  for (int i = 0; i < kColsPerThread; ++i) {
    const int64_t col = c0 + i * kThreads + threadIdx.x;
    key[i] = col < c1 ? make_key(row[col], static_cast<uint32_t>(col)) : 0;
  }
  auto for_each = [&](auto f) {
#pragma unroll
    for (int i = 0; i < kColsPerThread; ++i) f(key[i]);
  };
  const uint64_t list = block_best32(for_each, pool, sh, wave, lane);
  if (wave == 0 && lane < kTopMax)
    cand[(static_cast<uint64_t>(m) * S + s) * kTopMax + lane] = list;
}

struct SampleArgs {
  float temperature, top_p;
  int top_k, draft_k;
};

// Kernel 2: workgroup m merges row m's S lists, then lane 0 samples.
__global__ __launch_bounds__(kThreads) void sample_rows_kernel(
    const uint64_t *__restrict__ cand, int S, SampleArgs a,
    const int32_t *__restrict__ draft_tok, const int32_t *__restrict__ draft_idx,
    const float *__restrict__ draft_q, const float *__restrict__ u,
    const float *__restrict__ v, int32_t *__restrict__ top_idx,
    float *__restrict__ top_val, float *__restrict__ top_prob,
    int32_t *__restrict__ greedy, int32_t *__restrict__ accept,
    int32_t *__restrict__ token) {
  __shared__ uint64_t pool[kPoolKeys];
  __shared__ SelectLds sh;
  __shared__ float val[kTopMax], qc[kTopMax];
  __shared__ int32_t tok[kTopMax];
  __shared__ int32_t sdi[kDraftMax];
  __shared__ float sdq[kDraftMax];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = blockIdx.x;
  const uint64_t *rc = cand + static_cast<uint64_t>(m) * S * kTopMax;
  const int64_t nk = static_cast<int64_t>(S) * kTopMax;
  auto for_each = [&](auto f) {
    for (int64_t i = threadIdx.x; i < nk; i += kThreads) f(rc[i]);
  };
  const uint64_t list = block_best32(for_each, pool, sh, wave, lane);
  if (wave != 0) return;
  const int k = a.top_k;
  // the row's draft list, one entry per lane, then q of every candidate
  if (lane < a.draft_k) {
    sdi[lane] = draft_idx[m * a.draft_k + lane];
    sdq[lane] = draft_q[m * a.draft_k + lane];
  }
  const int32_t d = draft_tok[m];
  const float um = u[m], vm = v[m];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    val[lane] = key_value(list);
    tok[lane] = static_cast<int32_t>(key_token(list));
    top_idx[m * k + lane] = tok[lane];
    top_val[m * k + lane] = val[lane];
    float q = 0.0f;  // the first matching draft entry, as the scan finds it
    for (int j = a.draft_k - 1; j >= 0; --j)
      if (sdi[j] == tok[lane]) q = sdq[j];
    qc[lane] = q;
  }
  float qd = 0.0f;  // q of the drafted token
  for (int j = a.draft_k - 1; j >= 0; --j)
    if (sdi[j] == d) qd = sdq[j];

  // Lane i < k holds candidate i.  Sums are wave reductions and cumulative
  // sums lane scans over the candidates in order (fp32).
  const bool live = lane < k;
  const float vi = live ? val[lane] : 0.0f;
  const int32_t ti = live ? tok[lane] : -1;
  const float qi = live ? qc[lane] : 0.0f;
  const float v0 = val[0];
  float pi;
  if (a.temperature == 0.0f) {
    pi = lane == 0 ? 1.0f : 0.0f;
  } else {
    const float w = live ? expf((vi - v0) / a.temperature) : 0.0f;
    pi = w / wave_sum(w);
    // keep the shortest prefix whose mass reaches top_p
    const float c = lane_scan(pi);
    const uint64_t reach = __ballot(live && c >= a.top_p);
    const int keep = reach ? __builtin_ctzll(reach) + 1 : k;
    const float kept = __shfl(c, keep - 1, 64);
    pi = lane < keep ? pi / kept : 0.0f;
  }
  if (live) top_prob[m * k + lane] = pi;
  if (lane == 0) greedy[m] = tok[0];

  // accept test of the drafted token
  const uint64_t at_d = __ballot(live && ti == d);
  const float pd = at_d ? __shfl(pi, __builtin_ctzll(at_d), 64) : 0.0f;
  const bool ok = um * qd < pd;
  if (lane == 0) accept[m] = ok;
  if (ok) {
    if (lane == 0) token[m] = d;
    return;
  }

  // residual draw: the first candidate whose cumulative residual exceeds
  // v R (zero residuals skipped); with no residual mass, the same on p
  float ri = live && pi > qi ? pi - qi : 0.0f;
  float R = wave_sum(ri);
  if (!(R > 0.0f)) {
    ri = pi;
    R = 1.0f;
  }
  const float cr = lane_scan(ri);
  const uint64_t past = __ballot(ri > 0.0f && cr > vm * R);
  const uint64_t pos = __ballot(ri > 0.0f);
  const int pick = past ? __builtin_ctzll(past) : 63 - __builtin_clzll(pos);
  const int32_t drawn = __shfl(ti, pick, 64);  // every lane takes part
  if (lane == 0) token[m] = drawn;
}

int slices_for(int64_t V) {
  return static_cast<int>((V + kSliceCols - 1) / kSliceCols);
}

}  // namespace
}  // namespace q4v

extern "C" int q4_verify_sample_workspace(int M, int64_t V, uint64_t *bytes) {
  if (bytes == nullptr || M < 1 || M > Q4_SAMPLE_MAX_ROWS || V < 1 ||
      V > Q4_SAMPLE_MAX_VOCAB)
    return Q4_EINVAL;
  *bytes = static_cast<uint64_t>(M) * q4v::slices_for(V) * q4v::kTopMax * 8;
  return Q4_OK;
}

extern "C" int q4_verify_sample(const float *logits, int M, int64_t V,
                                const q4_sample_params *prm,
                                const int32_t *draft_tok,
                                const int32_t *draft_idx, const float *draft_q,
                                const float *u, const float *v,
                                int32_t *top_idx, float *top_val,
                                float *top_prob, int32_t *greedy,
                                int32_t *accept, int32_t *token,
                                void *workspace, uint64_t workspace_bytes,
                                void *stream) {
  uint64_t need = 0;
  int st = q4_verify_sample_workspace(M, V, &need);
  if (st != Q4_OK) return st;
  if (prm == nullptr || logits == nullptr || draft_tok == nullptr ||
      u == nullptr || v == nullptr || top_idx == nullptr ||
      top_val == nullptr || top_prob == nullptr || greedy == nullptr ||
      accept == nullptr || token == nullptr || workspace == nullptr)
    return Q4_EINVAL;
  const q4_sample_params p = *prm;
  if (p.top_k < 1 || p.top_k > q4v::kTopMax || p.top_k > V ||
      p.draft_k < 0 || p.draft_k > q4v::kDraftMax ||
      !(p.temperature >= 0.0f) || !(p.temperature < 3.0e38f) ||
      !(p.top_p > 0.0f && p.top_p <= 1.0f) ||
      (p.draft_k > 0 && (draft_idx == nullptr || draft_q == nullptr)) ||
      workspace_bytes < need)
    return Q4_EINVAL;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
    return Q4_EALIGN;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int S = q4v::slices_for(V);
  uint64_t *cand = static_cast<uint64_t *>(workspace);
  hipLaunchKernelGGL(q4v::topk_slices_kernel, dim3(S, M), dim3(64 * q4v::kWaves),
                     0, s, logits, V, S, cand);
  if (hipGetLastError() != hipSuccess) return Q4_ELAUNCH;
  const q4v::SampleArgs a{p.temperature, p.top_p, p.top_k, p.draft_k};
  hipLaunchKernelGGL(q4v::sample_rows_kernel, dim3(M), dim3(64 * q4v::kWaves), 0, s, cand, S,
                     a, draft_tok, draft_idx, draft_q, u, v, top_idx, top_val,
                     top_prob, greedy, accept, token);
  return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}
