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
//     waves; each wave keeps a sorted top-32 list of keys in lanes 0..31
//     while it reads its columns 64 at a time (four chunks' loads issued
//     together): a chunk with no key above the list's 32nd is skipped (one
//     compare and a ballot), otherwise it is sorted with a bitonic network
//     across the wave and merged with the list (the list and the chunk's
//     best 32 reversed form a bitonic sequence of 64, whose half-cleaner
//     cascade leaves the best 32 in lanes 0..31).  The 16 lists are merged
//     pairwise through LDS and the slice's best 32 written out.
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

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  return __shfl_xor(v, m, 64);
}

// Sort 64 keys (one per lane) descending across the wave.
__device__ __forceinline__ uint64_t sort64_desc(uint64_t key, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t other = shfl_xor64(key, j);
      const bool desc_block = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      const bool keep_max = lower == desc_block;
      key = keep_max ? (key > other ? key : other) : (key < other ? key : other);
    }
  }
  return key;
}

// Every lane takes the value of lane - 1; lane 0 takes UINT64_MAX (DPP
// wave shift, two 32-bit moves).
__device__ __forceinline__ uint64_t shift_down_one(uint64_t x) {
  constexpr int kWaveShr1 = 0x138;
  const uint32_t lo = __builtin_amdgcn_update_dpp(
      0xFFFFFFFFu, static_cast<uint32_t>(x), kWaveShr1, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(
      0xFFFFFFFFu, static_cast<uint32_t>(x >> 32), kWaveShr1, 0xF, 0xF, false);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t read_lane64(uint64_t x, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Sum over the wave (a fixed butterfly order, so repeatable).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) x += __shfl_xor(x, j, 64);
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

// Insert one key (wave-uniform, not already present) into the descending
// list of lanes 0..31: lanes past its place take their predecessor's key.
__device__ __forceinline__ uint64_t insert_key(uint64_t list, uint64_t key) {
  const uint64_t prev = shift_down_one(list);
  const bool gt = key > list;
  return gt ? (key < prev ? key : prev) : list;
}

// list: lanes 0..31 hold the best 32 so far, descending (lanes 32..63
// unused).  Merge one chunk of 64 keys (one per lane, any order) into it:
// keys that beat the list's 32nd entry are inserted one by one when few,
// else the chunk is sorted with a bitonic network and merged (the list and
// the chunk's best 32 reversed form a bitonic sequence of 64, whose
// half-cleaner cascade leaves the best 32 in lanes 0..31).
__device__ __forceinline__ uint64_t merge_chunk(uint64_t list, uint64_t chunk,
                                                int lane) {
  uint64_t floor32 = read_lane64(list, 31);
  uint64_t mask = __ballot(chunk > floor32);
  if (mask == 0) return list;
  if (__builtin_popcountll(mask) <= 12) {
    while (mask != 0) {
      const int b = __builtin_ctzll(mask);
      mask &= mask - 1;
      const uint64_t key = read_lane64(chunk, b);
      if (key > floor32) {
        list = insert_key(list, key);
        floor32 = read_lane64(list, 31);
      }
    }
    return list;
  }
  const uint64_t c = sort64_desc(chunk, lane);
  const uint64_t rev = __shfl(c, 63 - lane, 64);
  uint64_t key = lane < 32 ? list : rev;
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    const uint64_t other = shfl_xor64(key, j);
    const bool lower = (lane & j) == 0;
    key = lower ? (key > other ? key : other) : (key < other ? key : other);
  }
  return key;
}

// Best 32 of the keys get(i), i in [begin, end), for one wave: chunks of
// 64, sixteen chunks' loads issued together before they are merged.
template <typename Get>
__device__ __forceinline__ uint64_t wave_topk(Get get, int64_t begin,
                                              int64_t end, int lane) {
  uint64_t list = 0;  // empty entries (key 0) sort after every real key
  constexpr int kGroup = 16;
  for (int64_t b = begin; b < end; b += kGroup * 64) {
    uint64_t key[kGroup];
#pragma unroll
    for (int c = 0; c < kGroup; ++c) {
      const int64_t i = b + 64 * c + lane;
      key[c] = i < end ? get(i) : 0;
    }
#pragma unroll
    for (int c = 0; c < kGroup; ++c) list = merge_chunk(list, key[c], lane);
  }
  return list;
}

// Merge the lists of the W waves of a workgroup, pairwise through LDS;
// wave 0 returns with the best 32.
template <int W>
__device__ __forceinline__ uint64_t block_merge(uint64_t list,
                                                uint64_t (*lists)[kTopMax],
                                                int wave, int lane) {
#pragma unroll
  for (int stride = 1; stride < W; stride <<= 1) {
    if (lane < kTopMax) lists[wave][lane] = list;
    __syncthreads();
    if ((wave & (2 * stride - 1)) == 0) {
      const uint64_t other = lane < kTopMax ? lists[wave + stride][lane] : 0;
      list = merge_chunk(list, other, lane);
    }
    __syncthreads();
  }
  return list;
}

constexpr int kWaves = 16;

// Kernel 1: workgroup (s, m) takes columns [V s / S, V (s+1) / S) of row m.
__global__ __launch_bounds__(64 * kWaves) void topk_slices_kernel(
    const float *__restrict__ logits, int64_t V, int S,
    uint64_t *__restrict__ cand) {
  __shared__ uint64_t lists[kWaves][kTopMax];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int s = blockIdx.x;
  const int m = blockIdx.y;
  const int64_t c0 = V * s / S;
  const int64_t c1 = V * (s + 1) / S;
  const float *row = logits + static_cast<uint64_t>(m) * V;
  auto get = [&](int64_t col) {
    return make_key(row[col], static_cast<uint32_t>(col));
  };
  uint64_t list = wave_topk(get, c0 + (c1 - c0) * wave / kWaves,
                            c0 + (c1 - c0) * (wave + 1) / kWaves, lane);
  list = block_merge<kWaves>(list, lists, wave, lane);
  if (wave == 0 && lane < kTopMax)
    cand[(static_cast<uint64_t>(m) * S + s) * kTopMax + lane] = list;
}

struct SampleArgs {
  float temperature, top_p;
  int top_k, draft_k;
};

// Kernel 2: workgroup m merges row m's S lists, then lane 0 samples.
__global__ __launch_bounds__(64 * kWaves) void sample_rows_kernel(
    const uint64_t *__restrict__ cand, int S, SampleArgs a,
    const int32_t *__restrict__ draft_tok, const int32_t *__restrict__ draft_idx,
    const float *__restrict__ draft_q, const float *__restrict__ u,
    const float *__restrict__ v, int32_t *__restrict__ top_idx,
    float *__restrict__ top_val, float *__restrict__ top_prob,
    int32_t *__restrict__ greedy, int32_t *__restrict__ accept,
    int32_t *__restrict__ token) {
  __shared__ uint64_t lists[kWaves][kTopMax];
  __shared__ float val[kTopMax], qc[kTopMax];
  __shared__ int32_t tok[kTopMax];
  __shared__ int32_t sdi[kDraftMax];
  __shared__ float sdq[kDraftMax];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = blockIdx.x;
  const uint64_t *rc = cand + static_cast<uint64_t>(m) * S * kTopMax;
  const int64_t n = static_cast<int64_t>(S) * kTopMax;
  auto get = [&](int64_t i) { return rc[i]; };
  uint64_t list = wave_topk(get, n * wave / kWaves, n * (wave + 1) / kWaves,
                            lane);
  list = block_merge<kWaves>(list, lists, wave, lane);
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
      V > 0x7FFFFFFFLL)
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
