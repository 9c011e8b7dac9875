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
//     same way, writes the top_k candidates, and lane 0 evaluates the
//     probabilities, the accept test and the residual draw in candidate
//     order, in fp32.
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

// list: lanes 0..31 hold the best 32 so far, descending (lanes 32..63
// unused).  Merge one chunk of 64 keys (one per lane, any order) into it.
__device__ __forceinline__ uint64_t merge_chunk(uint64_t list, uint64_t chunk,
                                                int lane) {
  // skip the chunk when nothing in it beats the list's 32nd entry
  const uint64_t floor32 = __shfl(list, 31, 64);
  if (__ballot(chunk > floor32) == 0) return list;
  const uint64_t c = sort64_desc(chunk, lane);
  // lanes 32..63 take the chunk's best 32 in ascending order: a bitonic 64
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
// 64, four chunks' loads issued together before they are merged.
template <typename Get>
__device__ __forceinline__ uint64_t wave_topk(Get get, int64_t begin,
                                              int64_t end, int lane) {
  uint64_t list = 0;  // empty entries (key 0) sort after every real key
  for (int64_t b = begin; b < end; b += 4 * 64) {
    uint64_t key[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t i = b + 64 * c + lane;
      key[c] = i < end ? get(i) : 0;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) list = merge_chunk(list, key[c], lane);
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
  __shared__ float val[kTopMax], p[kTopMax], r[kTopMax];
  __shared__ int32_t tok[kTopMax];
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
  if (lane < k) {
    val[lane] = key_value(list);
    tok[lane] = static_cast<int32_t>(key_token(list));
    top_idx[m * k + lane] = tok[lane];
    top_val[m * k + lane] = val[lane];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (lane != 0) return;

  // target probabilities, in candidate order
  if (a.temperature == 0.0f) {
    p[0] = 1.0f;
    for (int i = 1; i < k; ++i) p[i] = 0.0f;
  } else {
    float z = 0.0f;
    for (int i = 0; i < k; ++i) {
      p[i] = expf((val[i] - val[0]) / a.temperature);
      z += p[i];
    }
    for (int i = 0; i < k; ++i) p[i] /= z;
    int keep = k;
    float c = 0.0f;
    for (int i = 0; i < k; ++i) {
      c += p[i];
      if (c >= a.top_p) {
        keep = i + 1;
        break;
      }
    }
    float kept = 0.0f;
    for (int i = 0; i < keep; ++i) kept += p[i];
    for (int i = 0; i < k; ++i) p[i] = i < keep ? p[i] / kept : 0.0f;
  }
  for (int i = 0; i < k; ++i) top_prob[m * k + i] = p[i];
  greedy[m] = tok[0];

  // accept test of the drafted token
  const int32_t d = draft_tok[m];
  const int32_t *di = draft_idx + m * a.draft_k;
  const float *dq = draft_q + m * a.draft_k;
  auto qof = [&](int32_t t) {
    for (int j = 0; j < a.draft_k; ++j)
      if (di[j] == t) return dq[j];
    return 0.0f;
  };
  float pd = 0.0f;
  for (int i = 0; i < k; ++i)
    if (tok[i] == d) pd = p[i];
  const bool ok = u[m] * qof(d) < pd;
  accept[m] = ok;
  if (ok) {
    token[m] = d;
    return;
  }

  // residual draw: first candidate whose cumulative residual exceeds v R
  float R = 0.0f;
  for (int i = 0; i < k; ++i) {
    const float qi = qof(tok[i]);
    r[i] = p[i] > qi ? p[i] - qi : 0.0f;
    R += r[i];
  }
  if (!(R > 0.0f)) {
    for (int i = 0; i < k; ++i) r[i] = p[i];
    R = 1.0f;
  }
  const float target = v[m] * R;
  int pick = -1;
  float c = 0.0f;
  for (int i = 0; i < k; ++i) {
    if (r[i] <= 0.0f) continue;
    c += r[i];
    if (c > target) {
      pick = i;
      break;
    }
  }
  if (pick < 0)
    for (int i = k - 1; i >= 0; --i)
      if (r[i] > 0.0f) {
        pick = i;
        break;
      }
  token[m] = tok[pick];
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
