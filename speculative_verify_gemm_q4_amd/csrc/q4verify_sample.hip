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
//  2. The row's candidates from its lists of 32, then the sampling:
//     - sample_rows_kernel (more than 32 lists a row, as the fused LM head
//       writes): one wave per row reads the first 4 keys of every list.
//       Each list is descending, so the lane maxima of the lists' heads
//       bound the row's 32nd best key from below; the keys read at or above
//       the bound are ranked, and the rare list that may hold more of them
//       past its first 4 is read whole.
//     - sample_rows_few_kernel (at most 32 lists, as the standalone
//       epilogue writes for rows of up to 524288 columns): 16 waves, one
//       key per thread, the waves' best 32 merged as in kernel 1.
//     Lane i of one wave then takes candidate i, and the probabilities, the
//     accept test and the residual draw are evaluated in fp32 with wave
//     reductions, lane scans and ballots over the candidates in order.

#include <hip/hip_runtime.h>

#include "q4v_internal.h"
#include "q4v_select.h"

namespace q4v {
namespace {

constexpr int kTopMax = 32;
constexpr int kDraftMax = 16;
constexpr int kSliceCols = 16384;  // columns per workgroup of kernel 1

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
// survivor pool of kernel 1: every key of its slice
constexpr int kPoolKeys = kColsPerThread * kThreads;
static_assert(static_cast<int64_t>(Q4_SAMPLE_MAX_VOCAB) <=
                  static_cast<int64_t>(kSampleMaxLists) * kSliceCols,
              "the row kernel reads at most kSampleMaxLists lists a row");
static_assert(kTopMax == kSampleTop, "one list length");

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
  __shared__ uint64_t pool[kPoolKeys];
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

// Wave-wide order of the wave's LDS accesses: earlier writes by any lane
// are seen by later reads of any lane.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS of the sampling tail: the candidates' values and tokens, q of each
// candidate, the row's draft list.
struct TailLds {
  float val[kTopMax], qc[kTopMax];
  int32_t tok[kTopMax];
  int32_t sdi[kDraftMax];
  float sdq[kDraftMax];
};

// The row's draft list into LDS (lanes < draft_k of one wave).
__device__ __forceinline__ void load_draft(TailLds &tl, const SampleArgs &a, int m,
                                           const int32_t *__restrict__ draft_idx,
                                           const float *__restrict__ draft_q,
                                           int lane) {
  if (lane < a.draft_k) {
    tl.sdi[lane] = draft_idx[m * a.draft_k + lane];
    tl.sdq[lane] = draft_q[m * a.draft_k + lane];
  }
}

// One wave samples row m from its candidates (lane i < 32: the i-th best
// key): lane i then holds candidate i, and the probabilities, the accept
// test and the residual draw are evaluated in fp32 with wave reductions,
// lane scans and ballots over the candidates in order.  The draft list must
// be in tl, visible to the wave.
__device__ __forceinline__ void sample_row(
    uint64_t list, int m, const SampleArgs &a, TailLds &tl, int32_t d, float um,
    float vm, int32_t *__restrict__ top_idx, float *__restrict__ top_val,
    float *__restrict__ top_prob, int32_t *__restrict__ greedy,
    int32_t *__restrict__ accept, int32_t *__restrict__ token, int lane) {
  const int k = a.top_k;
  // q of every candidate from the row's draft list
  if (lane < k) {
    tl.val[lane] = key_value(list);
    tl.tok[lane] = static_cast<int32_t>(key_token(list));
    top_idx[m * k + lane] = tl.tok[lane];
    top_val[m * k + lane] = tl.val[lane];
    float q = 0.0f;  // the first matching draft entry, as the scan finds it
    for (int j = a.draft_k - 1; j >= 0; --j)
      if (tl.sdi[j] == tl.tok[lane]) q = tl.sdq[j];
    tl.qc[lane] = q;
  }
  float qd = 0.0f;  // q of the drafted token
  for (int j = a.draft_k - 1; j >= 0; --j)
    if (tl.sdi[j] == d) qd = tl.sdq[j];

  // Lane i < k holds candidate i.  Sums are wave reductions and cumulative
  // sums lane scans over the candidates in order (fp32).
  const bool live = lane < k;
  const float vi = live ? tl.val[lane] : 0.0f;
  const int32_t ti = live ? tl.tok[lane] : -1;
  const float qi = live ? tl.qc[lane] : 0.0f;
  const float v0 = tl.val[0];
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
  if (lane == 0) greedy[m] = tl.tok[0];

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

constexpr int kListsPerLane = kSampleMaxLists / 64;
constexpr int kLead = 4;  // keys read first from every list

// Kernel 2: one wave per row m merges the row's S lists, then samples.
// Every list is descending, so its first key (its head) is its largest.
// Lane l reads the first 4 keys of lists l,
// l + 64, ..  T = the 32nd largest lane maximum of the heads: 32 distinct
// heads reach it, so the row's 32nd best key does too, and every key of
// the row's best 32 is >= T.  The keys read that are >= T are kept
// (usually 40 to 60; at most 32 lanes x 8 lists x 4).  A key of the best
// 32 past a list's first 4 needs that list's 4th key >= T; when some list
// has one, T is raised to the 32nd best kept key (again a lower bound of
// the row's 32nd best, now with at most 8 lists whose 4th key reaches it)
// and those lists are read whole.  The best 32 kept keys are the row's
// best 32.  (Rows of at most 32 lists go to sample_rows_few_kernel.)
__global__ __launch_bounds__(64) void sample_rows_kernel(
    const uint64_t *__restrict__ cand, int S, SampleArgs a,
    const int32_t *__restrict__ draft_tok, const int32_t *__restrict__ draft_idx,
    const float *__restrict__ draft_q, const float *__restrict__ u,
    const float *__restrict__ v, int32_t *__restrict__ top_idx,
    float *__restrict__ top_val, float *__restrict__ top_prob,
    int32_t *__restrict__ greedy, int32_t *__restrict__ accept,
    int32_t *__restrict__ token) {
  // kept keys: the first 4 of at most 32 x 8 lists and the other 28 of at
  // most 8 lists read whole, + 8 slots for the ranking
  constexpr int kPool = kTopMax * kListsPerLane * kLead + 8 * (kTopMax - kLead);
  __shared__ uint64_t pool[kPool + 8];
  __shared__ uint64_t sel[kTopMax];  // the lists read whole
  __shared__ uint64_t best[kTopMax];
  __shared__ uint64_t dummy;
  __shared__ TailLds tl;
  const int lane = threadIdx.x;
  const int m = blockIdx.x;
  const uint64_t *rc = cand + static_cast<uint64_t>(m) * S * kTopMax;
  // the row's draft list and scalars, loaded while the lists arrive
  load_draft(tl, a, m, draft_idx, draft_q, lane);
  const int32_t d = draft_tok[m];
  const float um = u[m], vm = v[m];
  uint32_t n = 0;
  {
    uint64_t lead[kListsPerLane][kLead];
    uint64_t mx = 0;
#pragma unroll
    for (int i = 0; i < kListsPerLane; ++i) {
      const int g = i * 64 + lane;
#pragma unroll
      for (int j = 0; j < kLead; ++j)
        lead[i][j] = g < S ? rc[static_cast<uint64_t>(g) * kTopMax + j] : 0;
      mx = lead[i][0] > mx ? lead[i][0] : mx;
    }
    uint64_t T = wave_kth_largest(mx, kTopMax);
    bool deep = false;  // some list's 4th key reaches T
#pragma unroll
    for (int i = 0; i < kListsPerLane; ++i) {
      if (i * 64 >= S) break;  // wave-uniform
#pragma unroll
      for (int j = 0; j < kLead; ++j) {
        const bool keep = lead[i][j] != 0 && lead[i][j] >= T;
        if (__ballot(keep) != 0) wave_append(lead[i][j], keep, pool, &n, &dummy);
        if (j == kLead - 1) deep = deep || keep;
      }
    }
    wave_sync();
    if (__ballot(deep) != 0) {
      // raise T to the 32nd best kept key; the lists whose 4th key reaches
      // it (at most 8: 32 kept keys reach T) are read whole: lane l takes
      // key l & 31 (past the first 4) of lists l >> 5, (l >> 5) + 2, ..
      wave_top32(pool, n, best, lane);
      wave_sync();
      T = best[kTopMax - 1];
      uint32_t ns = 0;
#pragma unroll
      for (int i = 0; i < kListsPerLane; ++i) {
        const bool whole = lead[i][kLead - 1] != 0 && lead[i][kLead - 1] >= T;
        wave_append(static_cast<uint64_t>(i * 64 + lane), whole, sel, &ns, &dummy);
      }
      wave_sync();
      for (uint32_t l0 = 0; l0 < ns; l0 += 2) {
        const uint32_t li = l0 + static_cast<uint32_t>(lane >> 5);
        const bool past = (lane & 31) >= kLead;
        const uint64_t key = li < ns && past ? rc[sel[li] * kTopMax + (lane & 31)] : 0;
        wave_append(key, key != 0 && key >= T, pool, &n, &dummy);
      }
      wave_sync();
    }
  }
  wave_top32(pool, n, best, lane);
  wave_sync();
  const uint64_t list = lane < kTopMax ? best[lane] : 0;
  sample_row(list, m, a, tl, d, um, vm, top_idx, top_val, top_prob, greedy,
             accept, token, lane);
}

// Kernel 2 for rows of at most 32 lists (the standalone epilogue on rows
// of up to 32 slices): one workgroup of 16 waves per row, one key per
// thread.  Each wave sorts its 64 keys and the waves' best 32 are merged
// pairwise through LDS, which leaves the row's best 32 in wave 0; wave 0
// then samples.
__global__ __launch_bounds__(kThreads) void sample_rows_few_kernel(
    const uint64_t *__restrict__ cand, int S, SampleArgs a,
    const int32_t *__restrict__ draft_tok, const int32_t *__restrict__ draft_idx,
    const float *__restrict__ draft_q, const float *__restrict__ u,
    const float *__restrict__ v, int32_t *__restrict__ top_idx,
    float *__restrict__ top_val, float *__restrict__ top_prob,
    int32_t *__restrict__ greedy, int32_t *__restrict__ accept,
    int32_t *__restrict__ token) {
  __shared__ uint64_t lists[kWaves][kTopMax];
  __shared__ TailLds tl;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = blockIdx.x;
  const uint64_t *rc = cand + static_cast<uint64_t>(m) * S * kTopMax;
  const uint64_t key =
      static_cast<int>(threadIdx.x) < S * kTopMax ? rc[threadIdx.x] : 0;
  if (wave == 0) load_draft(tl, a, m, draft_idx, draft_q, lane);
  const int32_t d = draft_tok[m];
  const float um = u[m], vm = v[m];
  const uint64_t list = block_merge(sort64_desc(key, lane), lists, wave, lane);
  if (wave != 0) return;
  sample_row(lane < kTopMax ? list : 0, m, a, tl, d, um, vm, top_idx, top_val,
             top_prob, greedy, accept, token, lane);
}

int slices_for(int64_t V) {
  return static_cast<int>((V + kSliceCols - 1) / kSliceCols);
}

}  // namespace

int check_sample_args(int M, int64_t V, const q4_sample_params *prm,
                      const int32_t *draft_tok, const int32_t *draft_idx,
                      const float *draft_q, const float *u, const float *v,
                      int32_t *top_idx, float *top_val, float *top_prob,
                      int32_t *greedy, int32_t *accept, int32_t *token) {
  if (M < 1 || M > Q4_SAMPLE_MAX_ROWS || V < 1 || V > Q4_SAMPLE_MAX_VOCAB ||
      prm == nullptr || draft_tok == nullptr || u == nullptr ||
      v == nullptr || top_idx == nullptr || top_val == nullptr ||
      top_prob == nullptr || greedy == nullptr || accept == nullptr ||
      token == nullptr)
    return Q4_EINVAL;
  const q4_sample_params p = *prm;
  if (p.top_k < 1 || p.top_k > kTopMax || p.top_k > V || p.draft_k < 0 ||
      p.draft_k > kDraftMax || !(p.temperature >= 0.0f) ||
      !(p.temperature < 3.0e38f) || !(p.top_p > 0.0f && p.top_p <= 1.0f) ||
      (p.draft_k > 0 && (draft_idx == nullptr || draft_q == nullptr)))
    return Q4_EINVAL;
  return Q4_OK;
}

int launch_sample_rows(const uint64_t *cand, int M, int S,
                       const q4_sample_params &p, const int32_t *draft_tok,
                       const int32_t *draft_idx, const float *draft_q,
                       const float *u, const float *v, int32_t *top_idx,
                       float *top_val, float *top_prob, int32_t *greedy,
                       int32_t *accept, int32_t *token, hipStream_t s) {
  if (S < 1 || S > kSampleMaxLists) return Q4_EINVAL;
  const SampleArgs a{p.temperature, p.top_p, p.top_k, p.draft_k};
  if (S <= kTopMax)
    hipLaunchKernelGGL(sample_rows_few_kernel, dim3(M), dim3(kThreads), 0, s,
                       cand, S, a, draft_tok, draft_idx, draft_q, u, v, top_idx,
                       top_val, top_prob, greedy, accept, token);
  else
    hipLaunchKernelGGL(sample_rows_kernel, dim3(M), dim3(64), 0, s,
                     cand, S, a, draft_tok, draft_idx, draft_q, u, v, top_idx,
                     top_val, top_prob, greedy, accept, token);
  return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

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
  st = q4v::check_sample_args(M, V, prm, draft_tok, draft_idx, draft_q, u, v,
                              top_idx, top_val, top_prob, greedy, accept,
                              token);
  if (st != Q4_OK) return st;
  if (logits == nullptr || workspace == nullptr || workspace_bytes < need)
    return Q4_EINVAL;
  const q4_sample_params p = *prm;
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
  return q4v::launch_sample_rows(cand, M, S, p, draft_tok, draft_idx, draft_q,
                                 u, v, top_idx, top_val, top_prob, greedy,
                                 accept, token, s);
}
