// q4verify_gdn.hip -- gfx950 kernel that writes a verify pass's accepted path
// into the Gated DeltaNet recurrent state, and its C-ABI entry point.
//
// The state is one dv x dk fp32 matrix per recurrent layer and value head,
// read and written back every step (Splash engine article, section on what
// one step reads: 48 layers x 48 value heads x 128 x 128 fp32).  After the
// check, the updates of the accepted tree nodes are applied in path order
// (qwen-spec page, the hybrid-model paragraph), each by the gated delta rule
//     S <- alpha S (I - beta k k^T) + beta v k^T.
//
// Rows of S (one per value index) evolve independently: with d = S_r . k,
// row r becomes alpha S_r + beta (v_r - alpha d) k^T.  The kernel is an HBM
// stream, one read and one write of every state byte, with the work per byte
// in registers:
//  * a workgroup of 4 waves owns 64 rows of one (layer, head) state; lane
//    (rho, j) of a wave (rho = lane / 8, j = lane % 8) holds columns
//    4 (j + 8 i) .. +3, i = 0..3, of rows 16 w + 8 g + rho, g = 0..1: each
//    load instruction reads 128 contiguous bytes of 8 rows.  (128 rows per
//    workgroup, with twice the registers, measured slower: the wider the
//    workgroup, the fewer of them share a compute unit and overlap one
//    another's loads with their arithmetic);
//  * the accepted nodes' keys, this block's value rows and the gates are
//    staged in LDS; per node a row's dot product is 16 FMAs per lane and a
//    3-step DPP sum over its 8 lanes;
//  * the gate is kept as one running factor sigma per (layer, head), so a
//    node costs one FMA per element: S = sigma St, St += (w / sigma') k with
//    sigma' = alpha sigma; when sigma' falls below 2^-30 (a gate near 0) St
//    is rescaled and sigma reset to 1;
//  * the accepted count and the path are read on the device, so the call can
//    follow the accept step on the stream without a host round trip; a count
//    of 0 ends every workgroup before it reads the state.
#include <hip/hip_runtime.h>

#include "q4v_internal.h"

namespace q4v {
namespace {

constexpr int kGdnDk = Q4_GDN_DK;
constexpr int kGdnRows = 64;         // state rows per workgroup
constexpr int kGdnThreads = 256;     // 4 waves x 16 rows
constexpr int kGdnGroups = 2;        // groups of 8 rows per wave
constexpr int kGdnVChunks = kGdnRows / 4;  // float4 of a node's value rows
constexpr float kGdnRenorm = 0x1p-30f;

static_assert(kGdnDk == 128, "one row is 8 lanes x 4 float4 chunks");

struct GdnCommitArgs {
  float *S;
  const float *k, *v, *alpha, *beta;
  const int32_t *path, *n_accept;
  int32_t *status;
  int H, Hk, dv, M, row_blocks;
};

// Sum over the 8 aligned lanes of a group: xor 1 and xor 2 by quad
// permutations, then the half-row mirror (lane i <-> 7 - i) adds the other
// quad.  Every lane of the group ends with the same value.
__device__ __forceinline__ float dpp_sum8(float x) {
  x += __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  return x;
}

__global__ __launch_bounds__(kGdnThreads) void gdn_commit_kernel(
    GdnCommitArgs a) {
  extern __shared__ float4 lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rho = lane >> 3;
  const int j = lane & 7;
  const int M = a.M;

  const int n = a.n_accept[0];
  if (n == 0) {
    if (blockIdx.x == 0 && tid == 0 && a.status != nullptr) a.status[0] = Q4_OK;
    return;
  }
  const bool bad_n = n < 0 || n > M;

  const int rb = blockIdx.x % a.row_blocks;
  const int lh = blockIdx.x / a.row_blocks;  // l * H + h
  const int h = lh % a.H;
  const int l = lh / a.H;
  float *Sb = a.S + (static_cast<size_t>(lh) * a.dv +
                     static_cast<size_t>(rb) * kGdnRows) * kGdnDk;

  // the state rows, issued first; nothing is stored unless the inputs pass
  float4 st[kGdnGroups][4];
#pragma unroll
  for (int g = 0; g < kGdnGroups; ++g) {
    const float4 *row = reinterpret_cast<const float4 *>(
        Sb + static_cast<size_t>(8 * kGdnGroups * w + 8 * g + rho) * kGdnDk);
#pragma unroll
    for (int i = 0; i < 4; ++i) st[g][i] = row[j + 8 * i];
  }

  // every wave checks the whole path itself (n <= M <= 32 < 64 lanes)
  int node = 0;
  bool bad_lane = false;
  if (!bad_n && lane < n) {
    node = a.path[lane];
    bad_lane = node < 0 || node >= M;
  }
  const bool bad = bad_n || __ballot(bad_lane) != 0;
  if (blockIdx.x == 0 && tid == 0 && a.status != nullptr)
    a.status[0] = bad ? Q4_EINVAL : Q4_OK;
  if (bad) return;  // the same decision in every wave of every workgroup

  // stage keys [n][32 float4], this block's value rows [n][16 float4] and
  // (alpha, beta) [n] in LDS
  float4 *ks = lds;
  float4 *vs = lds + 32 * M;
  float2 *gs = reinterpret_cast<float2 *>(lds + (32 + kGdnVChunks) * M);
  const int G = a.H / a.Hk;
  // up to 32 nodes x 32 key chunks = 4 rounds of 256 threads; a round runs
  // only if it holds a node (a uniform test: n <= 8 is one round)
  for (int r = 0; r < 4 && 8 * r < n; ++r) {
    const int e = tid + kGdnThreads * r;
    const int t = e >> 5;
    const int nd = __shfl(node, t & 31, 64);
    if (t < n) {
      const size_t kr = (static_cast<size_t>(l) * M + nd) * a.Hk + h / G;
      ks[e] = reinterpret_cast<const float4 *>(a.k + kr * kGdnDk)[e & 31];
    }
  }
  for (int r = 0; r < 2 && 16 * r < n; ++r) {
    const int e = tid + kGdnThreads * r;
    const int t = e / kGdnVChunks;
    const int nd = __shfl(node, t & 31, 64);
    if (t < n) {
      const size_t vr = (static_cast<size_t>(l) * M + nd) * a.H + h;
      vs[e] = reinterpret_cast<const float4 *>(
          a.v + vr * a.dv + static_cast<size_t>(rb) * kGdnRows)[e % kGdnVChunks];
    }
  }
  if (tid < n) {
    const size_t gi = (static_cast<size_t>(l) * M + node) * a.H + h;
    gs[tid] = make_float2(a.alpha[gi], a.beta[gi]);
  }
  __syncthreads();

  const float *vsf = reinterpret_cast<const float *>(vs);
  float sigma = 1.0f;
  for (int t = 0; t < n; ++t) {
    float4 kq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kq[i] = ks[t * 32 + j + 8 * i];
    const float2 ab = gs[t];
    float cf[kGdnGroups];
#pragma unroll
    for (int g = 0; g < kGdnGroups; ++g) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d = fmaf(st[g][i].x, kq[i].x, d);
        d = fmaf(st[g][i].y, kq[i].y, d);
        d = fmaf(st[g][i].z, kq[i].z, d);
        d = fmaf(st[g][i].w, kq[i].w, d);
      }
      d = dpp_sum8(d) * sigma;  // S_r . k
      const float vr = vsf[t * kGdnRows + 8 * kGdnGroups * w + 8 * g + rho];
      cf[g] = ab.y * (vr - ab.x * d);
    }
    float sn = ab.x * sigma;
    if (!(sn >= kGdnRenorm)) {  // the gate is uniform: so is the branch
#pragma unroll
      for (int g = 0; g < kGdnGroups; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          st[g][i].x *= sn;
          st[g][i].y *= sn;
          st[g][i].z *= sn;
          st[g][i].w *= sn;
        }
      sn = 1.0f;
    }
    const float inv = 1.0f / sn;
#pragma unroll
    for (int g = 0; g < kGdnGroups; ++g) {
      const float c = cf[g] * inv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st[g][i].x = fmaf(c, kq[i].x, st[g][i].x);
        st[g][i].y = fmaf(c, kq[i].y, st[g][i].y);
        st[g][i].z = fmaf(c, kq[i].z, st[g][i].z);
        st[g][i].w = fmaf(c, kq[i].w, st[g][i].w);
      }
    }
    sigma = sn;
  }

#pragma unroll
  for (int g = 0; g < kGdnGroups; ++g) {
    float4 *row = reinterpret_cast<float4 *>(
        Sb + static_cast<size_t>(8 * kGdnGroups * w + 8 * g + rho) * kGdnDk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 o = st[g][i];
      o.x *= sigma;
      o.y *= sigma;
      o.z *= sigma;
      o.w *= sigma;
      row[j + 8 * i] = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Tree-node outputs of one recurrent layer (qwen-spec page, the hybrid-model
// paragraph: every tree node reads the shared state after the context plus
// the updates along its own path).  Node i's output is o_i = S_i q_i, S_i
// being the state after the updates of the nodes root .. i.
//
// Rows stay independent, and along a path the row s evolves as
//     s_i = alpha_i s_p + c_i k_i,  c_i = beta_i (v_i[r] - alpha_i s_p . k_i)
// (p the parent), so s_i = A_i s_0 + sum_{m in path(i)} W_im c_m k_m with
// W_im the product of the gates of the path's nodes after m, down to i
// (W_ii = 1), and A_i the product over the whole path.  Hence, with the row's dot products
// s_0 . k_m and s_0 . q_i and the layer's key-key and key-query products,
//     s_p . k_i = A_p (s_0 . k_i) + sum_{m in path(p)} W_pm (k_m . k_i) c_m,
//     o_i[r]    = A_i (s_0 . q_i) + sum_{m in path(i)} W_im (k_m . q_i) c_m:
// a short triangular recurrence per row on the coefficients c, in node
// order (parents precede children).  The state is read once and not written.
//  * a workgroup owns 32 rows of one head; lane (rho, j) of wave w holds
//    columns 4 (j + 8 i) .. +3, i = 0..3, of row 8 w + rho, and a row's dot
//    product is 16 FMAs per lane and a 3-step DPP sum over its 8 lanes;
//  * the tree's keys and queries (for the head's key head), its values for
//    the workgroup's rows and the gates sit in LDS; one wave forms the path
//    weights (a lane per node walking its path once), then every wave forms
//    the products k_m . k_i and k_m . q_i in the row layout, the keys and
//    queries standing in for state rows;
//  * in the recurrence lane j keeps c_m, s_0 . k_m and s_0 . q_m for the
//    nodes m = j mod 8, so each step is a few FMAs and one 8-lane sum.
constexpr int kTreeRows = 32;
constexpr int kTreeThreads = 256;
constexpr int kTreeMax = Q4_GDN_MAX_NODES;
static_assert(kTreeMax == 32, "c, s0.k and s0.q: 4 registers per lane");

struct GdnTreeArgs {
  const float *S, *q, *k, *v, *alpha, *beta;
  const int32_t *parent;
  float *out;
  int32_t *status;
  int H, Hk, dv, M, row_blocks;
};

// NMAX (16 or 32) bounds the node loops: they run without per-node branches
// (the arrays are zero past M), so that the compiler can issue a later
// node's LDS reads early.
template <int NMAX>
__global__ __launch_bounds__(kTreeThreads) void gdn_tree_out_kernel(
    GdnTreeArgs a) {
  __shared__ float4 kq[2 * kTreeMax * 32];  // keys, then queries [node][32]
  __shared__ float vsm[kTreeMax * kTreeRows];   // values [node][row]
  __shared__ float kk[kTreeMax * kTreeMax];     // k_m . k_i at [m][i]
  __shared__ float kqd[kTreeMax * kTreeMax];    // k_m . q_i at [i][m]
  __shared__ float wk[kTreeMax * kTreeMax];     // W_pm at [i][m] (p = parent of i)
  __shared__ float wq[kTreeMax * kTreeMax];     // W_im at [i][m]
  __shared__ float obuf[kTreeMax * kTreeRows];  // outputs [node][row]
  __shared__ float al[kTreeMax], be[kTreeMax], ak[kTreeMax], aq[kTreeMax];
  __shared__ int par[kTreeMax];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rho = lane >> 3;
  const int j = lane & 7;
  const int M = a.M;
  const int rb = blockIdx.x % a.row_blocks;
  const int h = blockIdx.x / a.row_blocks;
  const int hk = h / (a.H / a.Hk);
  const int row = 8 * w + rho;  // within the block

  // Loads in the order they are needed: the tree and the gates (for the
  // check and the path weights), the keys, queries and values (for the
  // products), then this lane's part of its state row (for the row's
  // products, after the path weights); all issued before the tree check,
  // so that the workgroup waits for one round trip.
  int pi = -1;
  if (lane < M) pi = a.parent[lane];
  float ga = 0.0f, gb = 0.0f;
  if (tid < M) {
    ga = a.alpha[static_cast<size_t>(tid) * a.H + h];
    gb = a.beta[static_cast<size_t>(tid) * a.H + h];
  }
  float4 kqr[2 * kTreeMax * 32 / kTreeThreads];
  float vr[kTreeMax * kTreeRows / kTreeThreads];
#pragma unroll
  for (int r = 0; r < 2 * kTreeMax * 32 / kTreeThreads; ++r)
    kqr[r] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int r = 0; r < kTreeMax * kTreeRows / kTreeThreads; ++r) vr[r] = 0.0f;
#pragma unroll
  for (int r = 0; r < 2 * kTreeMax * 32 / kTreeThreads; ++r) {
    const int e = tid + kTreeThreads * r;
    if (e < 2 * M * 32) {
      const int node = (e >> 5) % M;
      const float *src = e < M * 32 ? a.k : a.q;
      kqr[r] = reinterpret_cast<const float4 *>(
          src + (static_cast<size_t>(node) * a.Hk + hk) * kGdnDk)[e & 31];
    }
  }
#pragma unroll
  for (int r = 0; r < kTreeMax * kTreeRows / kTreeThreads; ++r) {
    const int e = tid + kTreeThreads * r;
    if (e < M * kTreeRows)
      vr[r] = a.v[(static_cast<size_t>(e / kTreeRows) * a.H + h) * a.dv +
                  static_cast<size_t>(rb) * kTreeRows + e % kTreeRows];
  }
  const float4 *srow = reinterpret_cast<const float4 *>(
      a.S + (static_cast<size_t>(h) * a.dv + static_cast<size_t>(rb) * kTreeRows + row) *
                kGdnDk);
  float4 st[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) st[i] = srow[j + 8 * i];

  // every wave checks the whole tree: -1 <= parent[i] < i
  const bool bad_lane = lane < M && (pi < -1 || pi >= lane);
  const bool bad = __ballot(bad_lane) != 0;
  if (blockIdx.x == 0 && tid == 0 && a.status != nullptr)
    a.status[0] = bad ? Q4_EINVAL : Q4_OK;
  if (bad) return;  // the same decision in every wave of every workgroup

  if (w == 0 && lane < M) par[lane] = pi;
#pragma unroll
  for (int r = 0; r < 2 * kTreeMax * 32 / kTreeThreads; ++r) {
    const int e = tid + kTreeThreads * r;
    if (e < 2 * NMAX * 32) kq[e] = kqr[r];  // zeros past the queries
  }
#pragma unroll
  for (int r = 0; r < kTreeMax * kTreeRows / kTreeThreads; ++r) {
    const int e = tid + kTreeThreads * r;
    if (e < NMAX * kTreeRows) vsm[e] = vr[r];
  }
  if (tid < NMAX) {
    al[tid] = ga;  // 0 past M
    be[tid] = gb;
  }
  for (int e = tid; e < kTreeMax * kTreeMax; e += kTreeThreads) {
    wk[e] = 0.0f;  // zero off the paths
    wq[e] = 0.0f;
    kk[e] = 0.0f;  // and past M, so that every product read is finite
    kqd[e] = 0.0f;
  }
  __syncthreads();

  if (w == 0) {
    // path weights, one lane per node walking its path once: W_im for the
    // node's own path and W_pm for its parent's (W_pm = W_im / alpha_i,
    // carried as a second product rather than divided)
    if (lane >= M && lane < NMAX) {
      aq[lane] = 0.0f;
      ak[lane] = 0.0f;
    } else if (lane < M) {
      const int i = lane;
      wq[i * kTreeMax + i] = 1.0f;
      float wi = al[i], wp = 1.0f;
      for (int m = par[i]; m >= 0; m = par[m]) {
        wq[i * kTreeMax + m] = wi;
        wk[i * kTreeMax + m] = wp;
        const float g = al[m];
        wi *= g;
        wp *= g;
      }
      aq[i] = wi;  // A_i
      ak[i] = wp;  // A_p (1 for a child of the context)
    }
  }
  // k_m . k_i and k_m . q_i for every pair, in the row layout: the keys and
  // the queries (rows 0 .. 2M-1 of kq) take the place of state rows, 32 a
  // pass, and each is multiplied with every key m; the first pass also forms
  // the row's s_0 . k_m and s_0 . q_m (lane j keeps those of m = j mod 8),
  // sharing the read of key m
  float s0k[4] = {0.0f, 0.0f, 0.0f, 0.0f}, s0q[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g0 = 0; g0 < 2 * NMAX; g0 += kTreeRows) {
    const int gr = g0 + row;  // the key (gr < M) or query (gr - M) of this lane's row
    float4 kr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = kq[gr * 32 + j + 8 * i];
#pragma unroll 8
    for (int m = 0; m < NMAX; ++m) {
      float d = 0.0f, pk = 0.0f, pq = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = kq[m * 32 + j + 8 * i];
        d = fmaf(kr[i].x, x.x, d);
        d = fmaf(kr[i].y, x.y, d);
        d = fmaf(kr[i].z, x.z, d);
        d = fmaf(kr[i].w, x.w, d);
        if (g0 == 0) {
          const float4 z = kq[(M + m) * 32 + j + 8 * i];
          pk = fmaf(st[i].x, x.x, pk);
          pk = fmaf(st[i].y, x.y, pk);
          pk = fmaf(st[i].z, x.z, pk);
          pk = fmaf(st[i].w, x.w, pk);
          pq = fmaf(st[i].x, z.x, pq);
          pq = fmaf(st[i].y, z.y, pq);
          pq = fmaf(st[i].z, z.z, pq);
          pq = fmaf(st[i].w, z.w, pq);
        }
      }
      d = dpp_sum8(d);
      if (j == 0 && m < M) {
        if (gr < M)
          kk[m * kTreeMax + gr] = d;
        else if (gr < 2 * M)
          kqd[(gr - M) * kTreeMax + m] = d;
      }
      if (g0 == 0) {
        pk = dpp_sum8(pk);
        pq = dpp_sum8(pq);
        if (j == m % 8) {
          s0k[m / 8] = pk;
          s0q[m / 8] = pq;
        }
      }
    }
  }
  __syncthreads();  // path weights and products

  // the recurrence in node order
  float cl[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < NMAX; ++i) {
    {
      float part = j == i % 8 ? ak[i] * s0k[i / 8] : 0.0f;
#pragma unroll
      for (int t = 0; t < NMAX / 8; ++t) {
        const int m = 8 * t + j;
        part = fmaf(wk[i * kTreeMax + m] * kk[m * kTreeMax + i], cl[t], part);
      }
      const float d = dpp_sum8(part);  // s_p . k_i
      const float c = be[i] * (vsm[i * kTreeRows + row] - al[i] * d);
      if (j == i % 8) cl[i / 8] = c;
      part = j == i % 8 ? aq[i] * s0q[i / 8] : 0.0f;
#pragma unroll
      for (int t = 0; t < NMAX / 8; ++t) {
        const int m = 8 * t + j;
        part = fmaf(wq[i * kTreeMax + m] * kqd[i * kTreeMax + m], cl[t], part);
      }
      const float o = dpp_sum8(part);
      if (j == 0) obuf[i * kTreeRows + row] = o;
    }
  }
  __syncthreads();
  // out [M][H][dv]: 8 float4 of the block's rows per node
  for (int e = tid; e < M * 8; e += kTreeThreads) {
    const int node = e >> 3, c = e & 7;
    reinterpret_cast<float4 *>(a.out + (static_cast<size_t>(node) * a.H + h) * a.dv +
                               static_cast<size_t>(rb) * kTreeRows)[c] =
        reinterpret_cast<const float4 *>(obuf + node * kTreeRows)[c];
  }
}

}  // namespace
}  // namespace q4v

extern "C" int q4_gdn_tree_out(const float *S, int H, int Hk, int dv, int dk,
                               int M, const float *q, const float *k,
                               const float *v, const float *alpha,
                               const float *beta, const int32_t *parent,
                               float *out, int32_t *status, void *stream) {
  if (S == nullptr || q == nullptr || k == nullptr || v == nullptr ||
      alpha == nullptr || beta == nullptr || parent == nullptr ||
      out == nullptr || H < 1 || Hk < 1 || H % Hk != 0 || dk != Q4_GDN_DK ||
      dv < 1 || dv % q4v::kTreeRows != 0 || M < 1 || M > Q4_GDN_MAX_NODES)
    return Q4_EINVAL;
  const int64_t blocks = static_cast<int64_t>(H) * (dv / q4v::kTreeRows);
  if (blocks > 0x7FFFFFFF) return Q4_EINVAL;
  if ((reinterpret_cast<uintptr_t>(S) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(q) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(k) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(v) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(alpha) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(beta) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(parent) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(status) & 3u) != 0)
    return Q4_EALIGN;
  const int st = q4v::check_device();
  if (st != Q4_OK) return st;
  const q4v::GdnTreeArgs a{S, q, k, v, alpha, beta, parent, out, status,
                           H, Hk, dv, M, dv / q4v::kTreeRows};
  if (M <= 16)
    hipLaunchKernelGGL(q4v::gdn_tree_out_kernel<16>, dim3(static_cast<uint32_t>(blocks)),
                       dim3(q4v::kTreeThreads), 0, static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(q4v::gdn_tree_out_kernel<32>, dim3(static_cast<uint32_t>(blocks)),
                       dim3(q4v::kTreeThreads), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

extern "C" int q4_gdn_commit_lds_bytes(int M, int *bytes) {
  if (bytes == nullptr || M < 1 || M > Q4_GDN_MAX_NODES) return Q4_EINVAL;
  *bytes = M * ((32 + q4v::kGdnVChunks) * 16 + 8);
  return Q4_OK;
}

extern "C" int q4_gdn_commit(float *S, int L, int H, int Hk, int dv, int dk,
                             int M, const float *k, const float *v,
                             const float *alpha, const float *beta,
                             const int32_t *path, const int32_t *n_accept,
                             int32_t *status, void *stream) {
  int lds = 0;
  if (q4_gdn_commit_lds_bytes(M, &lds) != Q4_OK) return Q4_EINVAL;
  if (S == nullptr || k == nullptr || v == nullptr || alpha == nullptr ||
      beta == nullptr || path == nullptr || n_accept == nullptr || L < 1 ||
      H < 1 || Hk < 1 || H % Hk != 0 || dk != Q4_GDN_DK || dv < 1 ||
      dv % q4v::kGdnRows != 0)
    return Q4_EINVAL;
  const int64_t blocks = static_cast<int64_t>(L) * H * (dv / q4v::kGdnRows);
  if (blocks > 0x7FFFFFFF) return Q4_EINVAL;
  if ((reinterpret_cast<uintptr_t>(S) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(k) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(v) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(alpha) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(beta) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(path) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(n_accept) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(status) & 3u) != 0)
    return Q4_EALIGN;
  const int st = q4v::check_device();
  if (st != Q4_OK) return st;
  const q4v::GdnCommitArgs a{S, k, v, alpha, beta, path, n_accept, status,
                             H, Hk, dv, M, dv / q4v::kGdnRows};
  hipLaunchKernelGGL(q4v::gdn_commit_kernel, dim3(static_cast<uint32_t>(blocks)),
                     dim3(q4v::kGdnThreads), lds,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}
