// q4verify_attn.hip -- gfx950 kernels of tree-verify attention over the
// paged int8 KV cache, and their C-ABI entry points.
//
// One attention layer of the verify pass: every tree node (up to 16) and
// query head attends to the context and to its own ancestors in the tree,
// reading the cache in place (qwen-spec page, Notes and the hybrid-model
// paragraph).  Shapes and cache format: 24 query heads over 4 KV heads of
// dimension 256; pages of 32 tokens, int8, an fp32 scale per token per head
// (Splash engine article, the model listing and the paged KV pool).  The
// tree's keys and values follow the context in the cache: node j at
// position ctx_len + j.
//
// Kernel 1 (tree_attn_kernel<G>): a workgroup per (KV head, run of pages),
// one compute wave per query head of that KV head (G = Hq / Hkv) and two
// loader waves; when the runs leave CUs idle, h workgroups per (KV head,
// run), each with G = Hq / Hkv / h of its query heads (h up to 6).
//  * Per page the loader waves load the 8 KiB of keys ([32 tokens][256])
//    and 8 KiB of values (stored transposed, [256][32]) with their scales
//    into their registers, four pages ahead, turn the int8 keys into bf16
//    and the int8 values into fp16 (both exact: |v| <= 128) and write them
//    to an LDS tile (two tiles: the compute waves read one page while the
//    next is written).
//  * Scores on MFMA: S^T[token][node] = K Q^T, sixteen
//    v_mfma_f32_16x16x32_bf16 per page and wave (two token tiles, eight
//    32-dim steps), the key scale times the softmax scale (the loaders
//    form the product) applied per token afterwards; the queries stay in
//    registers for the whole run.
//  * Online softmax per node in base 2, its reference maximum moved only
//    when a score passes it by more than 2^8; each node's 32 scores of a
//    page sit in 4 lanes x 8 registers.  The ancestor mask applies to tree positions,
//    a 32-bit ancestor-or-self set per node.
//  * Values on MFMA: O^T[dim][node] += V^T P''^T with P'' = p * v_scale /
//    vlim rounded to fp16 (vlim a power of two at or above the value scales
//    seen, so P'' <= 2^8) and one v_mfma_f32_16x16x32_f16 per value tile;
//    the value tile's tokens are stored in the order in which the score
//    tiles hold them in a lane (tokens 4g..4g+3, 16+4g..16+4g+3 for lane
//    group g), so the probabilities need no shuffle.
//  * A run over the whole context writes normalised outputs; otherwise the
//    run writes its unnormalised output and (max, sum) to the workspace.
//  * Maxima and sums over a node's four lane groups use the gfx950 permlane
//    swaps; the page's largest value scale comes from the loader.
// Kernel 2 (attn_combine_kernel): per (node, query head) the runs' partial
// results are merged with their max and sum.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <type_traits>

#include "q4v_internal.h"

namespace q4v {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = Q4_ATTN_HEAD_DIM;       // 256
constexpr int kPage = Q4_ATTN_PAGE;        // 32
constexpr int kKStride = 2 * kD + 16;      // bytes per token row of bf16 keys
constexpr int kVStride = 2 * kPage + 16;   // bytes per dim row of bf16 values
constexpr int kKBytes = kPage * kKStride;  // 16896
constexpr int kVBytes = kD * kVStride;     // 20480
// the scales: 32 key scales, then 32 value scales, each in a 1 KiB area
// that a whole wave's 16-byte writes fill (lanes 8..63 write the zeros they
// loaded past the scales), so that the write needs no branch on the lane
constexpr int kScaleArea = 64 * 16;
constexpr int kBufBytes = kKBytes + kVBytes + 2 * kScaleArea;
constexpr uint32_t kBufferWord3 = 0x00020000u;
constexpr float kLog2e = 1.4426950408889634f;
// Headroom of the running maximum in the online softmax (base 2).
constexpr float kLazyMax = 8.0f;

struct AttnArgs {
  const uint16_t *q;
  const int8_t *kp, *vp;
  const float *ks, *vs;
  const int32_t *page_table;
  const uint32_t *anc;
  float *out, *part;
  int32_t *status;
  int M, Hq, Hkv, pool, ctx, pages, splits;
  float scale2;  // softmax scale times log2(e)
  int hsplit;    // workgroups per (KV head, run), each G of its query heads
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p,
                                                       uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0,
                                           static_cast<int>(bytes),
                                           kBufferWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r,
                                        uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// four int8 -> four bf16 (exact), as two packed pairs
__device__ __forceinline__ u32x2 i8x4_bf16(uint32_t w) {
  const bf16x2 a = {static_cast<__bf16>(static_cast<float>(static_cast<int8_t>(w))),
                    static_cast<__bf16>(static_cast<float>(static_cast<int8_t>(w >> 8)))};
  const bf16x2 b = {static_cast<__bf16>(static_cast<float>(static_cast<int8_t>(w >> 16))),
                    static_cast<__bf16>(static_cast<float>(static_cast<int8_t>(w >> 24)))};
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// four int8 -> four fp16 (exact: |v| <= 128 < 2^11), as two packed pairs
__device__ __forceinline__ u32x2 i8x4_f16(uint32_t w) {
  const f16x2 a = {static_cast<_Float16>(static_cast<float>(static_cast<int8_t>(w))),
                   static_cast<_Float16>(static_cast<float>(static_cast<int8_t>(w >> 8)))};
  const f16x2 b = {static_cast<_Float16>(static_cast<float>(static_cast<int8_t>(w >> 16))),
                   static_cast<_Float16>(static_cast<float>(static_cast<int8_t>(w >> 24)))};
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// two floats -> a packed fp16 pair, each rounded to nearest
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b),
                                                c, 0, 0, 0);
}

// A page of one KV head is loaded in 18 parts: 8 of keys and 8 of values
// (1 KiB each: 64 lanes x 16 bytes), one of the 32 key scales and one of
// the 32 value scales (8 lanes x 16 bytes).  Loader wave h of H takes parts
// h, h + H, .. into its own registers, and every loader issues the same
// number of loads per page (past the 18, and for pages past the run, a
// load whose data is not used), so that the loads of four pages stay in
// flight in every loader alike.
constexpr int kCopies = 18;
constexpr int kRing = 4;          // pages in flight per workgroup
constexpr int kLoaders = 2;       // loader waves per workgroup
constexpr int kMaxRun = 1024;     // pages per workgroup (ids staged in LDS)

// A workgroup barrier for LDS only: this wave's LDS accesses are complete,
// then s_barrier; the loads of later pages still in flight are not waited
// for (__syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait until none of this wave's vector memory operations is in flight
__device__ __forceinline__ void wait_vm0() {
  __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8) | (0x0 << 14));
  asm volatile("" ::: "memory");
}

// Reductions over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48)
// with the gfx950 permlane swaps: each swap of a register with itself leaves
// x[l] in one result and x[l ^ J] in the other, on the VALU, so the softmax's
// maxima and sums take no LDS round trip (an LDS permute would also wait for
// every tile read issued before it).
__device__ __forceinline__ float group_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int H>
struct Pages {
  static constexpr int NI = (kCopies + H - 1) / H;  // loads per wave and page

  // this wave's parts of a page, as loaded
  struct Stage {
    u32x4 d[NI];
  };

  // page pp (of KV head g) into st, or, for real == false, loads of page
  // `dummy` whose data is never used; a page id outside the pool reads as
  // zeros (the buffer's size is then 0).  One 16-byte load per part, with
  // no branch (the part's source is selected), so that the compiler's wait
  // before a conversion counts exactly the loads issued after it.  A scale
  // part is 128 bytes: lanes 0..7 get 4 scales each, the rest zeros.
  template <int h>
  __device__ __forceinline__ static void load(const AttnArgs &a, int pp,
                                              bool real, int dummy, int g,
                                              Stage &st, int lane) {
    const int id = real ? pp : dummy;
    const bool ok = id >= 0 && id < a.pool;
    const size_t pg = ok ? static_cast<size_t>(id) * a.Hkv + g : 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int e0 = h + H * j;  // a constant once unrolled
      const int e = real && e0 < kCopies ? e0 : 0;
      const char *base =
          e < 8    ? reinterpret_cast<const char *>(a.kp + pg * kPage * kD)
          : e < 16 ? reinterpret_cast<const char *>(a.vp + pg * kPage * kD)
          : reinterpret_cast<const char *>((e == 16 ? a.ks : a.vs) + pg * kPage);
      const uint32_t bytes = !ok ? 0 : e < 16 ? kPage * kD : kPage * 4;
      const uint32_t off = (e < 16 ? 1024 * (e & 7) : 0) + 16 * lane;
      st.d[j] = load16(rsrc(base, bytes), off);
    }
  }
  // the same wave's parts turned into tiles: bf16 keys [token][dim] (row
  // stride kKStride), fp16 values [dim][slot] (row stride kVStride) with token
  // 4g+e of the low half at slot 8g+e and token 16+4g+e at slot 8g+4+e, then
  // the fp32 key and value scales
  template <int h>
  __device__ __forceinline__ static void convert(const Stage &st, char *buf,
                                                 int lane, float scale2) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int e = h + H * j;  // a constant once unrolled
      const u32x4 v = st.d[j];
      if (e < 8) {
        const int c = 64 * e + lane;  // token c / 16, dims 16 (c % 16) ..
        const int tok = c >> 4, d0 = 16 * (c & 15);
        const u32x2 w0 = i8x4_bf16(v.x), w1 = i8x4_bf16(v.y);
        const u32x2 w2 = i8x4_bf16(v.z), w3 = i8x4_bf16(v.w);
        u32x4 *dst = reinterpret_cast<u32x4 *>(buf + tok * kKStride + 2 * d0);
        dst[0] = u32x4{w0.x, w0.y, w1.x, w1.y};
        dst[1] = u32x4{w2.x, w2.y, w3.x, w3.y};
      } else if (e < 16) {
        const int f = 64 * (e - 8) + lane;  // dim f / 2, tokens 16 (f % 2) ..
        char *row = buf + kKBytes + (f >> 1) * kVStride + 8 * (f & 1);
        // tokens 16 h + 4 i .. +3 -> slots 8 i + 4 h .. +3
        *reinterpret_cast<u32x2 *>(row + 0) = i8x4_f16(v.x);
        *reinterpret_cast<u32x2 *>(row + 16) = i8x4_f16(v.y);
        *reinterpret_cast<u32x2 *>(row + 32) = i8x4_f16(v.z);
        *reinterpret_cast<u32x2 *>(row + 48) = i8x4_f16(v.w);
      } else if (e == 16) {
        // the key scales times the softmax scale (base 2)
        const f32x4 ks = __builtin_bit_cast(f32x4, v) * scale2;
        *reinterpret_cast<f32x4 *>(buf + kKBytes + kVBytes + 16 * lane) = ks;
      } else if (e == 17) {
        // the value scales, and after them (lane 8's first word, otherwise
        // a zero) the page's largest |value scale|: the maximum over lanes
        // 0..7 by quad swaps and a half-row mirror (DPP), taken from lane 0
        float mx = fmaxf(fmaxf(fabsf(__uint_as_float(v.x)), fabsf(__uint_as_float(v.y))),
                         fmaxf(fabsf(__uint_as_float(v.z)), fabsf(__uint_as_float(v.w))));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_update_dpp(
                           0, __float_as_int(mx), 0xB1, 0xF, 0xF, false)));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_update_dpp(
                           0, __float_as_int(mx), 0x4E, 0xF, 0xF, false)));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_update_dpp(
                           0, __float_as_int(mx), 0x141, 0xF, 0xF, false)));
        const uint32_t pmx = __builtin_amdgcn_readlane(__float_as_uint(mx), 0);
        u32x4 vv = v;
        vv.x = lane == 8 ? pmx : vv.x;
        *reinterpret_cast<u32x4 *>(buf + kKBytes + kVBytes + kScaleArea + 16 * lane) = vv;
      }
    }
  }
};

template <int G>
__global__ __launch_bounds__(64 * (G + kLoaders)) void tree_attn_kernel(AttnArgs a) {
  using P = Pages<kLoaders>;
  __shared__ __attribute__((aligned(16))) char tile0[kBufBytes];
  __shared__ __attribute__((aligned(16))) char tile1[kBufBytes];
  __shared__ int ids[kMaxRun];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n = lane & 15;   // tree node of this lane's score/output column
  const int gq = lane >> 4;  // lane group: k slots 8 gq .. 8 gq + 7
  // block = (head group, run, KV head), the KV head fastest: the head
  // groups of one (KV head, run) read the same pages, on the same XCD when
  // runs x KV heads is a multiple of 8
  const int per = a.splits * a.Hkv;
  const int hgrp = static_cast<int>(blockIdx.x) / per;
  const int bb = static_cast<int>(blockIdx.x) - hgrp * per;
  const int g = bb % a.Hkv;
  const int run = bb / a.Hkv;
  const int hq = (g * a.hsplit + hgrp) * G + (w < G ? w : 0);  // (loader waves: unused)
  const int pa = static_cast<int>(static_cast<int64_t>(a.pages) * run / a.splits);
  const int pb = static_cast<int>(static_cast<int64_t>(a.pages) * (run + 1) / a.splits);
  const int len = pb - pa;  // 1 .. kMaxRun (the plan sees to it)

  // queries of this wave's head as the B operand: lane (n, gq), step s holds
  // q[n][hq][32 s + 8 gq .. +7]; nodes >= M read zeros
  const __amdgpu_buffer_rsrc_t qr =
      rsrc(a.q, static_cast<uint32_t>(a.M) * a.Hq * kD * 2);
  u32x4 qreg[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qreg[s] = load16(qr, static_cast<uint32_t>(((n * a.Hq + hq) * kD + 32 * s + 8 * gq) * 2));
  const uint32_t anc = n < a.M ? a.anc[n] : 0u;
  // the run's page ids, staged in LDS before any copy is issued
  bool bad_page = false;
  for (int i = tid; i < len; i += 64 * (G + kLoaders)) {
    const int pp = a.page_table[pa + i];
    ids[i] = pp;
    bad_page |= pp < 0 || pp >= a.pool;
  }
  if (__ballot(bad_page) != 0 && lane == 0 && a.status != nullptr)
    a.status[0] = Q4_EINVAL;
  __syncthreads();

  auto page_of = [&](int i) { return __builtin_amdgcn_readfirstlane(ids[i]); };
  const f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  f32x4 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = fz;
  // The reference maximum starts at the lowest finite float rather than
  // -inf, so that p - m is never inf - inf: a masked score (-inf) then
  // gives exp2 = 0 with no test, and the first visible score moves m.
  float m = -FLT_MAX, lsum = 0.0f;
  // A power of two at or above every value scale seen so far: the value
  // product's B operand is P'' = p * v_scale / vlim, at most 2^8, so fp16
  // carries it without overflow whatever the scales, and vlim tracks the
  // largest scale so that typical terms stay normal fp16 numbers.  When a
  // page's scale passes vlim, vlim moves up to a power of two at or above it
  // and the running output is rescaled by the (exact) ratio of the two.
  float vlim = 0x1.0p-126f;

  auto compute_page = [&](const char *buf, int lp) {
    // scores S^T[token 16 c + 4 gq + r][node n]
    f32x4 sc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      sc[c] = fz;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 ka = *reinterpret_cast<const u32x4 *>(
            buf + (16 * c + n) * kKStride + 2 * (32 * s + 8 * gq));
        sc[c] = mfma(ka, qreg[s], sc[c]);
      }
    }
    const float *kscale = reinterpret_cast<const float *>(buf + kKBytes + kVBytes);
    const float *vscale = kscale + kScaleArea / 4;
    float p[8], vsc[8];
    const int pos0 = kPage * lp;
    const bool all_visible = pos0 + kPage <= a.ctx;  // uniform
    float pm = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f32x4 ksv = *reinterpret_cast<const f32x4 *>(kscale + 16 * c + 4 * gq);
      const f32x4 vsv = *reinterpret_cast<const f32x4 *>(vscale + 16 * c + 4 * gq);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * c + 4 * gq + r;
        float s = sc[c][r] * ksv[r];  // ksv: key scale x softmax scale
        bool vis = true;
        if (!all_visible) {
          const int t = pos0 + tok - a.ctx;
          vis = t < 0 || (t < a.M && ((anc >> t) & 1u));
        }
        s = vis ? s : -INFINITY;
        p[4 * c + r] = s;
        vsc[4 * c + r] = vsv[r];
        pm = fmaxf(pm, s);
      }
    }
    pm = group_max(pm);
    // The reference maximum m moves only when some node's score passes it
    // by more than kLazyMax (base 2), so the exponentials stay below
    // 2^kLazyMax and the running output is rescaled on few pages.  The
    // final division by the sum (and the merge of runs) removes any common
    // reference, so the result is the same softmax.
    if (__ballot(pm > m + kLazyMax) != 0) {  // a wave-uniform test
      const float mn = fmaxf(m, pm);
      // exp2 of -FLT_MAX - mn is 0 at a node's first visible score, and
      // 1 where nothing is visible yet (mn = m)
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      lsum *= alpha;
      m = mn;
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] *= alpha;
    }
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(p[i] - m);  // masked: exp2(-inf) = 0
      ps += p[i];
    }
    lsum += ps;
    // the page's largest value scale, left by the loader after the scales
    const float vm = vscale[kPage];
    if (__ballot(vm > vlim) != 0) {  // wave-uniform: vm is the same in every lane
      int ex;
      (void)frexpf(vm, &ex);  // vm < 2^ex
      const float nl = ldexpf(1.0f, ex);
      const float f = vlim / nl;  // a power of two, exact
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] *= f;
      vlim = nl;
    }
    const float rl = 1.0f / vlim;  // exact: vlim is a power of two
    // P''^T as the B operand: slot 8 gq + e <- token 4 gq + e (e < 4) and
    // 16 + 4 gq + e - 4 (e >= 4), exactly the order of p[].  Each P'' is
    // rounded to fp16 (11 significant bits, a relative 2^-11 at most) and
    // meets the exact fp16 values in one MFMA per value tile.
    u32x4 pf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pf[i] = pack_f16(p[2 * i] * vsc[2 * i] * rl, p[2 * i + 1] * vsc[2 * i + 1] * rl);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const u32x4 va = *reinterpret_cast<const u32x4 *>(
          buf + kKBytes + (16 * dt + n) * kVStride + 16 * gq);
      o[dt] = mfma_f16(va, pf, o[dt]);
    }
  };

  // Waves G and G + 1 load the pages and turn them into bf16 tiles; waves
  // 0 .. G - 1 (one per query head) only compute, so that the compute units'
  // MFMA work is not held up by conversions.  Page i of the run is loaded
  // into stage i % 4 (a loader's registers) and turned into tile i % 2.
  // Step i: the loaders turn their parts of page i + 1 into its tile (the
  // loads of pages i + 2 .. i + 4 stay in flight: the compiler's wait
  // before the conversion counts them) and load page i + 5 (or unused
  // data) into the stage just freed, while the compute waves compute page
  // i; then one barrier of all waves: tile i % 2 is free for page i + 2 and
  // tile (i + 1) % 2 complete.
  if (w >= G) {
    // the loader's index as a constant: its parts (and so every branch on
    // them) are known at compile time
    auto loader = [&](auto hc) {
      constexpr int h = decltype(hc)::value;
      using Stage = typename P::Stage;
      const int first = page_of(0);
      auto load_page = [&](int i, Stage &st) {
        const bool real = i < len;
        P::template load<h>(a, real ? page_of(i) : first, real, first, g, st, lane);
      };
      Stage st0, st1, st2, st3;
      load_page(0, st0);
      load_page(1, st1);
      load_page(2, st2);
      load_page(3, st3);
      P::template convert<h>(st0, tile0, lane, a.scale2);
      load_page(kRing, st0);
      lds_barrier();
      // A stage is reloaded right after its conversion, so that its
      // registers are never free between the two (a temporary there would
      // make the compiler wait for every load in flight).  Past the run the
      // conversion writes unused data into a tile no wave reads any more.
      auto step = [&](int i, Stage &st, char *tile) {
        P::template convert<h>(st, tile, lane, a.scale2);
        load_page(i + 1 + kRing, st);
        lds_barrier();
      };
      // whole rounds of four steps with no exit inside (an exit would make
      // the compiler's waits at the loop's head drain the loads), then the
      // last steps
      int i = 0;
      for (; i + kRing <= len; i += kRing) {
        step(i, st1, tile1);
        step(i + 1, st2, tile0);
        step(i + 2, st3, tile1);
        step(i + 3, st0, tile0);
      }
      if (i < len) step(i, st1, tile1);
      if (i + 1 < len) step(i + 1, st2, tile0);
      if (i + 2 < len) step(i + 2, st3, tile1);
      wait_vm0();  // the unused loads past the run too
    };
    static_assert(kLoaders == 2, "two loader instantiations");
    if (w == G)
      loader(std::integral_constant<int, 0>{});
    else
      loader(std::integral_constant<int, 1>{});
    return;
  }
  lds_barrier();  // page 0 is in tile 0
  for (int i = 0; i < len; i += 2) {
    compute_page(tile0, pa + i);
    lds_barrier();
    if (i + 1 >= len) break;
    compute_page(tile1, pa + i + 1);
    lds_barrier();
  }

  lsum = group_sum(lsum);
  if (n >= a.M) return;
  if (a.splits == 1) {
    const float inv = vlim / lsum;
    float *dst = a.out + (static_cast<size_t>(n) * a.Hq + hq) * kD + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
      *reinterpret_cast<f32x4 *>(dst + 16 * dt) = o[dt] * inv;
  } else {
    const size_t row = (static_cast<size_t>(run) * a.Hq + hq) * a.M + n;
    float *dst = a.part + row * kD + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
      *reinterpret_cast<f32x4 *>(dst + 16 * dt) = o[dt] * vlim;
    if (gq == 0) {
      float *ml = a.part + static_cast<size_t>(a.splits) * a.Hq * a.M * kD;
      ml[2 * row] = m;
      ml[2 * row + 1] = lsum;
    }
  }
}

// out[n][hq][d] = sum_r 2^(m_r - m) O_r[d] / sum_r 2^(m_r - m) l_r, one
// workgroup per (node, query head): the runs' weights go to LDS first, then
// every thread sums its dimension over the runs with eight loads in flight.
constexpr int kCombineMaxRuns = 2048;
constexpr int kCombinePre = 16;  // runs whose partial outputs are all requested at once

__global__ __launch_bounds__(256) void attn_combine_kernel(const float *part,
                                                           float *out, int M,
                                                           int Hq, int splits) {
  __shared__ float wgt[kCombineMaxRuns];
  __shared__ float red[8];
  const int row = blockIdx.x;  // hq * M + n
  const int hq = row / M, n = row % M;
  const int d = threadIdx.x;
  const size_t rows = static_cast<size_t>(Hq) * M;
  const float *ml = part + static_cast<size_t>(splits) * rows * kD;
  const float *src = part + static_cast<size_t>(row) * kD + d;
  if (splits <= kCombinePre) {
    // Few runs (short contexts): every partial output is requested at once,
    // beside the runs' (max, sum) pairs, so the merge waits for one memory
    // round trip instead of three; same sums in the same order.
    float pv[kCombinePre];
#pragma unroll
    for (int i = 0; i < kCombinePre; ++i)
      pv[i] = src[static_cast<size_t>(i < splits ? i : splits - 1) * rows * kD];
    const int dr = d < splits ? d : splits - 1;
    const float2 pr = *reinterpret_cast<const float2 *>(&ml[2 * (dr * rows + row)]);
    const float mr = d < splits ? pr.x : -INFINITY;
    float mx = mr;
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((d & 63) == 0) red[d >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float w = mr == -INFINITY ? 0.0f : exp2f(mr - mx);
    if (d < splits) wgt[d] = w;
    float den = d < splits ? w * pr.y : 0.0f;
    for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
    __syncthreads();
    if ((d & 63) == 0) red[4 + (d >> 6)] = den;
    __syncthreads();
    den = red[4] + red[5] + red[6] + red[7];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombinePre; ++i)
      if (i < splits) acc += wgt[i] * pv[i];
    out[(static_cast<size_t>(n) * Hq + hq) * kD + d] = acc / den;
    return;
  }
  float mx = -INFINITY;
  for (int r = d; r < splits; r += 256) mx = fmaxf(mx, ml[2 * (r * rows + row)]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((d & 63) == 0) red[d >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float den = 0.0f;
  for (int r = d; r < splits; r += 256) {
    const float mr = ml[2 * (r * rows + row)];
    const float w = mr == -INFINITY ? 0.0f : exp2f(mr - mx);
    wgt[r] = w;
    den += w * ml[2 * (r * rows + row) + 1];
  }
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  __syncthreads();
  if ((d & 63) == 0) red[4 + (d >> 6)] = den;
  __syncthreads();
  den = red[4] + red[5] + red[6] + red[7];
  float acc = 0.0f;
  int r = 0;
  for (; r + 8 <= splits; r += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = src[(r + i) * rows * kD];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += wgt[r + i] * v[i];
  }
  for (; r < splits; ++r) acc += wgt[r] * src[r * rows * kD];
  out[(static_cast<size_t>(n) * Hq + hq) * kD + d] = acc / den;
}

}  // namespace

// splits: runs of about 8 pages, but at least 16 runs (the pages allowing)
// and at most one per CU for each KV head; the launch then gives each (KV
// head, run) as many workgroups, each with a share of the query heads, as
// the CUs hold.  Measured at 16 nodes, 24/4 heads: 16 runs in 3 head groups
// at 2K and 4K (15.3 and 19.1 us against 16.6 and 20.3 with 16 and 32 runs
// in 2 groups), 32 runs in 2 groups at 8K, 64 runs at 16K and 32K.
int attn_splits(int pages, int Hkv, int cus) {
  int s = pages / 8 > 16 ? pages / 8 : 16;
  const int most = (cus + Hkv - 1) / Hkv;
  if (s > most) s = most;
  if (s > pages) s = pages;
  const int least = (pages + kMaxRun - 1) / kMaxRun;
  if (s < least) s = least;
  return s < 1 ? 1 : s;
}

}  // namespace q4v

namespace {

int attn_shape(int M, int Hq, int Hkv, int D, int64_t ctx_len, int *pages) {
  if (M < 1 || M > Q4_ATTN_MAX_NODES || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      D != Q4_ATTN_HEAD_DIM || ctx_len < 0 || ctx_len > 0x7FFFFFFFLL - 64)
    return Q4_EINVAL;
  const int G = Hq / Hkv;
  if (G != 2 && G != 4 && G != 6 && G != 8) return Q4_EINVAL;
  *pages = static_cast<int>((ctx_len + M + Q4_ATTN_PAGE - 1) / Q4_ATTN_PAGE);
  return Q4_OK;
}

}  // namespace

extern "C" int q4_tree_attn_plan(int M, int Hq, int Hkv, int D,
                                 int64_t ctx_len, int splits,
                                 int *splits_used,
                                 uint64_t *workspace_bytes) {
  int pages = 0;
  if (splits_used == nullptr || workspace_bytes == nullptr || splits < 0)
    return Q4_EINVAL;
  const int st = attn_shape(M, Hq, Hkv, D, ctx_len, &pages);
  if (st != Q4_OK) return st;
  int s = splits > 0 ? splits : q4v::attn_splits(pages, Hkv, q4v::device_cus());
  if (s > pages) s = pages;
  if ((pages + s - 1) / s > q4v::kMaxRun || s > q4v::kCombineMaxRuns)
    return Q4_EINVAL;  // runs too long, or too many of them
  if (static_cast<int64_t>(s) * Hkv > 0x7FFFFFFF) return Q4_EINVAL;
  *splits_used = s;
  *workspace_bytes = s == 1 ? 0
                            : static_cast<uint64_t>(s) * Hq * M *
                                  (Q4_ATTN_HEAD_DIM + 2) * 4;
  return Q4_OK;
}

extern "C" int q4_tree_attn(const void *q, int M, int Hq, int Hkv, int D,
                            const int8_t *k_pages, const int8_t *v_pages,
                            const float *k_scale, const float *v_scale,
                            const int32_t *page_table, int pool_pages,
                            int64_t ctx_len, const uint32_t *anc, float scale,
                            float *out, int splits, void *workspace,
                            uint64_t workspace_bytes, int32_t *status,
                            void *stream) {
  int s = 0;
  uint64_t need = 0;
  int st = q4_tree_attn_plan(M, Hq, Hkv, D, ctx_len, splits, &s, &need);
  if (st != Q4_OK) return st;
  if (q == nullptr || k_pages == nullptr || v_pages == nullptr ||
      k_scale == nullptr || v_scale == nullptr || page_table == nullptr ||
      anc == nullptr || out == nullptr || pool_pages < 1 ||
      !(scale > 0.0f) || !(scale < 3.0e38f) ||
      (need > 0 && (workspace == nullptr || workspace_bytes < need)))
    return Q4_EINVAL;
  if ((static_cast<uint64_t>(pool_pages) * Hkv * Q4_ATTN_PAGE * Q4_ATTN_HEAD_DIM) >>
      62)
    return Q4_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(k_pages) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(v_pages) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(k_scale) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(v_scale) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(page_table) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(anc) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(status) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return Q4_EALIGN;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  const int pages =
      static_cast<int>((ctx_len + M + Q4_ATTN_PAGE - 1) / Q4_ATTN_PAGE);
  q4v::AttnArgs a{static_cast<const uint16_t *>(q), k_pages, v_pages, k_scale,
                  v_scale, page_table, anc, out,
                  static_cast<float *>(workspace), status, M, Hq, Hkv,
                  pool_pages, static_cast<int>(ctx_len), pages, s,
                  scale * q4v::kLog2e, 1};
  const int G = Hq / Hkv;
  // Head groups: when the runs leave CUs idle (short contexts), each (KV
  // head, run) takes h workgroups of G / h query heads each, the largest h
  // whose workgroups the CUs hold: each page is computed by h times as many
  // SIMDs and read h times, after the first mostly from the XCD's L2.
  for (int h : {6, 4, 3, 2})
    if (G % h == 0 && static_cast<int64_t>(h) * s * Hkv <= q4v::device_cus()) {
      a.hsplit = h;
      break;
    }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(s * Hkv * a.hsplit));
  switch (G / a.hsplit) {
    case 1:
      hipLaunchKernelGGL(q4v::tree_attn_kernel<1>, grid, dim3(64 + 64 * q4v::kLoaders), 0, hs, a);
      break;
    case 2:
      hipLaunchKernelGGL(q4v::tree_attn_kernel<2>, grid, dim3(128 + 64 * q4v::kLoaders), 0, hs, a);
      break;
    case 3:
      hipLaunchKernelGGL(q4v::tree_attn_kernel<3>, grid, dim3(192 + 64 * q4v::kLoaders), 0, hs, a);
      break;
    case 4:
      hipLaunchKernelGGL(q4v::tree_attn_kernel<4>, grid, dim3(256 + 64 * q4v::kLoaders), 0, hs, a);
      break;
    case 6:
      hipLaunchKernelGGL(q4v::tree_attn_kernel<6>, grid, dim3(384 + 64 * q4v::kLoaders), 0, hs, a);
      break;
    default:
      hipLaunchKernelGGL(q4v::tree_attn_kernel<8>, grid, dim3(512 + 64 * q4v::kLoaders), 0, hs, a);
      break;
  }
  if (hipGetLastError() != hipSuccess) return Q4_ELAUNCH;
  if (s > 1) {
    hipLaunchKernelGGL(q4v::attn_combine_kernel, dim3(M * Hq), dim3(256), 0,
                       hs, static_cast<const float *>(workspace), out, M, Hq,
                       s);
    if (hipGetLastError() != hipSuccess) return Q4_ELAUNCH;
  }
  return Q4_OK;
}
