// q4verify_kernels.hip -- gfx950 kernels of the Q4 verify GEMM and the
// device entry points of the C ABI.
//
// The GEMM (y = x * W^T, W in the planar group-affine Q4 layout, M <= 16
// activation rows) is bound by the weight stream: 9 bytes per 16 weights are
// read once and every activation row is multiplied while the codes are in
// registers (qwen-spec page, Notes: one read of each weight tile serves all
// rows; Splash engine article, "Why Apple silicon, and why not the M5": the
// verify rows make it a GEMM that still needs little compute per byte).
//
// Per wave: a tile of 16 output rows x a range of 64-input groups.  For each
// group the wave runs two v_mfma_f32_16x16x32_bf16 on the codes:
//   A = x (16 activation rows, rows >= M are zero),  B = codes as bf16,
// with the group scale applied afterwards, since it differs per group:
//   y[m,n] += s[n,g] * sum_k x[m,k] q[n,k]  +  b[n,g] * sum_k x[m,k].
// Codes reach bf16 without a conversion instruction: OR-ing a 4-bit code into
// the mantissa of bf16 128.0 (0x4300) gives exactly 128 + q.  The extra
// 128 * sum_k x is cancelled by seeding the accumulator with an MFMA against
// a constant -128 operand, which also yields the group sums of x that the
// bias term needs (XN = -128 * sum_k x, so b * sum_k x = (-b/128) * XN).
// Products of bf16 x with 128 + q are exact; accumulation is fp32.
//
// To make the unpack cheap the 8 codes of a 32-bit word are paired as
// (q0,q4) (q1,q5) (q2,q6) (q3,q7) -- one mask per pair -- and the activation
// operand is permuted the same way with v_perm_b32, so both operands agree on
// which input sits in which MFMA k-slot.
#include <hip/hip_runtime.h>

#include <atomic>

#include "q4v_internal.h"
#include "q4v_select.h"

// Scratch of q4_gemm_verify_tiled_noalloc: the partial products of parts
// 1 .. P-1 of a K split, Q4_NOALLOC_SCRATCH_BYTES per device, held by each
// GPU the library runs on until the process ends.  Host code never passes
// this name to a kernel (on the host it is only a handle of the symbol): it
// uses the device address that noalloc_scratch() looks up once per device.
static __device__ __align__(256) float scratch[Q4_NOALLOC_SCRATCH_BYTES / 4];

namespace q4v {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// A 32-bit word as a bf16 pair.  (Passing a vector element straight to
// __builtin_bit_cast made the compiler read element 0 for every index.)
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2, w);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kMagic128Pair = 0x43004300u;  // bf16 (128.0, 128.0)
constexpr uint32_t kNeg128Pair = 0xC300C300u;    // bf16 (-128.0, -128.0)
constexpr float kMinusInv128 = -0.0078125f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// The two constants of the unpack, kept in registers so that each
// (code pair & mask) | magic is one v_and_or_b32 (gfx9 VOP3 encodings take
// no literal operands, so with literals it would take two instructions).
struct UnpackConsts {
  uint32_t mask;   // scalar register
  uint32_t magic;  // vector register
};

__device__ __forceinline__ UnpackConsts unpack_consts() {
  UnpackConsts c;
  c.mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.magic) : "s"(kMagic128Pair));
  return c;
}

// Codes q0..q7 (bits 4i..4i+3 of w) -> bf16 pairs (128+q0, 128+q4),
// (128+q1, 128+q5), (128+q2, 128+q6), (128+q3, 128+q7).
__device__ __forceinline__ u32x4 unpack_codes(uint32_t w, UnpackConsts c) {
  u32x4 r;
  r.x = (w & c.mask) | c.magic;
  r.y = ((w >> 4) & c.mask) | c.magic;
  r.z = ((w >> 8) & c.mask) | c.magic;
  r.w = ((w >> 12) & c.mask) | c.magic;
  return r;
}

// Eight consecutive bf16 activations (x0,x1)(x2,x3)(x4,x5)(x6,x7) ->
// (x0,x4)(x1,x5)(x2,x6)(x3,x7), the k-slot order of unpack_codes.
__device__ __forceinline__ u32x4 pair_activations(u32x4 d) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
  return r;
}

// A per-lane value the compiler must treat as changed here: keeps the
// values derived from it inside a loop (one register held across the loop
// instead of every derived offset).
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// floor(a / d) for 0 <= a < 2^24, 1 <= d < 2^24 and a / d < 2^21 (a few
// instructions instead of an integer division): the fp32 product with the
// reciprocal lies within 0.2 of a / d, so the truncated quotient is off by
// at most one, and one step on the remainder corrects it.
__device__ __forceinline__ int small_div(int a, int d) {
  int q = static_cast<int>(static_cast<float>(a) *
                           __builtin_amdgcn_rcpf(static_cast<float>(d)));
  const int r = a - q * d;
  q += static_cast<int>(r >= d) - static_cast<int>(r < 0);
  return q;
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
      0);
}

// One workgroup = NTW tiles of 16 output rows x KSW waves splitting the
// groups of K; U groups are loaded ahead of their use.
//
// Lane l of a wave: j = l % 16, kb = l / 16.  MFMA 16x16x32 operand layout:
//   A (16 x 32): lane holds row j, k-slots 8*kb .. 8*kb+7  -> x row m = j;
//   B (32 x 16): lane holds column j, k-slots 8*kb .. +7   -> W row n0 + j;
//   C (16 x 16): lane holds column j, rows 4*kb .. 4*kb+3 -> y[4kb+r][n0+j].
// In group g the first MFMA covers inputs 64g + 16kb + 0..7 and the second
// 64g + 16kb + 8..15 of each lane, i.e. 8 code bytes per lane per group.
template <int NTW, int KSW, int U>
__global__ __launch_bounds__(64 * NTW * KSW) void gemm_verify_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ W,
    float *__restrict__ y, int M, int N, int K) {
  const int G = K >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nt = wave % NTW;
  const int ks = wave / NTW;
  const int j = lane & 15;
  const int kb = lane >> 4;
  const int n0 = (blockIdx.x * NTW + nt) * 16;
  const int n = n0 + j;
  const bool row_ok = n < N;
  const bool x_ok = j < M;
  const int gb = static_cast<int>((static_cast<int64_t>(G) * ks) / KSW);
  const int ge = static_cast<int>((static_cast<int64_t>(G) * (ks + 1)) / KSW);

  const uint64_t NK = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  const uint64_t nrow = row_ok ? static_cast<uint64_t>(n) : 0;
  const uint8_t *codes = W + nrow * static_cast<uint64_t>(K >> 1) + kb * 8;
  const uint16_t *scales =
      reinterpret_cast<const uint16_t *>(W + NK / 2) + nrow * G;
  const uint16_t *biases =
      reinterpret_cast<const uint16_t *>(W + NK / 2 + NK / 32) + nrow * G;
  const uint16_t *xrow =
      x + static_cast<uint64_t>(x_ok ? j : 0) * static_cast<uint64_t>(K) +
      kb * 16;

  const u32x4 neg = {kNeg128Pair, kNeg128Pair, kNeg128Pair, kNeg128Pair};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  const UnpackConsts uc = unpack_consts();
  f32x4 acc = fzero;

  for (int g = gb; g < ge; g += U) {
    u32x2 cw[U];
    uint32_t sv[U], bv[U];
    u32x4 xa[U], xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gg = g + u;
      const bool ok = gg < ge;
      cw[u] = u32x2{0u, 0u};
      sv[u] = 0u;
      bv[u] = 0u;
      xa[u] = zero4;
      xb[u] = zero4;
      if (ok && row_ok) {
        cw[u] = *reinterpret_cast<const u32x2 *>(codes +
                                                 static_cast<uint64_t>(gg) * 32);
        sv[u] = scales[gg];
        bv[u] = biases[gg];
      }
      if (ok && x_ok) {
        const uint16_t *xp = xrow + static_cast<uint64_t>(gg) * 64;
        xa[u] = *reinterpret_cast<const u32x4 *>(xp);
        xb[u] = *reinterpret_cast<const u32x4 *>(xp + 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 a0 = pair_activations(xa[u]);
      const u32x4 a1 = pair_activations(xb[u]);
      f32x4 xn = mfma16x16x32(a0, neg, fzero);
      xn = mfma16x16x32(a1, neg, xn);
      f32x4 t = mfma16x16x32(a0, unpack_codes(cw[u].x, uc), xn);
      t = mfma16x16x32(a1, unpack_codes(cw[u].y, uc), t);
      const float s = bf16_to_f32(sv[u]);
      const float bn = bf16_to_f32(bv[u]) * kMinusInv128;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[r] = __builtin_fmaf(bn, xn[r], acc[r]);
        acc[r] = __builtin_fmaf(s, t[r], acc[r]);
      }
    }
  }

  if constexpr (KSW > 1) {
    __shared__ f32x4 partial[KSW][NTW][64];
    partial[ks][nt][lane] = acc;
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int s = 1; s < KSW; ++s) acc += partial[s][nt][lane];
  }
  if (row_ok) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = kb * 4 + r;
      if (m < M) y[static_cast<uint64_t>(m) * N + n] = acc[r];
    }
  }
}

// The same product for weights in Q4_LAYOUT_TILED16.  A record (16 rows x 4
// groups, 2304 bytes = 144 16-byte units) is laid out so that lane l's
// operands are unit l (groups 0-1), unit 64 + l (groups 2-3) and unit
// 128 + j (the row's four scale/bias pairs): every load of a wave is a
// contiguous, fully used 1 KB (codes) or 256 B (scales and biases) block.
// The repack stores each code word's even inputs in its low half and its odd
// inputs in its high half, so the code pairs come out of unpack_codes in the
// activations' own order and the activation operand needs no permutation.
// Each wave multiplies TNT tiles with one activation operand over a
// contiguous range of records, and issues the loads of record r + 1 before
// it computes record r (two register stages used in turn).
//
// Loads go through buffer resources bounded to the wave's own range: a load
// past the range returns zeros without touching memory.  That makes the
// prefetch past the last record free, and gives activation rows m >= M (and
// tiles past N) zeros without a branch.  Weight loads are non-temporal: each
// byte is used once and should not displace the activations from the caches.
constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer descriptor format
constexpr int kNonTemporal = 2;           // cache policy bit of the load

template <int kPolicy>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r,
                                               uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPolicy));
}

template <int TNT>
struct TiledStage {
  u32x4 c0[TNT], c1[TNT], sb[TNT];
  u32x4 xa[4], xb[4];
};

template <int TNT, int NTW, int KSW>
__global__ __launch_bounds__(64 * NTW * KSW) void gemm_tiled_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ Wt,
    float *__restrict__ y, int M, int N, int K) {
  const int T = N >> 4;
  const int Q = K >> 8;
  const int lane = threadIdx.x & 63;
  // wave-uniform, so the buffer descriptors below live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = wave % NTW;
  const int ks = wave / NTW;
  const int j = lane & 15;
  const int kb = lane >> 4;
  const int set = blockIdx.x * NTW + nt;
  const int qb = static_cast<int>((static_cast<int64_t>(Q) * ks) / KSW);
  const int qe = static_cast<int>((static_cast<int64_t>(Q) * (ks + 1)) / KSW);
  const int nq = qe - qb;

  __amdgpu_buffer_rsrc_t wr[TNT];
#pragma unroll
  for (int t = 0; t < TNT; ++t) {
    const int tile = set * TNT + t;
    const bool ok = tile < T;
    const uint8_t *base =
        Wt + (static_cast<uint64_t>(ok ? tile : 0) * Q + qb) * kRecordBytes;
    wr[t] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(base), 0, ok ? nq * kRecordBytes : 0,
        kBufferWord3);
  }
  // activations: rows >= M fall past the M*K*2 bytes of the resource
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x), 0,
      static_cast<int>(static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u),
      kBufferWord3);
  const uint32_t xoff =
      (static_cast<uint32_t>(j) * K + kb * 16 + static_cast<uint32_t>(qb) * 256) *
      2;

  const u32x4 neg = {kNeg128Pair, kNeg128Pair, kNeg128Pair, kNeg128Pair};
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  const UnpackConsts uc = unpack_consts();
  f32x4 acc[TNT];
#pragma unroll
  for (int t = 0; t < TNT; ++t) acc[t] = fzero;

  auto load = [&](int q, TiledStage<TNT> &st) {
    const uint32_t rq = static_cast<uint32_t>(q) * kRecordBytes;
#pragma unroll
    for (int t = 0; t < TNT; ++t) {
      st.c0[t] = buffer_load16<kNonTemporal>(wr[t], lane * 16, rq);
      st.c1[t] = buffer_load16<kNonTemporal>(wr[t], 1024 + lane * 16, rq);
      st.sb[t] = buffer_load16<kNonTemporal>(wr[t], 2048 + j * 16, rq);
    }
    const uint32_t xq = xoff + static_cast<uint32_t>(q) * 512;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      st.xa[gi] = buffer_load16<0>(xr, xq + gi * 128, 0);
      st.xb[gi] = buffer_load16<0>(xr, xq + gi * 128 + 16, 0);
    }
  };

  auto compute = [&](const TiledStage<TNT> &st) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const u32x4 a0 = st.xa[gi];
      const u32x4 a1 = st.xb[gi];
      f32x4 xn = mfma16x16x32(a0, neg, fzero);
      xn = mfma16x16x32(a1, neg, xn);
#pragma unroll
      for (int t = 0; t < TNT; ++t) {
        const u32x4 cw = gi < 2 ? st.c0[t] : st.c1[t];
        const uint32_t w0 = (gi & 1) ? cw.z : cw.x;
        const uint32_t w1 = (gi & 1) ? cw.w : cw.y;
        f32x4 tq = mfma16x16x32(a0, unpack_codes(w0, uc), xn);
        tq = mfma16x16x32(a1, unpack_codes(w1, uc), tq);
        const uint32_t sbw = st.sb[t][gi];
        const float s = __uint_as_float(sbw << 16);
        const float bn = __uint_as_float(sbw & 0xFFFF0000u) * kMinusInv128;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[t][r] = __builtin_fmaf(bn, xn[r], acc[t][r]);
          acc[t][r] = __builtin_fmaf(s, tq[r], acc[t][r]);
        }
      }
    }
  };

  // Both stages are computed unconditionally: a stage past the range holds
  // zeros and adds exactly zero, and a branch would let the compiler sink the
  // prefetch next to its use.
  // The scheduling barriers keep each stage's loads together, issued before
  // the other stage's arithmetic, so one whole stage is always in flight.
  TiledStage<TNT> sa, sbuf;
  load(0, sa);
  for (int q = 0; q < nq; q += 2) {
    load(q + 1, sbuf);  // past the range: zeros, no memory traffic
    __builtin_amdgcn_sched_barrier(0);
    compute(sa);
    __builtin_amdgcn_sched_barrier(0);
    load(q + 2, sa);
    __builtin_amdgcn_sched_barrier(0);
    compute(sbuf);
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (KSW > 1) {
    __shared__ f32x4 partial[KSW][NTW][TNT][64];
#pragma unroll
    for (int t = 0; t < TNT; ++t) partial[ks][nt][t][lane] = acc[t];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int s = 1; s < KSW; ++s)
#pragma unroll
      for (int t = 0; t < TNT; ++t) acc[t] += partial[s][nt][t][lane];
  }
#pragma unroll
  for (int t = 0; t < TNT; ++t) {
    const int tile = set * TNT + t;
    if (tile < T) {
      const int n = tile * 16 + j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = kb * 4 + r;
        if (m < M) y[static_cast<uint64_t>(m) * N + n] = acc[t][r];
      }
    }
  }
}

// The same product with the activations resident in LDS.  The workgroups
// form P groups of Gt, one group per part of K: part p is the records
// [Q p / P, Q (p+1) / P) of every tile, at most 20 of them (16 rows x 20 x 256
// bf16 = the 160 KB of a CU's LDS).  P = 1 whenever K <= 5120.  One
// workgroup per CU:
//  * it copies its part of x once into LDS with direct-to-LDS buffer loads:
//    block (q, gi, r) is 1 KB and its 16-byte slot s holds the eight inputs
//    256q + 64gi + 8(s%8) .. +7 of row 8r + s/8 (q counted within the part),
//    so one copy instruction moves 8 whole 128-byte rows (lane l lands at
//    block + 16 l; rows >= M fall past the resource and arrive as zeros).
//    The MFMA operand of lane (j, kb), half h, is slot 8(j%8) + 2kb + h of
//    block (q, gi, j/8);
//  * it owns whole tiles [t0, t1) of its group, i.e. U = (t1 - t0) * nq
//    records in tile-major order, and gives each of its W waves a contiguous
//    range of them, so every wave streams the same number of records (+-1)
//    and no wave reloads activation operands from the memory hierarchy;
//  * a tile that lies wholly inside one wave's range is written by that wave
//    as soon as its last record is done; a tile split between waves is
//    reduced after the loop through LDS, in wave order, by the wave holding
//    the tile's first record;
//  * part 0 writes y, part p > 0 its own M x N slice of the workspace, and
//    reduce_parts_kernel then adds the slices to y in part order.
// Summation orders depend only on (N, K, P), so results do not depend on M
// and repeated calls are bitwise equal.
// Weight records go through S register stages: the loads of record i + S - 1
// are issued before record i is multiplied.
typedef __attribute__((address_space(3))) void lds_void;

template <int W, int S, int RT>
__global__ __launch_bounds__(64 * W) void gemm_resident_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ Wt,
    float *__restrict__ y, float *__restrict__ ws, int M, int N, int K,
    int P, int Gt) {
  __shared__ u32x4 lds[kLdsBytes / 16];
  const int T = N >> 4;
  const int Q = K >> 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;
  const int kb = lane >> 4;
  const int p = blockIdx.x / Gt;
  const int bt = blockIdx.x % Gt;
  const int qa = static_cast<int>(static_cast<int64_t>(Q) * p / P);
  const int nq = static_cast<int>(static_cast<int64_t>(Q) * (p + 1) / P) - qa;
  const int t0 = static_cast<int>(static_cast<int64_t>(T) * bt / Gt);
  const int t1 = static_cast<int>(static_cast<int64_t>(T) * (bt + 1) / Gt);
  const int U = (t1 - t0) * nq;
  const int u0 = static_cast<int>(static_cast<int64_t>(U) * wave / W);
  const int u1 = static_cast<int>(static_cast<int64_t>(U) * (wave + 1) / W);

  // activations -> LDS, block f = (4q + gi) 2RT + r (rows 8r .. 8r+7)
  // copied by wave f % W
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x), 0,
      static_cast<int>(static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u),
      kBufferWord3);
  const uint32_t xslot =
      (static_cast<uint32_t>(lane >> 3) * K + 8 * (lane & 7)) * 2;
  for (int f = wave; f < 8 * RT * nq; f += W) {
    const int q = qa + f / (8 * RT), gi = (f / (2 * RT)) & 3, r = f % (2 * RT);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xr, (lds_void *)&lds[f * 64], 16,  // address-space cast
        xslot + static_cast<uint32_t>(8 * r) * K * 2,
        static_cast<uint32_t>(256 * q + 64 * gi) * 2, 0, 0);
  }

  // This wave's weights: a resource over the whole tiles its range touches;
  // a record past the range gets an offset past the resource, so that
  // prefetch returns zeros and moves no bytes.
  const int nrec = u1 - u0;
  const int ft = u0 / nq;
  const int nt = nrec > 0 ? (u1 - 1) / nq + 1 - ft : 0;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(Wt + static_cast<uint64_t>(t0 + ft) * Q * kRecordBytes),
      0, nt * Q * kRecordBytes, kBufferWord3);
  struct Stage {
    u32x4 c0, c1, sb;
  };
  int lq = u0 % nq, ltl = 0, nload = 0;  // next load: record qa + lq of tile ft + ltl
  auto load = [&](Stage &st) {
    const uint32_t o = nload < nrec
                           ? static_cast<uint32_t>((ltl * Q + qa + lq) * kRecordBytes)
                           : 0x7FFFFFF0u;
    st.c0 = buffer_load16<kNonTemporal>(wr, lane * 16, o);
    st.c1 = buffer_load16<kNonTemporal>(wr, 1024 + lane * 16, o);
    st.sb = buffer_load16<kNonTemporal>(wr, 2048 + j * 16, o);
    ++nload;
    if (++lq == nq) {
      lq = 0;
      ++ltl;
    }
  };
  Stage st[S];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) load(st[i]);
  // Every outstanding vector memory operation, this wave's activation copies
  // included, must be complete before the barrier: direct-to-LDS loads need
  // not complete in order with the weight loads issued after them (a weight
  // load past the wave's range returns at once), so no partial count would
  // prove the copies done.  The first weight stage is needed next anyway.
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  const u32x4 neg = {kNeg128Pair, kNeg128Pair, kNeg128Pair, kNeg128Pair};
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  const UnpackConsts uc = unpack_consts();
  // Row tile rt (rows 16 rt ..) of lane (j, kb), half h: slot
  // 8(j%8) + 2kb + h of block (4q + gi) 2RT + 2rt + j/8.  The codes are
  // unpacked once and multiplied with every row tile.
  auto compute = [&](const Stage &s, int q, f32x4 (&acc)[RT]) {
    const u32x4 *xf = lds + q * (512 * RT) + (j >> 3) * 64 + (j & 7) * 8 + 2 * kb;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const u32x4 cw = gi < 2 ? s.c0 : s.c1;
      const u32x4 b0 = unpack_codes((gi & 1) ? cw.z : cw.x, uc);
      const u32x4 b1 = unpack_codes((gi & 1) ? cw.w : cw.y, uc);
      const uint32_t sbw = s.sb[gi];
      const float sc = __uint_as_float(sbw << 16);
      const float bn = __uint_as_float(sbw & 0xFFFF0000u) * kMinusInv128;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const u32x4 a0 = xf[(gi * 2 * RT + 2 * rt) * 64];
        const u32x4 a1 = xf[(gi * 2 * RT + 2 * rt) * 64 + 1];
        f32x4 xn = mfma16x16x32(a0, neg, fzero);
        xn = mfma16x16x32(a1, neg, xn);
        f32x4 tq = mfma16x16x32(a0, b0, xn);
        tq = mfma16x16x32(a1, b1, tq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[rt][r] = __builtin_fmaf(bn, xn[r], acc[rt][r]);
          acc[rt][r] = __builtin_fmaf(sc, tq[r], acc[rt][r]);
        }
      }
    }
  };
  float *dst = p == 0 ? y : ws + static_cast<uint64_t>(p - 1) * M * N;
  auto store = [&](int tile, const f32x4 (&v)[RT]) {
    const int n = tile * 16 + j;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * rt + kb * 4 + r;
        if (m < M) dst[static_cast<uint64_t>(m) * N + n] = v[rt][r];
      }
  };

  // head: partial sum of a first tile entered past its first record;
  // tail: partial sum of a last tile left before its last record
  f32x4 acc[RT], head_sum[RT], tail_sum[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = head_sum[rt] = tail_sum[rt] = fzero;
  int q = u0 % nq;
  int tl = u0 / nq;
  bool in_head = q != 0;
  for (int i0 = 0; i0 < nrec; i0 += S) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      load(st[(i + S - 1) % S]);
      __builtin_amdgcn_sched_barrier(0);
      if (i0 + i < nrec) {
        compute(st[i], q, acc);
        if (++q == nq) {
          if (in_head) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) head_sum[rt] = acc[rt];
            in_head = false;
          } else {
            store(t0 + tl, acc);
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt] = fzero;
          q = 0;
          ++tl;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (q != 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (in_head)
        head_sum[rt] = acc[rt];
      else
        tail_sum[rt] = acc[rt];
    }
  }

  // split tiles: the activations are no longer needed, so their LDS holds
  // each wave's two partial sums (slot (2 wave + half) RT + rt)
  __syncthreads();
  f32x4 *part = reinterpret_cast<f32x4 *>(lds);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    part[((wave * 2 + 0) * RT + rt) * 64 + lane] = head_sum[rt];
    part[((wave * 2 + 1) * RT + rt) * 64 + lane] = tail_sum[rt];
  }
  __syncthreads();
  if (nrec > 0) {
    const int lt = (u1 - 1) / nq;
    if (lt * nq >= u0 && lt * nq + nq > u1) {
      // this wave holds lt's first record but not its last: its share is
      // its tail sum, the following waves' shares their head sums
      f32x4 v[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        v[rt] = part[((wave * 2 + 1) * RT + rt) * 64 + lane];
      for (int w2 = wave + 1; w2 < W; ++w2) {
        const int a0 = static_cast<int>(static_cast<int64_t>(U) * w2 / W);
        const int a1 = static_cast<int>(static_cast<int64_t>(U) * (w2 + 1) / W);
        if (a0 >= lt * nq + nq) break;
        if (a1 > a0)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            v[rt] += part[((w2 * 2) * RT + rt) * 64 + lane];
      }
      store(t0 + lt, v);
    }
  }
}

// y += sum over parts p = 1 .. P-1 of workspace slice p - 1, in part order
// (four outputs per thread; M * N is a multiple of 16).
__global__ __launch_bounds__(256) void reduce_parts_kernel(
    float *__restrict__ y, const float *__restrict__ ws, uint32_t mn4, int P) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= mn4) return;
  f32x4 v = reinterpret_cast<f32x4 *>(y)[i];
  for (int p = 1; p < P; ++p)
    v += reinterpret_cast<const f32x4 *>(ws)[static_cast<uint64_t>(p - 1) * mn4 + i];
  reinterpret_cast<f32x4 *>(y)[i] = v;
}

// Code word q0..q7 (nibble i = input i) -> nibbles q0 q2 q4 q6 q1 q3 q5 q7,
// so that unpack_codes yields the pairs (q0,q1) (q2,q3) (q4,q5) (q6,q7):
// consecutive inputs, the order of the activations in memory.
__device__ __forceinline__ uint32_t split_even_odd(uint32_t w) {
  uint32_t e = w & 0x0F0F0F0Fu;
  uint32_t o = (w >> 4) & 0x0F0F0F0Fu;
  e = (e | (e >> 4)) & 0x00FF00FFu;
  o = (o | (o >> 4)) & 0x00FF00FFu;
  e = (e | (e >> 8)) & 0x0000FFFFu;
  o = (o | (o >> 8)) & 0x0000FFFFu;
  return e | (o << 16);
}

// Planar -> tiled, one thread per 16-byte unit of the output.
__global__ __launch_bounds__(256) void repack_kernel(
    const uint8_t *__restrict__ W, u32x4 *__restrict__ out, int N, int K) {
  constexpr int kUnits = kRecordBytes / 16;
  const int G = K >> 6;
  const int Q = K >> 8;
  const uint64_t NK = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  const uint64_t units = NK * 9 / 16 / 16;
  const uint16_t *scales = reinterpret_cast<const uint16_t *>(W + NK / 2);
  const uint16_t *biases = reinterpret_cast<const uint16_t *>(W + NK / 2 + NK / 32);
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t u = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       u < units; u += stride) {
    const uint64_t record = u / kUnits;
    const int within = static_cast<int>(u % kUnits);
    const uint64_t tile = record / Q;
    const int q = static_cast<int>(record % Q);
    u32x4 v;
    if (within < 128) {
      const int pair = within >> 6;
      const int l = within & 63;
      const uint64_t n = tile * 16 + (l & 15);
      const int kb = l >> 4;
      const int g0 = 4 * q + 2 * pair;
      const uint8_t *row = W + n * static_cast<uint64_t>(K >> 1);
      const u32x2 a = *reinterpret_cast<const u32x2 *>(row + g0 * 32 + kb * 8);
      const u32x2 b = *reinterpret_cast<const u32x2 *>(row + (g0 + 1) * 32 + kb * 8);
      v = u32x4{split_even_odd(a.x), split_even_odd(a.y), split_even_odd(b.x),
                split_even_odd(b.y)};
    } else {
      const uint64_t n = tile * 16 + (within - 128);
      const uint64_t gi = n * G + 4 * q;
      const u32x2 sv = *reinterpret_cast<const u32x2 *>(scales + gi);
      const u32x2 bv = *reinterpret_cast<const u32x2 *>(biases + gi);
      v.x = (sv.x & 0xFFFFu) | (bv.x << 16);
      v.y = (sv.x >> 16) | (bv.x & 0xFFFF0000u);
      v.z = (sv.y & 0xFFFFu) | (bv.y << 16);
      v.w = (sv.y >> 16) | (bv.y & 0xFFFF0000u);
    }
    out[u] = v;
  }
}

// W_out[n][k] = s * q + b, one thread per 32-bit code word (8 inputs).
__global__ __launch_bounds__(256) void dequant_kernel(
    const uint8_t *__restrict__ W, float *__restrict__ out, int N, int K) {
  const int G = K >> 6;
  const uint64_t NK = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  const uint64_t words = NK / 8;
  const uint64_t words_per_row = static_cast<uint64_t>(K) / 8;
  const uint32_t *codes = reinterpret_cast<const uint32_t *>(W);
  const uint16_t *scales = reinterpret_cast<const uint16_t *>(W + NK / 2);
  const uint16_t *biases = reinterpret_cast<const uint16_t *>(W + NK / 2 + NK / 32);
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < words; i += stride) {
    const uint64_t n = i / words_per_row;
    const uint64_t k0 = (i % words_per_row) * 8;
    const uint64_t gi = n * G + k0 / 64;
    const float s = bf16_to_f32(scales[gi]);
    const float b = bf16_to_f32(biases[gi]);
    const uint32_t w = codes[i];
    float4 lo, hi;
    lo.x = __builtin_fmaf(s, static_cast<float>(w & 15u), b);
    lo.y = __builtin_fmaf(s, static_cast<float>((w >> 4) & 15u), b);
    lo.z = __builtin_fmaf(s, static_cast<float>((w >> 8) & 15u), b);
    lo.w = __builtin_fmaf(s, static_cast<float>((w >> 12) & 15u), b);
    hi.x = __builtin_fmaf(s, static_cast<float>((w >> 16) & 15u), b);
    hi.y = __builtin_fmaf(s, static_cast<float>((w >> 20) & 15u), b);
    hi.z = __builtin_fmaf(s, static_cast<float>((w >> 24) & 15u), b);
    hi.w = __builtin_fmaf(s, static_cast<float>(w >> 28), b);
    float4 *o = reinterpret_cast<float4 *>(out + n * K + k0);
    o[0] = lo;
    o[1] = hi;
  }
}

// Read-only stream: 4 independent 16-byte loads per thread per step.
// Streaming read probe: workgroup b reads the contiguous share
// [b chunk16, (b+1) chunk16) of the buffer (16-byte units); its waves take
// the share's 1 KiB blocks in turn, U non-temporal loads in flight per wave
// (one workgroup of 512 threads per CU; U = 8 read 715 MB at 6.7 TB/s on
// MI355X and U = 4 100 MB at 5.8 TB/s, against 5.8 and 5.1 TB/s for a
// grid-stride loop of plain loads).
template <int kStreamUnroll>
__global__ __launch_bounds__(512) void stream_read_kernel(
    const u32x4 *__restrict__ buf, uint64_t n16, uint64_t chunk16,
    uint32_t *__restrict__ sink) {
  const uint64_t beg = static_cast<uint64_t>(blockIdx.x) * chunk16;
  const uint64_t end = beg + chunk16 < n16 ? beg + chunk16 : n16;
  const uint64_t step = blockDim.x;
  uint64_t i = beg + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * step < end; i += kStreamUnroll * step) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      v[u] = __builtin_nontemporal_load(&buf[i + u * step]);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += step) {
    const u32x4 a = __builtin_nontemporal_load(&buf[i]);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

__global__ __launch_bounds__(256) void stream_copy_kernel(
    const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, uint64_t n16) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride],
                d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

template <int TNT, int NTW, int KSW>
int launch_tiled(const q4_plan &p, const void *x, const void *W, float *y,
                 int M, int N, int K, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_tiled_kernel<TNT, NTW, KSW>), dim3(p.grid),
                     dim3(p.block), 0, stream, static_cast<const uint16_t *>(x),
                     static_cast<const uint8_t *>(W), y, M, N, K);
  return launch_status();
}

// s_barrier after this wave's LDS accesses have completed; unlike
// __syncthreads it does not wait for outstanding global loads.
__device__ __forceinline__ void kslice_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The product for M <= 16 with each wave's slice of K of the activations in
// registers (K <= 6144, or parts of K of at most 24 records).  One workgroup per CU owns whole tiles
// [t0, t1); its W = ceil(Q / 2) waves all work on the same tile at once,
// wave w on records 2w and 2w + 1 of it, so that the workgroup reads each
// tile's 46 KB (at K = 5120) as one contiguous run:
//  * the wave loads its two records' activations once into MFMA operand
//    registers (lane (j, kb), half h: inputs 64 gi + 16 kb + 8 h .. +7 of
//    row j of record q; rows >= M, and a second record past K, are zeros),
//    and forms the seed -128 * sum(x) of each of its 8 groups once, with
//    two MFMAs per group -- not per tile;
//  * per tile it multiplies its two records (two MFMAs per group, seeded
//    with that group's sum) and writes its partial 16 x 16 sum to LDS;
//  * every kslice_batch(W) tiles the workgroup adds the waves' partial sums
//    in wave order and writes y.
// The activation loads are issued first, without branches, and the first
// tile's weights after them.  They are row-contiguous (each load brings
// 512 B runs of two rows; only the row pairs below M at M <= 4) and pass
// through LDS into the operand layout, most often written by the loads
// themselves: loads straight in the operand layout touch 16 rows 2K bytes
// apart each, which the L2 serves far more slowly (the first tile at M = 16
// came 2 us later), and at small M they issue 16 instructions for a few
// active lanes each.  Only parts of K taken in turn at M <= 4 keep the
// operand-layout loads.  The weights of tile t + 1 are in flight while tile
// t is multiplied.
//
// With a workspace, K beyond 24 records is cut into P parts: the grid is P
// groups of Gt workgroups, the group of part p takes records
// [Q p / P, Q (p+1) / P) of every tile, part 0 writes y and part p > 0 its
// M x N slice p - 1 of the workspace, which reduce_parts_kernel then adds to
// y in part order.
//
// Workgroups are dealt to the 8 XCDs in turn (b, b + 8, ... on XCD b % 8), so
// tiles (and parts) are assigned by rank XCD after XCD: every XCD streams the
// same share (+-1 tile per workgroup), and with parts an XCD reads one or
// two parts' activations.  A CU serves the loads of its older waves first,
// so without a barrier the youngest waves of a long run fall microseconds
// behind and finish alone, with few loads in flight; with 8 or more tiles
// per workgroup the waves therefore meet at a barrier once per tile, after
// issuing the next tile's loads.  (With fewer tiles the barrier costs more
// than the lag: the first tile's wait then dominates.)  Summation order
// depends only on (N, K), so results do not depend on M and repeated calls
// are bitwise equal.
//
// With kSample (the LM head of a verify step) the logits are not stored:
// each batch's sums go to an LDS array of the workgroup's logits, and after
// the last batch each wave takes rows m = wave, wave + W, ... and writes the
// row's best 32 candidate keys among the workgroup's columns to
// cand[(m * G + g) * 32 ..] (g the workgroup's tile group, G the grid),
// which launch_sample_rows then merges.  Selection per row: the 32nd best
// of the 64 lane maxima's upper halves bounds the row's 32nd best key from
// below, so only keys at or above it survive; the survivors (usually a few
// more than 32) are packed into the wave's part of the partial-sum area and
// sorted 64 at a time with bitonic networks, merging into the running list.
template <int W, int kRowLoads, bool kSample, bool kPlanar, bool kSeq, int RT,
          bool kDot = false>
__global__ __launch_bounds__(64 * W) void gemm_kslice_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ Wt,
    float *__restrict__ y, float *__restrict__ ws, int N, int K, uint32_t mp,
    int per, uint32_t gr) {
  // Packed by the host (kslice_args): mp = M | P << 8 | Pin << 20 (rows,
  // part groups, parts per group), gr = Gt | rem << 16 with Gt workgroups
  // per part group and T = per * Gt + rem tiles.  Every argument arrives in
  // SGPRs at wave launch (kernarg preload), and no integer division stands
  // between the launch and the first loads.
  const int M = static_cast<int>(mp & 0xFFu);
  const int P = static_cast<int>((mp >> 8) & 0xFFFu);
  const int Pin_ = static_cast<int>(mp >> 20);
  // RT = 2 (M = 17..32): two MFMA row tiles multiply the same unpacked codes,
  // and a wave owns one record (R = 1) so that its activation operands stay
  // at the registers of two records of one row tile
  static_assert(RT == 1 || (RT == 2 && !kSample && !kPlanar), "row tiles");
  // kDot: the VALU variant for M <= 4 (v_dot2_f32_bf16 instead of MFMA)
  static_assert(!kDot || (RT == 1 && !kSample && !kPlanar && !kSeq && !kRowLoads),
                "dot variant");
  // kRowLoads: activation row pairs loaded per record (1, 2 or 8), or 0
  // for direct operand-layout loads (parts in turn at M <= 4)
  static_assert(kDot || kRowLoads == 1 || kRowLoads == 2 || kRowLoads == 8 ||
                    (kRowLoads == 0 && kSeq),
                "row pairs");
  constexpr int R = RT == 1 ? 2 : 1;  // records per wave
  // parts of K taken in turn: a run-time count only in the kSeq kernels
  const int Pin = kSeq ? Pin_ : 1;
  // tiles per reduction batch
  constexpr int NB = kSample   ? kslice_sample_batch(W)
                     : kPlanar ? kslice_planar_batch(W, kSeq)
                     : RT == 2 ? kslice_batch2(W, kSeq)
                     : kDot    ? kslice_batch(W) - 4
                               : kslice_batch(W);
  static_assert(NB * RT >= 8, "the activation staging areas (8 KB per wave) fit in part");
  // kDmaX: the activation rows go from memory straight to LDS, both of a
  // wave's units at once (kXU KB each: 1 KB per row pair), when the
  // partial-sum area holds them or can grow to (tiled, at most 10 waves)
  constexpr int kXU = kRowLoads > 0 ? kRowLoads : 1;
  constexpr bool kDmaX = !kSample && !kSeq && !kDot && RT == 1 && kRowLoads > 0 &&
                         (2 * kXU <= NB || (!kPlanar && W <= 10));
  constexpr int kPartTiles = kDmaX && NB < 2 * kXU ? 2 * kXU : NB;  // 1 KB per wave and tile
  __shared__ f32x4 part[kPartTiles * W * RT * 64];
  // planar: each wave's two records of codes of the next tile (16 rows x
  // 128 B each), and the workgroup's scales and biases of the current and
  // the next tile, written by the loads themselves
  __shared__ u32x4 ccode[kPlanar ? W * (kPlanarCodeLds / 16) : 1];
  __shared__ u32x4 csb[kPlanar ? 2 * kPlanarSbLds / 16 : 1];
  // kDot: rows 0..3 of the activations of the wave's two records (1 KiB a
  // row), read back as broadcast operands
  __shared__ u32x4 xdot[kDot ? W * 4 * 64 : 1];
  __shared__ float lg[kSample ? Q4_MAX_ROWS * kSampleLgStride : 1];
  // running sums of the workgroup's tiles over parts of K taken in turn
  __shared__ f32x4 tacc[kSeq ? (kPlanar ? kInMaxTilesPlanar : kInMaxTiles) * RT * 64 : 1];

  const int Q = K >> 8;
  const int G8 = K >> 6;  // groups per row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;
  const int kb = lane >> 4;
  // the grid: P part groups of Gt workgroups (from the arguments rather than
  // the dispatch packet, which would cost a load)
  const int G = static_cast<int>(gr & 0xFFFFu) * P;
  const int b = static_cast<int>(blockIdx.x);
  const int rank = (b & 7) * (G >> 3) + min(b & 7, G & 7) + (b >> 3);
  // rank -> part group pk of K and tile group g; part group pk holds parts
  // pk * Pin .. pk * Pin + Pin - 1, taken one after another
  // t0 = floor(T g / Gt) = per g + floor(rem g / Gt) for T = ceil(N / 16)
  // tiles (per and rem come from the host), likewise t1
  const int Gt = static_cast<int>(gr & 0xFFFFu);
  const int rem = static_cast<int>(gr >> 16);
  const int pk = P == 1 ? 0 : small_div(rank, Gt);
  const int g = rank - pk * Gt;
  const int t0 = g * per + small_div(g * rem, Gt);
  const int t1 = (g + 1) * per + small_div((g + 1) * rem, Gt);
  __builtin_assume(t1 > t0);  // a part has at most one workgroup per tile
  // (planar: the waves meet once per tile anyway, for the shared scales)
  const bool in_step = !kPlanar && t1 - t0 >= 8;
  const int Ptot = P * Pin;
  float *const out = pk == 0 ? y : ws + static_cast<uint64_t>(pk - 1) * M * N;

  // Weights of the workgroup's tiles (all of K); a record past them or
  // past the wave's slice gets an offset past the resource and reads zeros.
  // Tiled: record (tile, q) at (tile Q + q) * 2304 bytes.  Planar: the
  // codes of the tiles' rows (rows past N fall past the resource), their
  // scales and their biases, three resources.
  const int rows = min(N - 16 * t0, 16 * (t1 - t0));
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(
          kPlanar ? Wt + static_cast<uint64_t>(t0) * 16 * (K >> 1)
                  : Wt + static_cast<uint64_t>(t0) * Q * kRecordBytes),
      0, kPlanar ? rows * (K >> 1) : (t1 - t0) * Q * kRecordBytes, kBufferWord3);
  const uint64_t NK = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  // Planar scales of the workgroup's rows and, NK / 32 bytes on, their
  // biases: one resource whose range ends after the last row's biases (a
  // scale row past N reads finite biases, and is never stored).
  const __amdgpu_buffer_rsrc_t sbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(Wt + NK / 2 + static_cast<uint64_t>(t0) * 16 * G8 * 2),
      0, kPlanar ? static_cast<int>(NK / 32) + rows * G8 * 2 : 0, kBufferWord3);
  // Per stage, two records of one tile: for each, the codes of groups 0-1
  // (c0) and 2-3 (c1), 16 bytes per lane, and the (scale, bias) words;
  // tiled: sb[qq] word gi = scale | bias << 16 of group gi; planar: sc and
  // bi hold the 8 groups' scales and biases (bf16 pairs) of both records.
  struct Stage {
    u32x4 c0[R], c1[R], sb[2];
  };
  int q0 = 0, nq = 0;  // the wave's records in the current part
  int tl = 0;          // next tile to load, counted from t0
  // Planar scales and biases of the part (set per part): this wave's loads
  // (at most two: ins = wave, wave + W of 2 nk) -- lane offsets at tile 0
  // and LDS offsets -- and where the wave reads its own chunk.
  constexpr uint32_t kNoChunk = 0xFFFFFFFFu;
  int sb_n = 0;                  // loads of this wave
  uint32_t sb_o0 = 0, sb_o1 = 0;  // lane offsets (past the range: nothing)
  int sb_l0 = 0, sb_l1 = 0;      // LDS offsets in a buffer
  int sb_rd = 0, sb_bias = 0;    // the wave's scales, and biases after them
  // Planar codes go straight from memory to the wave's LDS area: load i of
  // record qq brings rows 8i .. 8i+7 of the tile, 128 B (the record's 256
  // codes) each, lane l chunk (l & 7) ^ (l >> 3) of row 8i + (l >> 3), so
  // every load covers whole 128-byte runs.  Lane l lands at l * 16, which
  // puts chunk c of row r at r * 128 + (c ^ (r & 7)) * 16.
  char *const cwave = reinterpret_cast<char *>(ccode) + wave * kPlanarCodeLds;
  // the lane's part of those offsets: row l >> 3 of the eight, its chunk
  const uint32_t cl_lane =
      static_cast<uint32_t>((lane >> 3) * (K >> 1) + (((lane & 7) ^ (lane >> 3)) << 4));
  // where lane (j, kb) reads group 0 of record 0 (group g: ^ (g << 5))
  const uint32_t cr_lane = static_cast<uint32_t>(
      j * 128 + (((kb >> 1) ^ (j & 7)) << 4) + ((kb & 1) << 3));
  auto load = [&](Stage &st) {
#pragma unroll
    for (int qq = 0; qq < R; ++qq) {
      const bool ok = tl < t1 - t0 && qq < nq;
      if constexpr (kPlanar) {
        // none past the last tile: the area then belongs to the next part
        if (tl < t1 - t0) {
          const uint32_t lo = opaque_v(cl_lane);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t o =
                ok ? lo + static_cast<uint32_t>((tl * 16 + 8 * i) * (K >> 1) + (q0 + qq) * 128)
                   : 0x7FFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (__attribute__((address_space(3))) void *)(cwave + qq * 2048 + i * 1024),
                16, o, 0, 0, kNonTemporal);
          }
        }
      } else {
        const uint32_t o = ok ? static_cast<uint32_t>((tl * Q + q0 + qq) * kRecordBytes)
                              : 0x7FFFFFF0u;
        st.c0[qq] = buffer_load16<kNonTemporal>(wr, lane * 16, o);
        st.c1[qq] = buffer_load16<kNonTemporal>(wr, 1024 + lane * 16, o);
        st.sb[qq] = buffer_load16<kNonTemporal>(wr, 2048 + j * 16, o);
      }
    }
    if constexpr (kPlanar) {
      // The tile's scales (array 0) and biases (array 1) of the part's
      // groups: per array 16 rows of cpr 16-byte chunks (chunk c = groups
      // 8c .. 8c+7 from the part's first, the records of wave c), each row's
      // chunks one contiguous run.  Load k of array a brings chunks
      // 64k .. 64k+63 of it to LDS buffer tl & 1, shared by the workgroup;
      // the loads are dealt to the waves in turn.
      // (lanes past the array's chunks stay idle: a load would write zeros
      // over the other array's chunks)
      if (tl < t1 - t0 && sb_n > 0) {
        char *const buf = reinterpret_cast<char *>(csb) + (tl & 1) * kPlanarSbLds;
        const uint32_t dt = static_cast<uint32_t>(tl * 32 * G8);  // 16 rows
        const uint32_t o0 = opaque_v(sb_o0);
        if (o0 != kNoChunk)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              sbr, (__attribute__((address_space(3))) void *)(buf + sb_l0), 16,
              o0 + dt, 0, 0, kNonTemporal);
        if (sb_n > 1) {
          const uint32_t o1 = opaque_v(sb_o1);
          if (o1 != kNoChunk)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                sbr, (__attribute__((address_space(3))) void *)(buf + sb_l1), 16,
                o1 + dt, 0, 0, kNonTemporal);
        }
      }
    }
    ++tl;
  };
  // register stages: S - 1 tiles' weights in flight while one is
  // multiplied.  (Two row tiles hold one record a stage; a third stage for
  // them kept twice the bytes in flight but measured the same on MI355X:
  // gate+up at M = 32 29.0 us with either, and spilled once parts of K are
  // taken in turn.)
  constexpr int S = 2;
  Stage st[S];
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x), 0,
      static_cast<int>(static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u),
      kBufferWord3);
  const u32x4 neg = {kNeg128Pair, kNeg128Pair, kNeg128Pair, kNeg128Pair};
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  // Activation operand (gi, h) of lane (j, kb): eight inputs of row j.
  // Tiled: inputs 64 gi + 16 kb + 8 h .. +7 in order (the repack splits each
  // code word into even and odd inputs).  Planar: lane (j, kb) reads words
  // 2 kb and 2 kb + 1 of each group of row j from LDS, so operand h meets
  // inputs 64 gi + 8 (2 kb + h) .. +7, permuted to the pairs (0,4) (1,5)
  // (2,6) (3,7) in which unpack_codes yields a word's codes.  (The inputs of
  // an operand slot depend on kb alone: the MFMA pairs slot kb of every row
  // of x with slot kb of every row of W.)
  const int w_h0 = 2 * kb;
  const int w_h1 = 2 * kb + 1;
  // activation operand units u = 0, 1: records 0 and 1 of the wave's pair
  // (RT = 1), or row tiles 0 and 1 of its one record (RT = 2)
  u32x4 xa[2][4][2];
  f32x4 xn[2][4];
  const UnpackConsts uc = unpack_consts();
  auto compute = [&](const Stage &s, f32x4 (&acc)[RT]) {
#pragma unroll
    for (int qq = 0; qq < R; ++qq) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const u32x4 cw = gi < 2 ? s.c0[qq] : s.c1[qq];
        const u32x4 b0 = unpack_codes((gi & 1) ? cw.z : cw.x, uc);
        const u32x4 b1 = unpack_codes((gi & 1) ? cw.w : cw.y, uc);
        float sc, bn;
        if constexpr (kPlanar) {
          const int e = 4 * qq + gi;  // group of the wave's pair of records
          const uint32_t sw = s.sb[0][e >> 1], bw = s.sb[1][e >> 1];
          sc = __uint_as_float((e & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
          bn = __uint_as_float((e & 1) ? (bw & 0xFFFF0000u) : (bw << 16)) * kMinusInv128;
        } else {
          const uint32_t sbw = s.sb[qq][gi];
          sc = __uint_as_float(sbw << 16);
          bn = __uint_as_float(sbw & 0xFFFF0000u) * kMinusInv128;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int u = qq + rt;  // the unit of (record qq, row tile rt)
          f32x4 tq = mfma16x16x32(xa[u][gi][0], b0, xn[u][gi]);
          tq = mfma16x16x32(xa[u][gi][1], b1, tq);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[rt][r] = __builtin_fmaf(bn, xn[u][gi][r], acc[rt][r]);
            acc[rt][r] = __builtin_fmaf(sc, tq[r], acc[rt][r]);
          }
        }
      }
    }
  };
  // kDot: lane (j, kb) multiplies row j of the tile with rows m < M of the
  // activations over its slots (inputs 64 gi + 16 kb .. +15 of each group,
  // read from LDS, where all 16 lanes of a kb group read the same bytes)
  // with v_dot2_f32_bf16, 8 per group and row; the codes enter as
  // bf16 128 + q as in the MFMA path, and xs, the slot's sum of x, removes
  // the offset and carries the bias: per group s (dot - 128 xs) + b xs.  The
  // four kb lanes' sums of a row are added with two permlane swaps, and
  // lane (j, 0) returns rows 0..3 in the MFMA result's layout (rows 4..15,
  // in the other lanes, are zero).
  float xs[2][4][4];
  auto compute_dot = [&](const Stage &s, f32x4 &res) {
    float am[4] = {0.f, 0.f, 0.f, 0.f};
    const u32x4 *xw = xdot + wave * 256;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const u32x4 cw = gi < 2 ? s.c0[qq] : s.c1[qq];
        const u32x4 b0 = unpack_codes((gi & 1) ? cw.z : cw.x, uc);
        const u32x4 b1 = unpack_codes((gi & 1) ? cw.w : cw.y, uc);
        const uint32_t sbw = s.sb[qq][gi];
        const float sc = __uint_as_float(sbw << 16);
        const float bb = __uint_as_float(sbw & 0xFFFF0000u);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (m < M) {  // uniform
            const u32x4 v0 = xw[m * 64 + qq * 32 + 8 * gi + 2 * kb];
            const u32x4 v1 = xw[m * 64 + qq * 32 + 8 * gi + 2 * kb + 1];
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(b0[e]), as_bf16x2(v0[e]), d,
                                                  false);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(b1[e]), as_bf16x2(v1[e]), d,
                                                  false);
            const float x1 = xs[qq][gi][m];
            am[m] = __builtin_fmaf(sc, __builtin_fmaf(-128.0f, x1, d), am[m]);
            am[m] = __builtin_fmaf(bb, x1, am[m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t v = __float_as_uint(am[m]);
      const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      const float s16 = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
      const uint32_t w = __float_as_uint(s16);
      const auto p32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
      am[m] = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    }
    const f32x4 mine = {am[0], am[1], am[2], am[3]};
    res = kb == 0 ? mine : fzero;
  };
  // Planar: once the tile's codes have landed in the wave's LDS area, each
  // lane takes words 2 kb, 2 kb + 1 of groups 0-1 (c0: .x .y, .z .w) and
  // 2-3 (c1) of both records of row j.  The area is free again once the
  // reads have returned.
  auto fetch = [&](Stage &s, int tt) {
    if constexpr (kPlanar) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loads have landed
      __builtin_amdgcn_s_barrier();        // ... those of every wave
      asm volatile("" ::: "memory");
      // scales and biases of the wave's records (chunk `wave` of row j); a
      // wave without records takes zeros (the LDS may hold any bits there)
      {
        const char *buf = reinterpret_cast<const char *>(csb) + (tt & 1) * kPlanarSbLds;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const uint32_t rd = opaque_v(sb_rd);
        s.sb[0] = nq > 0 ? *reinterpret_cast<const u32x4 *>(buf + rd) : zero;
        s.sb[1] = nq > 0 ? *reinterpret_cast<const u32x4 *>(buf + rd + sb_bias) : zero;
      }
      const uint32_t cr = opaque_v(cr_lane);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint2 v = *reinterpret_cast<const uint2 *>(cwave + qq * 2048 + (cr ^ (g << 5)));
          u32x4 &d = g < 2 ? s.c0[qq] : s.c1[qq];
          if (g & 1) {
            d.z = v.x;
            d.w = v.y;
          } else {
            d.x = v.x;
            d.y = v.y;
          }
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the area is free
      asm volatile("" ::: "memory");
    }
  };

  for (int ip = 0; ip < Pin; ++ip) {
    const int pp = pk * Pin + ip;  // part of K
    // records [floor(Q pp / Ptot), floor(Q (pp + 1) / Ptot)), with
    // Q = qd Ptot + qr
    const int qd = Ptot == 1 ? Q : small_div(Q, Ptot);
    const int qr = Q - qd * Ptot;
    const int qa = qd * pp + (Ptot == 1 ? 0 : small_div(qr * pp, Ptot));
    const int nrec = qd * (pp + 1) + (Ptot == 1 ? 0 : small_div(qr * (pp + 1), Ptot)) - qa;
    q0 = qa + R * wave;
    nq = min(max(nrec - R * wave, 0), R);  // 0 .. R
    tl = 0;
    if constexpr (kPlanar) {
      // Per tile and array (scales 0, biases 1): 16 rows of cpr 16-byte
      // chunks (chunk c = groups 8c .. 8c+7 from the part's first, the
      // records of wave c), each row's chunks one contiguous run.  Load k
      // of array a brings chunks 64k .. 64k+63 of it, lane l chunk
      // f = 64k + l (row f / cpr), to LDS a 256 cpr + f 16 of the buffer of
      // the tile's parity, shared by the workgroup.  The 2 nk loads are
      // dealt to the waves in turn, at most two each (W >= cpr).
      const int cpr = (nrec + 1) >> 1;
      const int nk = (16 * cpr + 63) >> 6;
      sb_n = (wave < 2 * nk) + (wave + W < 2 * nk);
      uint32_t o[2];
      int l[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ins = wave + u * W;
        const int a = ins >= nk;
        const int k = ins - a * nk;
        const int f = 64 * k + lane;
        const int r = f / cpr;
        o[u] = f < 16 * cpr ? static_cast<uint32_t>(a * static_cast<int>(NK / 32) +
                                                    (r * G8 + 4 * qa) * 2 + 16 * (f - r * cpr))
                            : kNoChunk;
        l[u] = a * 256 * cpr + k * 1024;
      }
      sb_o0 = o[0];
      sb_o1 = o[1];
      sb_l0 = l[0];
      sb_l1 = l[1];
      sb_rd = (j * cpr + wave) * 16;
      sb_bias = 256 * cpr;
    }
    if constexpr (kDot) {
      // rows m < M of the wave's two records (inputs 256 q0 .. +511), 16
      // bytes a lane, into the wave's LDS area (a record past the part
      // reads zeros); then each lane's slot sums xs
      const u32x4 zero4 = {0u, 0u, 0u, 0u};
      u32x4 xv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        xv[m] = m < M ? buffer_load16<0>(xr, static_cast<uint32_t>((m * K + 256 * q0 + 8 * lane) * 2),
                                         (lane >> 5) < nq ? 0u : 0x7FFFFFF0u)
                      : zero4;
      load(st[0]);
#pragma unroll
      for (int m = 0; m < 4; ++m) xdot[wave * 256 + m * 64 + lane] = xv[m];
      const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float t = 0.f;
            if (m < M) {
              const u32x4 v0 = xdot[wave * 256 + m * 64 + qq * 32 + 8 * gi + 2 * kb];
              const u32x4 v1 = xdot[wave * 256 + m * 64 + qq * 32 + 8 * gi + 2 * kb + 1];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v0[e]), ones, t, false);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v1[e]), ones, t, false);
            }
            xs[qq][gi][m] = t;
          }
    } else if constexpr (kRowLoads > 0) {
      // Row-contiguous loads (load i < kRowLoads of record qq brings rows 2i
      // and 2i + 1, 512 B each), then through LDS into the operand layout;
      // rows from 2 kRowLoads on (all >= M) are zeros without a load.  Lane l of
      // load i holds chunk c = l & 31 (inputs 8c .. 8c+7) of row
      // r = 2i + (l >> 5); it is stored at row r, chunk c ^ (r & 7) of the
      // wave's 8 KB area, and lane (j, kb) reads chunk 8 gi + w of row j for
      // operand (gi, h): the XOR keeps both sides free of bank conflicts.
      // (unit u: record qu of the wave's records, rows 16 ru .. 16 ru + 15)
      // With kDmaX both units go straight from memory to LDS (load i of
      // unit u to u kXU KB + i KB, lane l at l * 16, so lane l loads the
      // chunk that belongs at its place: (l & 31) ^ (r & 7)), and only then
      // are the first tile's weights requested.
      char *area = reinterpret_cast<char *>(part) + wave * (kDmaX ? 2 * kXU * 1024 : 8192);
      u32x4 xrow[2][8];
      if constexpr (kDmaX) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int qu = RT == 1 ? u : 0, ru = RT == 1 ? 0 : u;
#pragma unroll
          for (int i = 0; i < kRowLoads; ++i) {
            const uint32_t rl = 2 * i + (lane >> 5);
            const uint32_t off = ((16 * ru + rl) * K + 256 * (q0 + qu) +
                                  8 * ((lane & 31) ^ (rl & 7))) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void *)(area + (u * kXU + i) * 1024), 16,
                off, qu < nq ? 0u : 0x7FFFFFF0u, 0, 0);
          }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the rows are in LDS
        asm volatile("" ::: "memory");
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int qu = RT == 1 ? u : 0, ru = RT == 1 ? 0 : u;
#pragma unroll
          for (int i = 0; i < kRowLoads; ++i) {
            const uint32_t r = 16 * ru + 2 * i + (lane >> 5);
            const uint32_t off = (r * K + 256 * (q0 + qu) + 8 * (lane & 31)) * 2;
            xrow[u][i] = buffer_load16<0>(xr, off, qu < nq ? 0u : 0x7FFFFFF0u);
          }
        }
      }
      load(st[0]);
      if constexpr (S > 2) load(st[1]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        char *uarea = area + (kDmaX ? u * kXU * 1024 : 0);
        if constexpr (!kDmaX) {
#pragma unroll
          for (int i = 0; i < kRowLoads; ++i) {
            const int r = 2 * i + (lane >> 5);
            const int c = (lane & 31) ^ (r & 7);
            *reinterpret_cast<u32x4 *>(area + r * 512 + c * 16) = xrow[u][i];
          }
        }
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int c = (8 * gi + (h ? w_h1 : w_h0)) ^ (j & 7);
            // rows past the loaded pairs are zeros (not in the area)
            const u32x4 v = j < 2 * kRowLoads
                                 ? *reinterpret_cast<const u32x4 *>(uarea + j * 512 + c * 16)
                                 : u32x4{0u, 0u, 0u, 0u};
            xa[u][gi][h] = kPlanar ? pair_activations(v) : v;
          }
      }
      // the areas alias the partial sums: every wave has its operands in
      // registers before any wave writes a partial sum
      kslice_lds_barrier();
    } else {
      // kRowLoads == 0 (parts of K in turn at M <= 4): loads straight in the
      // operand layout, no LDS round trip and no barrier per part -- lane
      // (j, kb), operand (gi, h) reads inputs 64 gi + 8 w .. +7 of row j
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qu = RT == 1 ? u : 0, ru = RT == 1 ? 0 : u;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t off = (static_cast<uint32_t>(16 * ru + j) * K + 256 * (q0 + qu) +
                                  64 * gi + 8 * (h ? w_h1 : w_h0)) * 2;
            xa[u][gi][h] = buffer_load16<0>(xr, off, qu < nq ? 0u : 0x7FFFFFF0u);
          }
      }
      load(st[0]);
      __builtin_amdgcn_sched_barrier(0);  // every load issued before the seeds
      if constexpr (kPlanar) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int gi = 0; gi < 4; ++gi)
#pragma unroll
            for (int h = 0; h < 2; ++h) xa[qq][gi][h] = pair_activations(xa[qq][gi][h]);
      }
    }
    if constexpr (!kDot) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const f32x4 s0 = mfma16x16x32(xa[qq][gi][0], neg, fzero);
          xn[qq][gi] = mfma16x16x32(xa[qq][gi][1], neg, s0);
        }
    }

    int tb = t0;  // first tile of the current batch
    for (int t = t0; t < t1; t += S) {
#pragma unroll
      for (int i = 0; i < S; ++i) {
        if (t + i < t1) fetch(st[i], t + i - t0);
        __builtin_amdgcn_sched_barrier(0);
        load(st[(i + S - 1) % S]);
        __builtin_amdgcn_sched_barrier(0);
        if (in_step) __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (t + i < t1) {  // the same for every wave: barriers below are safe
          f32x4 acc[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt] = fzero;
          if constexpr (kDot)
            compute_dot(st[i], acc[0]);
          else
            compute(st[i], acc);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            part[(((t + i - tb) * W + wave) * RT + rt) * 64 + lane] = acc[rt];
          if (t + i - tb == NB - 1 || t + i == t1 - 1) {
            __syncthreads();
            const int nb = t + i - tb + 1;
            // entry e: tile tt, row tile rt, lane l of the partial sums
            for (int e = threadIdx.x; e < nb * RT * 64; e += 64 * W) {
              const int tt = e / (RT * 64), rt = (e >> 6) - tt * RT, l = e & 63;
              f32x4 v = part[((tt * W) * RT + rt) * 64 + l];
              for (int w2 = 1; w2 < W; ++w2) v += part[(((tt * W + w2) * RT) + rt) * 64 + l];
              if constexpr (kSeq) {
                // parts of K in turn: parts before the last keep running
                // sums, in part order (at most kInMaxTiles tiles then)
                {
                  f32x4 *a = &tacc[((tb + tt - t0) * RT + rt) * 64 + l];
                  if (ip > 0) v = *a + v;
                  if (ip + 1 < Pin) {
                    *a = v;
                    continue;
                  }
                }
              }
              const int n = (tb + tt) * 16 + (l & 15);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int m = 16 * rt + (l >> 4) * 4 + r;
                if constexpr (kSample) {
                  if (m < M) lg[m * kSampleLgStride + (n - t0 * 16)] = v[r];
                } else {
                  // non-temporal: on the LM head at M = 16 (15.9 MB of y)
                  // plain stores cost 124 us per call against 119
                  if (m < M && n < N)
                    __builtin_nontemporal_store(v[r], &out[static_cast<uint64_t>(m) * N + n]);
                }
              }
            }
            __syncthreads();
            tb = t + i + 1;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (kSample) {
    // The last batch ended with a barrier: the logits are complete and the
    // partial-sum area is free.  A wave takes rows m and m + W together
    // (two independent chains), m = wave, wave + 2W, ...  Per row: its keys
    // in registers (16 per lane); the bound T = the 32nd largest lane
    // maximum (32 distinct keys reach it, so the row's 32nd best does);
    // the keys >= T packed into the wave's part of the area; their best 32
    // ranked into the candidate list.
    constexpr int kPer = kSampleMaxCols / 64;
    static_assert(NB * 128 >= kSampleMaxCols, "survivor area");
    const int ncols = (t1 - t0) * 16;
    const uint32_t tok0 = static_cast<uint32_t>(t0) * 16u;
    uint64_t *area = reinterpret_cast<uint64_t *>(part) + wave * (NB * 128);
    // appends of up to kSampleMaxCols keys, 64 at a time, stay inside the
    // wave's area (NB * 128 >= kSampleMaxCols slots)
    uint64_t *dummy = nullptr;
    uint64_t *c = reinterpret_cast<uint64_t *>(ws);
    for (int m0 = wave; m0 < M; m0 += 2 * W) {
      const int m1 = m0 + W;
      const bool two = m1 < M;  // wave-uniform
      uint64_t k0[kPer], k1[kPer];
      uint64_t mx0 = 0, mx1 = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int col = 64 * i + lane;
        const bool in = col < ncols;
        k0[i] = in ? make_key(lg[m0 * kSampleLgStride + col], tok0 + col) : 0;
        k1[i] = in && two ? make_key(lg[m1 * kSampleLgStride + col], tok0 + col) : 0;
        mx0 = k0[i] > mx0 ? k0[i] : mx0;
        mx1 = k1[i] > mx1 ? k1[i] : mx1;
      }
      const uint64_t T0 = wave_kth_largest(mx0, kSampleTop);
      const uint64_t T1 = wave_kth_largest(mx1, kSampleTop);
      // the area holds one row's survivors at a time
      uint32_t n = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) wave_append(k0[i], k0[i] != 0 && k0[i] >= T0, area, &n, dummy);
      wave_top32(area, n, c + (static_cast<uint64_t>(m0) * Gt + g) * kSampleTop, lane);
      if (two) {
        n = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) wave_append(k1[i], k1[i] != 0 && k1[i] >= T1, area, &n, dummy);
        wave_top32(area, n, c + (static_cast<uint64_t>(m1) * Gt + g) * kSampleTop, lane);
      }
    }
  }
}

// The K-slice kernel's packed arguments (see gemm_kslice_kernel): the plan
// keeps P, the parts in turn and Gt below 4096, and M <= 32.
struct KsliceArgs {
  uint32_t mp;
  int per;
  uint32_t gr;
};

KsliceArgs kslice_args(const q4_plan &p, int M, int N) {
  const uint32_t parts = p.k_parts, seq = p.k_seq_parts;
  const int gt = static_cast<int>(p.grid / parts);
  const int T = (N + 15) / 16;
  return {static_cast<uint32_t>(M) | parts << 8 | seq << 20, T / gt,
          static_cast<uint32_t>(gt) | static_cast<uint32_t>(T % gt) << 16};
}

template <int W, bool kSample, bool kPlanar, bool kSeq, int RT = 1>
void launch_kslice_v(const q4_plan &p, const void *x, const void *Wt, float *y,
                     float *ws, int M, int N, int K, hipStream_t stream) {
  const KsliceArgs a = kslice_args(p, M, N);
  // Activation rows come as row-contiguous pairs through LDS, only the
  // pairs that hold rows < M at M <= 4 (one load per pair and record): at
  // M = 1 a wave issues 2 activation loads instead of 16 operand-layout
  // loads of 4 active lanes each (o/out 7.37 -> 7.07 us, gate+up 19.35 ->
  // 19.18 us on MI355X).  From M = 5 on all 8 pairs are loaded: 4 pairs at
  // M = 8 measured 0.05-0.4 us slower than 8 (the pairs past M read nothing).
  // Two row tiles take all 16 rows of each.
  auto go = [&](auto lr) {
    hipLaunchKernelGGL((gemm_kslice_kernel<W, decltype(lr)::value, kSample, kPlanar, kSeq, RT>),
                       dim3(p.grid), dim3(64 * W), 0, stream,
                       static_cast<const uint16_t *>(x),
                       static_cast<const uint8_t *>(Wt), y, ws, N, K, a.mp, a.per, a.gr);
  };
  if (RT == 2 || M > 4)
    go(std::integral_constant<int, 8>{});
  else if constexpr (kSeq)
    // parts of K in turn repeat the activation staging per part, with its
    // barrier: there the direct loads measured faster at M <= 4 (down, three
    // parts: 19.3 against 22.0 us at M = 1 with the rows staged in LDS
    // through registers, and against 22.1 us with the loads writing LDS)
    go(std::integral_constant<int, 0>{});
  else if (M > 2)
    go(std::integral_constant<int, 2>{});
  else
    go(std::integral_constant<int, 1>{});
}

template <int W, bool kSample = false, bool kPlanar = false>
void launch_kslice_w(const q4_plan &p, const void *x, const void *Wt, float *y,
                     float *ws, int M, int N, int K, hipStream_t stream) {
  if constexpr (!kSample && !kPlanar) {
    if (p.m_tiles == 2) {
      if (p.k_seq_parts > 1)
        launch_kslice_v<W, false, false, true, 2>(p, x, Wt, y, ws, M, N, K, stream);
      else
        launch_kslice_v<W, false, false, false, 2>(p, x, Wt, y, ws, M, N, K, stream);
      return;
    }
  }
  if constexpr (!kSample) {
    if (p.k_seq_parts > 1) {
      launch_kslice_v<W, kSample, kPlanar, true>(p, x, Wt, y, ws, M, N, K, stream);
      return;
    }
  }
  launch_kslice_v<W, kSample, kPlanar, false>(p, x, Wt, y, ws, M, N, K, stream);
}

// Part sums of a K split: y += workspace slices 1 .. P-1, in part order.
int launch_reduce_parts(float *y, const float *ws, int M, int N, int parts,
                        hipStream_t stream) {
  const uint32_t mn4 = static_cast<uint32_t>(M) * static_cast<uint32_t>(N) / 4;
  hipLaunchKernelGGL(reduce_parts_kernel, dim3((mn4 + 255) / 256), dim3(256), 0,
                     stream, y, ws, mn4, parts);
  return launch_status();
}

// The VALU (v_dot2_f32_bf16) variant of the K-slice kernel, M <= 4, one
// pass of K, tiled layout (the caller has checked all three).
int launch_kslice_dot(const q4_plan &p, const void *x, const void *Wt, float *y,
                      int M, int N, int K, hipStream_t stream) {
  if (p.k_parts != 1 || p.k_seq_parts != 1 || p.m_tiles != 1 || M > 4 ||
      p.layout_id != Q4_LAYOUT_TILED16)
    return Q4_EINVAL;
  const KsliceArgs a = kslice_args(p, M, N);
  switch (p.block / 64) {
#define Q4V_KSLICE_DOT_CASE(W)                                                  \
  case W:                                                                       \
    hipLaunchKernelGGL((gemm_kslice_kernel<W, 0, false, false, false, 1, true>), \
                       dim3(p.grid), dim3(64 * W), 0, stream,                   \
                       static_cast<const uint16_t *>(x),                        \
                       static_cast<const uint8_t *>(Wt), y, nullptr, N, K, a.mp, a.per, \
                       a.gr);                                                   \
    break;
    Q4V_KSLICE_DOT_CASE(1) Q4V_KSLICE_DOT_CASE(2) Q4V_KSLICE_DOT_CASE(3)
    Q4V_KSLICE_DOT_CASE(4) Q4V_KSLICE_DOT_CASE(5) Q4V_KSLICE_DOT_CASE(6)
    Q4V_KSLICE_DOT_CASE(7) Q4V_KSLICE_DOT_CASE(8) Q4V_KSLICE_DOT_CASE(9)
    Q4V_KSLICE_DOT_CASE(10) Q4V_KSLICE_DOT_CASE(11) Q4V_KSLICE_DOT_CASE(12)
#undef Q4V_KSLICE_DOT_CASE
    default: return Q4_EINVAL;
  }
  return launch_status();
}

int launch_kslice(const q4_plan &p, const void *x, const void *Wt, float *y,
                  float *ws, int M, int N, int K, hipStream_t stream) {
  // sequential parts keep one running sum per tile of the workgroup; two
  // row tiles come on the tiled layout only, one record per wave
  if (p.k_seq_parts > 1 && p.row_tiles > static_cast<uint32_t>(kInMaxTiles))
    return Q4_EINVAL;
  if (p.m_tiles == 2 && (p.layout_id != Q4_LAYOUT_TILED16 || M <= Q4_MAX_ROWS))
    return Q4_EINVAL;
  if (p.m_tiles == 1 && M > Q4_MAX_ROWS) return Q4_EINVAL;
  const bool planar = p.layout_id == Q4_LAYOUT_PLANAR;
  switch (p.block / 64) {
#define Q4V_KSLICE_CASE(W)                                                  \
  case W:                                                                   \
    if (planar)                                                             \
      launch_kslice_w<W, false, true>(p, x, Wt, y, ws, M, N, K, stream);    \
    else                                                                    \
      launch_kslice_w<W, false, false>(p, x, Wt, y, ws, M, N, K, stream);   \
    break;
    Q4V_KSLICE_CASE(1) Q4V_KSLICE_CASE(2) Q4V_KSLICE_CASE(3)
    Q4V_KSLICE_CASE(4) Q4V_KSLICE_CASE(5) Q4V_KSLICE_CASE(6)
    Q4V_KSLICE_CASE(7) Q4V_KSLICE_CASE(8) Q4V_KSLICE_CASE(9)
    Q4V_KSLICE_CASE(10) Q4V_KSLICE_CASE(11) Q4V_KSLICE_CASE(12)
#undef Q4V_KSLICE_CASE
    default: return Q4_EINVAL;
  }
  int st = launch_status();
  if (st != Q4_OK || p.k_parts == 1) return st;
  return launch_reduce_parts(y, ws, M, N, static_cast<int>(p.k_parts), stream);
}

// The K-slice kernel with the fused sampling epilogue: candidate lists to
// cand instead of logits to y (one part of K, at most kSampleMaxTiles tiles
// per workgroup; the caller has checked both).
int launch_kslice_sample(const q4_plan &p, const void *x, const void *Wt,
                         uint64_t *cand, int M, int N, int K,
                         hipStream_t stream) {
  if (p.k_parts != 1 || p.k_seq_parts != 1 ||
      p.row_tiles > static_cast<uint32_t>(kSampleMaxTiles))
    return Q4_EINVAL;
  float *c = reinterpret_cast<float *>(cand);
  switch (p.block / 64) {
#define Q4V_KSLICE_SAMPLE_CASE(W)                                         \
  case W:                                                                 \
    launch_kslice_w<W, true>(p, x, Wt, nullptr, c, M, N, K, stream);      \
    break;
    Q4V_KSLICE_SAMPLE_CASE(1) Q4V_KSLICE_SAMPLE_CASE(2)
    Q4V_KSLICE_SAMPLE_CASE(3) Q4V_KSLICE_SAMPLE_CASE(4)
    Q4V_KSLICE_SAMPLE_CASE(5) Q4V_KSLICE_SAMPLE_CASE(6)
    Q4V_KSLICE_SAMPLE_CASE(7) Q4V_KSLICE_SAMPLE_CASE(8)
    Q4V_KSLICE_SAMPLE_CASE(9) Q4V_KSLICE_SAMPLE_CASE(10)
    Q4V_KSLICE_SAMPLE_CASE(11) Q4V_KSLICE_SAMPLE_CASE(12)
#undef Q4V_KSLICE_SAMPLE_CASE
    default: return Q4_EINVAL;
  }
  return launch_status();
}

template <int W, int RT>
void launch_resident_kernel(const q4_plan &p, const void *x, const void *Wt,
                            float *y, float *ws, int M, int N, int K,
                            hipStream_t stream) {
  const int parts = static_cast<int>(p.k_parts);
  hipLaunchKernelGGL((gemm_resident_kernel<W, kResidentStages, RT>),
                     dim3(p.grid), dim3(64 * W), 0, stream,
                     static_cast<const uint16_t *>(x),
                     static_cast<const uint8_t *>(Wt), y, ws, M, N, K, parts,
                     static_cast<int>(p.grid) / parts);
}

int launch_resident(const q4_plan &p, const void *x, const void *W, float *y,
                    float *ws, int M, int N, int K, hipStream_t stream) {
  const int parts = static_cast<int>(p.k_parts);
  const bool wide = p.block == 64 * kResidentWavesWide;
  if (p.m_tiles == 2) {
    if (wide)
      launch_resident_kernel<kResidentWavesWide, 2>(p, x, W, y, ws, M, N, K, stream);
    else
      launch_resident_kernel<kResidentWaves, 2>(p, x, W, y, ws, M, N, K, stream);
  } else {
    if (wide)
      launch_resident_kernel<kResidentWavesWide, 1>(p, x, W, y, ws, M, N, K, stream);
    else
      launch_resident_kernel<kResidentWaves, 1>(p, x, W, y, ws, M, N, K, stream);
  }
  int st = launch_status();
  if (st != Q4_OK || parts == 1) return st;
  return launch_reduce_parts(y, ws, M, N, parts, stream);
}

template <int NTW, int KSW>
int launch_gemm(const q4_plan &p, const void *x, const void *W, float *y,
                int M, int N, int K, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_verify_kernel<NTW, KSW, 4>), dim3(p.grid),
                     dim3(p.block), 0, stream, static_cast<const uint16_t *>(x),
                     static_cast<const uint8_t *>(W), y, M, N, K);
  return launch_status();
}

}  // namespace
}  // namespace q4v

extern "C" int q4_gemm_verify(const void *x, const void *W, float *y, int M,
                              int64_t N, int64_t K, void *stream) {
  int st = q4v::check_gemm_args(x, W, y, M, N, K);
  if (st != Q4_OK) return st;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  const q4_plan p = q4v::plan_gemm_planar(M, N, K, q4v::device_cus());
  if (p.kernel == Q4_KERNEL_TILED_KSLICE)  // the K-slice kernel, planar codes
    return q4v::launch_kslice(p, x, W, y, nullptr, M, n, k, s);
  switch (p.k_splits) {
    case 1: return q4v::launch_gemm<4, 1>(p, x, W, y, M, n, k, s);
    case 2: return q4v::launch_gemm<2, 2>(p, x, W, y, M, n, k, s);
    case 4: return q4v::launch_gemm<1, 4>(p, x, W, y, M, n, k, s);
    case 8: return q4v::launch_gemm<1, 8>(p, x, W, y, M, n, k, s);
    case 16: return q4v::launch_gemm<1, 16>(p, x, W, y, M, n, k, s);
    default: return Q4_EINVAL;
  }
}

extern "C" int q4_gemm_verify_tiled_dot(const void *x, const void *W, float *y,
                                        int M, int64_t N, int64_t K,
                                        void *stream) {
  int st = q4v::check_gemm_args(x, W, y, M, N, K, Q4_DOT_MAX_ROWS);
  if (st != Q4_OK) return st;
  st = q4v::check_tiled_shape(N, K);
  if (st != Q4_OK) return st;
  const q4_plan p = q4v::plan_gemm_tiled(M, N, K, q4v::device_cus());
  if (p.kernel != Q4_KERNEL_TILED_KSLICE || p.k_parts != 1 || p.k_seq_parts != 1)
    return Q4_EINVAL;  // K beyond 24 records
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  return q4v::launch_kslice_dot(p, x, W, y, M, static_cast<int>(N),
                                static_cast<int>(K), static_cast<hipStream_t>(stream));
}

extern "C" int q4_gemm_verify_tiled(const void *x, const void *W, float *y,
                                    int M, int64_t N, int64_t K,
                                    void *stream) {
  int st = q4v::check_gemm_args(x, W, y, M, N, K, Q4_MAX_ROWS_TILED);
  if (st != Q4_OK) return st;
  st = q4v::check_tiled_shape(N, K);
  if (st != Q4_OK) return st;
  const q4_plan p = q4v::plan_gemm_tiled(M, N, K, q4v::device_cus());
  if (p.grid == 0) return Q4_EINVAL;  // M > 16 with K > 2560: needs a workspace
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (p.kernel == Q4_KERNEL_TILED_KSLICE)
    return q4v::launch_kslice(p, x, W, y, nullptr, M, n, k, s);
  if (p.kernel == Q4_KERNEL_TILED_RESIDENT)
    return q4v::launch_resident(p, x, W, y, nullptr, M, n, k, s);
  const int key = static_cast<int>(p.tiles_per_wave * 100 + p.k_splits);
  switch (key) {
#define Q4V_TILED_CASE(TNT, KSW) \
  case TNT * 100 + KSW:          \
    return q4v::launch_tiled<TNT, 1, KSW>(p, x, W, y, M, n, k, s);
    Q4V_TILED_CASE(1, 1) Q4V_TILED_CASE(1, 2) Q4V_TILED_CASE(1, 4)
    Q4V_TILED_CASE(1, 8) Q4V_TILED_CASE(2, 1) Q4V_TILED_CASE(2, 2)
    Q4V_TILED_CASE(2, 4) Q4V_TILED_CASE(2, 8) Q4V_TILED_CASE(3, 1)
    Q4V_TILED_CASE(3, 2) Q4V_TILED_CASE(3, 4) Q4V_TILED_CASE(3, 8)
    Q4V_TILED_CASE(4, 1) Q4V_TILED_CASE(4, 2) Q4V_TILED_CASE(4, 4)
    Q4V_TILED_CASE(4, 8)
#undef Q4V_TILED_CASE
    default: return Q4_EINVAL;
  }
}

extern "C" int q4_gemm_verify_tiled_ws(const void *x, const void *W, float *y,
                                       int M, int64_t N, int64_t K,
                                       void *workspace,
                                       uint64_t workspace_bytes,
                                       void *stream) {
  int st = q4v::check_gemm_args(x, W, y, M, N, K, Q4_MAX_ROWS_TILED);
  if (st != Q4_OK) return st;
  st = q4v::check_tiled_shape(N, K);
  if (st != Q4_OK) return st;
  const q4_plan p = q4v::plan_gemm_tiled_ws(M, N, K, q4v::device_cus());
  if (p.grid == 0) return Q4_EINVAL;
  if (p.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < p.workspace_bytes)
      return Q4_EINVAL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return Q4_EALIGN;
  }
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  float *ws = static_cast<float *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (p.kernel == Q4_KERNEL_TILED_KSLICE)
    return q4v::launch_kslice(p, x, W, y, ws, M, n, k, s);
  if (p.kernel == Q4_KERNEL_TILED_RESIDENT)
    return q4v::launch_resident(p, x, W, y, ws, M, n, k, s);
  return q4_gemm_verify_tiled(x, W, y, M, N, K, stream);
}

// The plan of the LM-head GEMM with the fused sampling epilogue: the
// K-slice kernel in one part of K, at most kSampleMaxTiles tiles per
// workgroup; grid == 0 when the shape does not qualify.
static q4_plan plan_gemm_sample(int M, int64_t N, int64_t K) {
  q4_plan p = q4v::plan_gemm_tiled(M, N, K, q4v::device_cus());
  if (p.kernel != Q4_KERNEL_TILED_KSLICE || p.k_parts != 1 || p.k_seq_parts != 1 ||
      p.row_tiles > static_cast<uint32_t>(q4v::kSampleMaxTiles) || M > Q4_MAX_ROWS)
    p.grid = 0;
  return p;
}

extern "C" int q4_gemm_verify_sample_workspace(int M, int64_t N, int64_t K,
                                               uint64_t *bytes) {
  if (bytes == nullptr || M < 1 || M > Q4_MAX_ROWS) return Q4_EINVAL;
  int st = q4v::check_tiled_shape(N, K);
  if (st != Q4_OK) return st;
  const q4_plan p = plan_gemm_sample(M, N, K);
  if (p.grid == 0) return Q4_EINVAL;
  *bytes = static_cast<uint64_t>(M) * p.grid * q4v::kSampleTop * 8;
  return Q4_OK;
}

extern "C" int q4_gemm_verify_sample(
    const void *x, const void *W, int M, int64_t N, int64_t K,
    const q4_sample_params *prm, const int32_t *draft_tok,
    const int32_t *draft_idx, const float *draft_q, const float *u,
    const float *v, int32_t *top_idx, float *top_val, float *top_prob,
    int32_t *greedy, int32_t *accept, int32_t *token, void *workspace,
    uint64_t workspace_bytes, void *stream) {
  uint64_t need = 0;
  int st = q4_gemm_verify_sample_workspace(M, N, K, &need);
  if (st != Q4_OK) return st;
  // y is not written: its alignment rule is checked on a stand-in
  st = q4v::check_gemm_args(x, W, reinterpret_cast<const float *>(W), M, N, K);
  if (st != Q4_OK) return st;
  st = q4v::check_sample_args(M, N, prm, draft_tok, draft_idx, draft_q, u, v,
                              top_idx, top_val, top_prob, greedy, accept,
                              token);
  if (st != Q4_OK) return st;
  if (workspace == nullptr || workspace_bytes < need) return Q4_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return Q4_EALIGN;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  const q4_plan p = plan_gemm_sample(M, N, K);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t *cand = static_cast<uint64_t *>(workspace);
  st = q4v::launch_kslice_sample(p, x, W, cand, M, static_cast<int>(N),
                                 static_cast<int>(K), s);
  if (st != Q4_OK) return st;
  return q4v::launch_sample_rows(cand, M, static_cast<int>(p.grid), *prm,
                                 draft_tok, draft_idx, draft_q, u, v, top_idx,
                                 top_val, top_prob, greedy, accept, token, s);
}

namespace {

// Device address of `scratch` on the current device, looked up with that
// device current on the first call there and kept per device ordinal.
int noalloc_scratch(void **out) {
  static std::atomic<void *> addr[256];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) {
    (void)hipGetLastError();
    return Q4_EDEVICE;
  }
  void *p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess ||
        p == nullptr) {
      (void)hipGetLastError();
      return Q4_EDEVICE;
    }
    addr[dev].store(p, std::memory_order_release);  // the same value if raced
  }
  *out = p;
  return Q4_OK;
}

}  // namespace

extern "C" int q4_gemm_verify_tiled_noalloc(const void *x, const void *W,
                                            float *y, int M, int64_t N,
                                            int64_t K, void *stream) {
  int st = q4v::check_gemm_args(x, W, y, M, N, K, Q4_MAX_ROWS_TILED);
  if (st != Q4_OK) return st;
  st = q4v::check_tiled_shape(N, K);
  if (st != Q4_OK) return st;
  const q4_plan p = q4v::plan_gemm_tiled_ws(M, N, K, q4v::device_cus());
  if (p.grid == 0) return Q4_EINVAL;
  if (p.workspace_bytes > Q4_NOALLOC_SCRATCH_BYTES) return Q4_ESCRATCH;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  void *ws = nullptr;
  if (p.workspace_bytes > 0) {
    st = noalloc_scratch(&ws);
    if (st != Q4_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  float *w = static_cast<float *>(ws);
  if (p.kernel == Q4_KERNEL_TILED_KSLICE)
    return q4v::launch_kslice(p, x, W, y, w, M, n, k, s);
  if (p.kernel == Q4_KERNEL_TILED_RESIDENT)
    return q4v::launch_resident(p, x, W, y, w, M, n, k, s);
  return q4_gemm_verify_tiled(x, W, y, M, N, K, stream);
}

extern "C" int q4_repack(const void *W, void *W_tiled, int64_t N, int64_t K,
                         void *stream) {
  int st = q4v::check_dequant_args(W, static_cast<const float *>(W_tiled), N, K);
  if (st != Q4_OK) return st;
  st = q4v::check_tiled_shape(N, K);
  if (st != Q4_OK) return st;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  const uint64_t units = static_cast<uint64_t>(N) * static_cast<uint64_t>(K) * 9 / 256;
  const uint64_t want = (units + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(q4v::repack_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t *>(W),
                     static_cast<q4v::u32x4 *>(W_tiled), static_cast<int>(N),
                     static_cast<int>(K));
  return q4v::launch_status();
}

extern "C" int q4_dequant(const void *W, float *W_out, int64_t N, int64_t K,
                          void *stream) {
  int st = q4v::check_dequant_args(W, W_out, N, K);
  if (st != Q4_OK) return st;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  const uint64_t words = static_cast<uint64_t>(N) * static_cast<uint64_t>(K) / 8;
  const uint64_t want = (words + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(q4v::dequant_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t *>(W), W_out,
                     static_cast<int>(N), static_cast<int>(K));
  return q4v::launch_status();
}

extern "C" int q4_stream_read(const void *buf, uint64_t bytes, uint32_t *sink,
                              void *stream) {
  int st = q4v::check_stream_args(buf, sink, bytes);
  if (st != Q4_OK) return st;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  const uint64_t n16 = bytes / 16;
  // one workgroup per CU, each at least 8 KiB
  const uint64_t cus = static_cast<uint64_t>(q4v::device_cus());
  const uint64_t want = (n16 + 511) / 512;
  const uint64_t blocks = want < cus ? want : cus;
  const uint64_t chunk16 = (n16 + blocks - 1) / blocks;
  // deeper unrolling only pays on shares of a MiB or more
  if (chunk16 >= (1u << 16))
    hipLaunchKernelGGL(q4v::stream_read_kernel<8>, dim3(static_cast<unsigned>(blocks)),
                       dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const q4v::u32x4 *>(buf), n16, chunk16, sink);
  else
    hipLaunchKernelGGL(q4v::stream_read_kernel<4>, dim3(static_cast<unsigned>(blocks)),
                       dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const q4v::u32x4 *>(buf), n16, chunk16, sink);
  return q4v::launch_status();
}

extern "C" int q4_stream_copy(const void *src, void *dst, uint64_t bytes,
                              void *stream) {
  int st = q4v::check_stream_args(src, dst, bytes);
  if (st != Q4_OK) return st;
  if ((reinterpret_cast<uintptr_t>(dst) & 15u) != 0) return Q4_EALIGN;
  st = q4v::check_device();
  if (st != Q4_OK) return st;
  const uint64_t n16 = bytes / 16;
  const uint64_t want = (n16 + 1023) / 1024;
  const unsigned blocks = static_cast<unsigned>(want < 8192 ? (want ? want : 1) : 8192);
  hipLaunchKernelGGL(q4v::stream_copy_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const q4v::u32x4 *>(src),
                     static_cast<q4v::u32x4 *>(dst), n16);
  return q4v::launch_status();
}
