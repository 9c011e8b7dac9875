// q4verify_host.cpp -- host-only part of the library: the packed layout,
// argument checks, device check and status strings.  Nothing here touches the
// GPU except check_device(), which asks the HIP runtime for the current
// device's architecture.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "q4v_internal.h"

namespace q4v {
namespace {

constexpr int64_t kMaxIndex = 2147483647;  // rows and inputs are int32 in kernels
constexpr int64_t kMaxTiledK = int64_t{1} << 26;

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// N*K/16*9 with overflow checks (the q4PackedBytes rule of the Splash engine
// article, section "The engine hard-codes the model").
int packed_bytes(int64_t N, int64_t K, uint64_t *out) {
  if (N < 1 || K < Q4_GROUP || K % Q4_GROUP != 0) return Q4_EINVAL;
  uint64_t elements;
  if (__builtin_mul_overflow(static_cast<uint64_t>(N),
                             static_cast<uint64_t>(K), &elements))
    return Q4_EOVERFLOW;
  uint64_t bytes;
  if (__builtin_mul_overflow(elements / 16u, uint64_t{9}, &bytes))
    return Q4_EOVERFLOW;
  *out = bytes;
  return Q4_OK;
}

}  // namespace

int check_matrix_shape(int64_t N, int64_t K) {
  uint64_t bytes;
  const int st = packed_bytes(N, K, &bytes);
  if (st != Q4_OK) return st;
  if (N > kMaxIndex || K > kMaxIndex - Q4_GROUP + 1) return Q4_EINVAL;
  // Element offsets n*K (dequant output) are 64-bit in the kernels; they
  // must also fit 64 bits as byte offsets of an fp32 array.
  uint64_t elems, out_bytes;
  if (__builtin_mul_overflow(static_cast<uint64_t>(N),
                             static_cast<uint64_t>(K), &elems) ||
      __builtin_mul_overflow(elems, uint64_t{4}, &out_bytes))
    return Q4_EOVERFLOW;
  return Q4_OK;
}

int check_gemm_args(const void *x, const void *W, const float *y, int M,
                    int64_t N, int64_t K, int max_rows) {
  if (M < 1 || M > max_rows) return Q4_EINVAL;
  const int st = check_matrix_shape(N, K);
  if (st != Q4_OK) return st;
  if (x == nullptr || W == nullptr || y == nullptr) return Q4_EINVAL;
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(y, 4)) return Q4_EALIGN;
  return Q4_OK;
}

int check_dequant_args(const void *W, const float *W_out, int64_t N,
                       int64_t K) {
  const int st = check_matrix_shape(N, K);
  if (st != Q4_OK) return st;
  if (W == nullptr || W_out == nullptr) return Q4_EINVAL;
  if (!aligned(W, 16) || !aligned(W_out, 16)) return Q4_EALIGN;
  return Q4_OK;
}

int check_stream_args(const void *a, const void *b, uint64_t bytes) {
  if (a == nullptr || b == nullptr || bytes == 0 || bytes % 16 != 0)
    return Q4_EINVAL;
  if (!aligned(a, 16)) return Q4_EALIGN;
  return Q4_OK;
}

int check_tiled_shape(int64_t N, int64_t K) {
  const int st = check_matrix_shape(N, K);
  if (st != Q4_OK) return st;
  if (N % kTileRows != 0 || K % (kRecordGroups * Q4_GROUP) != 0)
    return Q4_EINVAL;
  // buffer offsets are 32-bit: M*K*2 activation bytes and K*9 bytes of one
  // tile's records must stay below 2^32
  if (K > kMaxTiledK) return Q4_EINVAL;
  return Q4_OK;
}

q4_plan plan_gemm_planar(int M, int64_t N, int64_t K, int cus) {
  {
    // the K-slice kernel on the planar codes (K % 256 == 0, up to 16 rows)
    q4_plan p;
    if (plan_kslice(M, N, K, cus, 1, seq_parts_for(K, M), Q4_LAYOUT_PLANAR, &p))
      return p;
  }
  // Waves per tile splitting K so that the grid holds enough waves (about 16
  // per CU on 256 CUs) to keep the weight stream in flight, with at least
  // four groups per wave; large-N shapes put several tiles in a workgroup.
  const int64_t tiles = (N + 15) / 16;
  const int64_t groups = K / Q4_GROUP;
  int ksw = 1;
  while (ksw < 16 && tiles * ksw < 4096 && groups >= 4 * ksw) ksw *= 2;
  const int ntw = ksw >= 4 ? 1 : 4 / ksw;
  q4_plan p;
  std::memset(&p, 0, sizeof p);
  p.row_tiles = static_cast<uint32_t>(ntw);
  p.tiles_per_wave = 1;
  p.k_splits = static_cast<uint32_t>(ksw);
  p.block = static_cast<uint32_t>(64 * ntw * ksw);
  p.grid = static_cast<uint32_t>((tiles + ntw - 1) / ntw);
  p.lookahead = 4;
  p.kernel = Q4_KERNEL_PLANAR;
  p.k_parts = 1;
  p.k_seq_parts = 1;
  p.layout_id = Q4_LAYOUT_PLANAR;
  p.m_tiles = 1;
  p.lds_bytes = ksw > 1 ? static_cast<uint32_t>(ksw * ntw * 64 * 16) : 0;
  return p;
}

// Plan of the resident-activation kernel with K split into `parts` parts
// (one group of workgroups per part, one workgroup per CU); false when a
// part's activations exceed the LDS or a wave's 32-bit buffer offsets could
// overflow (then the streaming kernel runs).
bool plan_resident(int M, int64_t N, int64_t K, int cus, int parts,
                   q4_plan *out) {
  const int64_t tiles = N / kTileRows;
  const int64_t records = K / (kRecordGroups * Q4_GROUP);
  const int m_tiles = M > Q4_MAX_ROWS ? 2 : 1;
  if (parts < 1 ||
      (records + parts - 1) / parts > kResidentMaxRecords / m_tiles)
    return false;
  int64_t gt = cus / parts;
  if (gt < 1) gt = 1;
  if (gt > tiles) gt = tiles;
  // a wave's resource spans at most its workgroup's tiles, all records
  const int64_t span = ((tiles + gt - 1) / gt) * records * kRecordBytes;
  if (span >= 0x7FFFFFF0LL) return false;
  q4_plan p;
  std::memset(&p, 0, sizeof p);
  p.grid = static_cast<uint32_t>(gt * parts);
  p.row_tiles = static_cast<uint32_t>((tiles + gt - 1) / gt);
  p.block = 64 * (p.row_tiles >= static_cast<uint32_t>(kResidentWideTiles)
                      ? kResidentWavesWide
                      : kResidentWaves);
  p.tiles_per_wave = 1;
  p.k_splits = 1;
  p.lookahead = kRecordGroups * (kResidentStages - 1);
  p.kernel = Q4_KERNEL_TILED_RESIDENT;
  p.k_seq_parts = 1;
  p.layout_id = Q4_LAYOUT_TILED16;
  p.lds_bytes = kLdsBytes;
  p.k_parts = static_cast<uint32_t>(parts);
  p.m_tiles = static_cast<uint32_t>(m_tiles);
  p.workspace_bytes = static_cast<uint64_t>(parts - 1) *
                      static_cast<uint64_t>(M) * static_cast<uint64_t>(N) * 4;
  *out = p;
  return true;
}

// Plan of the K-slice kernel (M <= 16): ceil(Q_p / 2) waves for parts of
// Q_p <= 24 records.  K is cut into P * seq parts: P groups of workgroups
// take one part each (parts 1 .. P-1 write a workspace), and within a group
// every workgroup takes its seq parts one after another, keeping its tiles'
// running sums on chip (then at most kInMaxTiles tiles per workgroup).  With
// one part group one workgroup per CU owns a run of tiles; with P groups the
// grid is P groups of min(tiles, CUs / P) workgroups.  layout is the
// weights' Q4_LAYOUT_*: the planar layout takes any N (the last tile's rows
// past N read zeros) and K % 256 == 0.
bool plan_kslice(int M, int64_t N, int64_t K, int cus, int parts, int seq,
                 uint32_t layout, q4_plan *out) {
  // M = 17..32: two row tiles, one record per wave (tiled layout only)
  const int rt = M > Q4_MAX_ROWS ? 2 : 1;
  if (M > Q4_MAX_ROWS_TILED || parts < 1 || seq < 1 || parts > cus || N < 1 ||
      K < kRecordGroups * Q4_GROUP || K % (kRecordGroups * Q4_GROUP) != 0 ||
      (rt == 2 && layout != Q4_LAYOUT_TILED16))
    return false;
  const int64_t tiles = (N + kTileRows - 1) / kTileRows;
  const int64_t records = K / (kRecordGroups * Q4_GROUP);
  const int64_t nparts = static_cast<int64_t>(parts) * seq;
  const int64_t part_records = (records + nparts - 1) / nparts;
  if (part_records > (rt == 2 ? kKsliceMaxRecords2 : kKsliceMaxRecords) ||
      nparts > records)
    return false;
  const int64_t per_part_cus = cus / parts;
  const int64_t g0 = tiles < per_part_cus ? tiles : per_part_cus;
  const int64_t per = (tiles + g0 - 1) / g0;
  // With 3 or more tiles per workgroup, just enough workgroups for `per`
  // tiles each, so that none finishes a tile after the others (gate+up:
  // 242 x 9 tiles instead of 256 x 8 or 9, 20.9 against 21.9 us at M = 16
  // on MI355X); with fewer, every CU's share matters more.
  const int64_t g = per >= 3 ? (tiles + per - 1) / per : g0;
  // the kernel's index arithmetic (packed arguments, fp32 quotients) takes
  // fewer than 4096 workgroups per part and parts
  if (g >= 4096 || nparts >= 4096) return false;
  const bool planar = layout == Q4_LAYOUT_PLANAR;
  if (seq > 1 && per > (planar ? kInMaxTilesPlanar : kInMaxTiles)) return false;
  // planar: one resource over a workgroup's scales and the biases after them
  if (planar && N * (K / 32) + per * kTileRows * (K / 32) >= 0x7FFFFFF0LL) return false;
  // 32-bit buffer offsets over a workgroup's weights
  const int64_t span = layout == Q4_LAYOUT_PLANAR
                           ? per * kTileRows * (K / 2)
                           : per * records * kRecordBytes;
  if (span >= 0x7FFFFFF0LL) return false;
  const int waves = static_cast<int>(rt == 2 ? part_records : (part_records + 1) / 2);
  q4_plan p;
  std::memset(&p, 0, sizeof p);
  p.grid = static_cast<uint32_t>(g * parts);
  p.block = static_cast<uint32_t>(64 * waves);
  p.row_tiles = static_cast<uint32_t>(per);
  p.tiles_per_wave = 1;
  p.k_splits = static_cast<uint32_t>(waves);
  p.lookahead = kRecordGroups * 2;
  p.kernel = Q4_KERNEL_TILED_KSLICE;
  p.lds_bytes = static_cast<uint32_t>(
      planar    ? kslice_planar_batch(waves, seq > 1) * waves * 1024 +
                      waves * kPlanarCodeLds + 2 * kPlanarSbLds +
                      (seq > 1 ? kInMaxTilesPlanar * 1024 : 0)
      : rt == 2 ? kslice_batch2(waves, seq > 1) * waves * 2048 +
                      (seq > 1 ? kInMaxTiles * 2048 : 0)
      : seq > 1 ? kslice_batch(waves) * waves * 1024 + kInMaxTiles * 1024
                // one part, at most 10 waves: the activation rows go straight
                // to LDS, 16 KB per wave, in the partial-sum area
                : std::max(kslice_batch(waves), waves <= 10 ? 16 : 0) * waves * 1024);
  p.k_parts = static_cast<uint32_t>(parts);
  p.k_seq_parts = static_cast<uint32_t>(seq);
  p.m_tiles = static_cast<uint32_t>(rt);
  p.layout_id = layout;
  p.workspace_bytes = static_cast<uint64_t>(parts - 1) *
                      static_cast<uint64_t>(M) * static_cast<uint64_t>(N) * 4;
  *out = p;
  return true;
}

// Parts of K taken one after another by each workgroup, for the K-slice
// kernel without a workspace (at most 24 records a part, 12 at M > 16).
int seq_parts_for(int64_t K, int M) {
  const int64_t records = K / (kRecordGroups * Q4_GROUP);
  const int64_t most = M > Q4_MAX_ROWS ? kKsliceMaxRecords2 : kKsliceMaxRecords;
  const int64_t s = (records + most - 1) / most;
  return s < 1 ? 1 : s > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(s);
}

q4_plan plan_gemm_tiled_ws(int M, int64_t N, int64_t K, int cus) {
  // Up to 16 rows the K-slice kernel: in one part up to 24 records per tile,
  // beyond that in P parts of K (at least 4, a power of two, so that the 320
  // tiles of the N = 5120 projections give every CU whole tiles): 15.9
  // against 16.9 us for the resident kernel's split on 5120 x 17408 at
  // M = 16, measured on MI355X.  32 rows: the K-slice kernel with two row
  // tiles, else the resident kernel, split whenever its activations exceed
  // the LDS.
  const int m_tiles = M > Q4_MAX_ROWS ? 2 : 1;
  const int64_t records = K / (kRecordGroups * Q4_GROUP);
  if (m_tiles == 1) {
    // no split for K <= 6144; the rule looks at (N, K) only, so that every
    // M <= 16 runs the same plan and a row's bits do not depend on M
    if (records <= kKsliceMaxRecords) return plan_gemm_tiled(M, N, K, cus);
    int64_t parts = 4;
    while (parts * kKsliceMaxRecords < records) parts *= 2;
    q4_plan p;
    if (plan_kslice(M, N, K, cus, static_cast<int>(parts), 1, Q4_LAYOUT_TILED16, &p))
      return p;
    return plan_gemm_tiled(M, N, K, cus);
  }
  {
    // 32 rows: the K-slice kernel with two row tiles on the same unpacked
    // codes, one record per wave, so at most 12 records a part: P parts of
    // K across workgroups (a power of two)
    int64_t parts = 1;
    while (parts * kKsliceMaxRecords2 < records) parts *= 2;
    q4_plan p;
    if (plan_kslice(M, N, K, cus, static_cast<int>(parts), 1, Q4_LAYOUT_TILED16, &p))
      return p;
  }
  const int64_t per_part = kResidentMaxRecords / m_tiles;
  if (records > per_part) {
    // 32 rows: split whenever the activations exceed the LDS, into a power
    // of two parts (2 for K = 5120, 8 for 17408)
    int64_t parts = 2;
    while (parts * per_part < records) parts *= 2;
    q4_plan p;
    if (parts <= cus && plan_resident(M, N, K, cus, static_cast<int>(parts), &p))
      return p;
    std::memset(&p, 0, sizeof p);  // no plan: the call is rejected
    return p;
  }
  return plan_gemm_tiled(M, N, K, cus);
}

q4_plan plan_gemm_tiled(int M, int64_t N, int64_t K, int cus) {
  const int64_t tiles = N / kTileRows;
  {
    // Up to 16 rows: each wave keeps its slice of K of the activations in
    // registers (measured on MI355X: gate+up, the LM head and the GDN
    // in-projection faster than with the activations in LDS, attention's
    // in-projection at M = 16 even); beyond 24 records per tile the
    // workgroups take the parts of K one after another.
    q4_plan p;
    if (plan_kslice(M, N, K, cus, 1, seq_parts_for(K, M), Q4_LAYOUT_TILED16, &p))
      return p;
  }
  if (K <= kResidentMaxK) {
    // Activations resident in LDS: one workgroup per CU (the LDS admits no
    // second), each owning whole tiles; its waves split its records evenly.
    q4_plan p;
    if (plan_resident(M, N, K, cus, 1, &p)) return p;
  }
  if (M > Q4_MAX_ROWS) {  // 32 rows without a workspace: resident only
    q4_plan p;
    std::memset(&p, 0, sizeof p);
    return p;
  }
  // Tiles per wave: each wave multiplies its activation operand with 1-4
  // tiles, so the activation loads per weight byte fall with more tiles
  // while the registers per wave (and so the waves per SIMD) rise; wide
  // matrices take more.  Waves splitting K (one workgroup = those waves) are
  // then added until about 1024 waves stream at once, keeping at least one
  // 4-group record per wave.  Both rules follow measured sweeps on MI355X of
  // the 27B model's projection shapes.
  const int64_t records = K / (kRecordGroups * Q4_GROUP);
  const int tnt = tiles >= 4096 ? 4 : tiles >= 1536 ? 3 : tiles >= 2 ? 2 : 1;
  const int64_t sets = (tiles + tnt - 1) / tnt;
  int ksw = 1;
  while (ksw < 8 && sets * ksw < 1024 && records >= 2 * ksw) ksw *= 2;
  q4_plan p;
  std::memset(&p, 0, sizeof p);
  p.row_tiles = static_cast<uint32_t>(tnt);
  p.tiles_per_wave = static_cast<uint32_t>(tnt);
  p.k_splits = static_cast<uint32_t>(ksw);
  p.block = static_cast<uint32_t>(64 * ksw);
  p.grid = static_cast<uint32_t>(sets);
  p.lookahead = kRecordGroups;
  p.kernel = Q4_KERNEL_TILED_STREAM;
  p.k_seq_parts = 1;
  p.layout_id = Q4_LAYOUT_TILED16;
  p.k_parts = 1;
  p.m_tiles = 1;
  p.lds_bytes = ksw > 1 ? static_cast<uint32_t>(ksw * tnt * 64 * 16) : 0;
  return p;
}

int check_device() {
  static std::atomic<int> verdict[256];  // 0 unknown, 1 gfx950, -1 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return Q4_EDEVICE;
  }
  if (dev >= 256) return Q4_EDEVICE;
  int v = verdict[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return Q4_EDEVICE;
    }
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    verdict[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? Q4_OK : Q4_EDEVICE;
}

int device_cus() {
  static std::atomic<int> cached[256];  // 0 unknown
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        n < 1) {
      (void)hipGetLastError();
      return 256;
    }
    v = n;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace q4v

extern "C" int q4_pack_layout(int64_t N, int64_t K, uint32_t layout_id,
                              q4_layout *out) {
  if (out == nullptr) return Q4_EINVAL;
  if (layout_id != Q4_LAYOUT_PLANAR && layout_id != Q4_LAYOUT_TILED16)
    return Q4_EINVAL;
  uint64_t total;
  int st = q4v::packed_bytes(N, K, &total);
  if (st != Q4_OK) return st;
  if (layout_id == Q4_LAYOUT_TILED16) {
    st = q4v::check_tiled_shape(N, K);
    if (st != Q4_OK) return st;
    q4_layout l;
    std::memset(&l, 0, sizeof l);
    l.abi_version = Q4_ABI_VERSION;
    l.layout_id = layout_id;
    l.N = N;
    l.K = K;
    l.group = Q4_GROUP;
    l.total_bytes = total;
    l.tile_rows = q4v::kTileRows;
    l.record_groups = q4v::kRecordGroups;
    l.record_bytes = q4v::kRecordBytes;
    *out = l;
    return Q4_OK;
  }
  const uint64_t elements = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  q4_layout l;
  std::memset(&l, 0, sizeof l);
  l.abi_version = Q4_ABI_VERSION;
  l.layout_id = layout_id;
  l.N = N;
  l.K = K;
  l.group = Q4_GROUP;
  l.total_bytes = total;
  l.code_off = 0;
  l.code_bytes = elements / 2;
  l.scale_off = l.code_off + l.code_bytes;
  l.scale_bytes = (elements / Q4_GROUP) * 2;
  l.bias_off = l.scale_off + l.scale_bytes;
  l.bias_bytes = l.scale_bytes;
  *out = l;
  return Q4_OK;
}

extern "C" int q4_gemm_verify_plan(int M, int64_t N, int64_t K,
                                   uint32_t layout_id, q4_plan *out) {
  if (out == nullptr || M < 1 || M > Q4_MAX_ROWS_TILED) return Q4_EINVAL;
  if (layout_id == Q4_LAYOUT_PLANAR) {
    if (M > Q4_MAX_ROWS) return Q4_EINVAL;
    const int st = q4v::check_matrix_shape(N, K);
    if (st != Q4_OK) return st;
    *out = q4v::plan_gemm_planar(M, N, K, q4v::device_cus());
    return Q4_OK;
  }
  if (layout_id == Q4_LAYOUT_TILED16) {
    const int st = q4v::check_tiled_shape(N, K);
    if (st != Q4_OK) return st;
    const q4_plan p = q4v::plan_gemm_tiled(M, N, K, q4v::device_cus());
    if (p.grid == 0) return Q4_EINVAL;
    *out = p;
    return Q4_OK;
  }
  return Q4_EINVAL;
}

extern "C" int q4_gemm_verify_tiled_ws_plan(int M, int64_t N, int64_t K,
                                            q4_plan *out) {
  if (out == nullptr || M < 1 || M > Q4_MAX_ROWS_TILED) return Q4_EINVAL;
  const int st = q4v::check_tiled_shape(N, K);
  if (st != Q4_OK) return st;
  const q4_plan p = q4v::plan_gemm_tiled_ws(M, N, K, q4v::device_cus());
  if (p.grid == 0) return Q4_EINVAL;
  *out = p;
  return Q4_OK;
}

extern "C" const char *q4_status_string(int status) {
  switch (status) {
    case Q4_OK: return "Q4_OK: success";
    case Q4_EINVAL: return "Q4_EINVAL: invalid size, pointer or layout id";
    case Q4_EALIGN: return "Q4_EALIGN: pointer not aligned as required";
    case Q4_EOVERFLOW: return "Q4_EOVERFLOW: byte count overflows 64 bits";
    case Q4_EDEVICE: return "Q4_EDEVICE: no HIP device or device is not gfx950";
    case Q4_ELAUNCH: return "Q4_ELAUNCH: kernel launch failed";
    case Q4_ESCRATCH:
      return "Q4_ESCRATCH: the call needs more than the library's static "
             "scratch (Q4_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown q4 status";
  }
}
