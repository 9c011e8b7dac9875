// q4v_internal.h -- declarations shared by the library's host and device
// translation units (not part of the public ABI).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "q4verify.h"

namespace q4v {

// Argument checks of q4_gemm_verify / q4_dequant that need no device: sizes,
// NULL pointers, alignment and 64-bit overflow.  Return Q4_OK or an error.
int check_matrix_shape(int64_t N, int64_t K);
int check_gemm_args(const void *x, const void *W, const float *y, int M,
                    int64_t N, int64_t K, int max_rows = Q4_MAX_ROWS);
int check_dequant_args(const void *W, const float *W_out, int64_t N,
                       int64_t K);
int check_stream_args(const void *a, const void *b, uint64_t bytes);
// Extra shape rule of Q4_LAYOUT_TILED16: N % 16 == 0 and K % 256 == 0.
int check_tiled_shape(int64_t N, int64_t K);

// Launch plans of the two GEMM kernels (see q4_gemm_verify_plan); the shape
// has already been checked.
// `cus` is the compute-unit count of the device the plan is for.
q4_plan plan_gemm_planar(int M, int64_t N, int64_t K, int cus);
q4_plan plan_gemm_tiled(int M, int64_t N, int64_t K, int cus);
// Plan of the K-slice kernel for `parts` groups of workgroups, each taking
// `seq` parts of K in turn, on weights in Q4_LAYOUT_* `layout`; false when
// the shape does not fit it.
bool plan_kslice(int M, int64_t N, int64_t K, int cus, int parts, int seq,
                 uint32_t layout, q4_plan *out);
// Parts of K a K-slice workgroup takes in turn when nothing else splits K.
int seq_parts_for(int64_t K, int M);
// The plan of the workspace path (q4_gemm_verify_tiled_ws).
q4_plan plan_gemm_tiled_ws(int M, int64_t N, int64_t K, int cus);

// Bytes of one record of the tiled layout: 16 rows x 4 groups x 36 bytes.
constexpr int kTileRows = 16;
constexpr int kRecordGroups = 4;
constexpr int kRecordBytes = kTileRows * kRecordGroups * 36;

// LDS of one gfx950 CU (and the most one workgroup may use), and the largest
// K whose 16 activation rows fit in it as bf16.
constexpr int kLdsBytes = 163840;
constexpr int kResidentMaxK = kLdsBytes / 32;
constexpr int kResidentMaxRecords = kResidentMaxK / 256;  // per part, M <= 16
// Waves per workgroup (two sizes) and register stages of the
// resident-activation kernel.  A workgroup with at least
// kResidentWideTiles tiles runs the wider size: twice the records in flight
// per CU (measured on MI355X: gate+up and the LM head 15 % faster, the
// shapes with 4-5 tiles per CU no faster).
constexpr int kResidentWaves = 8;
constexpr int kResidentWavesWide = 16;
constexpr int kResidentWideTiles = 8;
constexpr int kResidentStages = 2;
// K-slice kernel: two records of every tile per wave, so at most 12 waves
// (K <= 6144); tiles per reduction batch fill the LDS with the waves'
// partial sums (16 x 10 x 1 KiB at K = 5120).
constexpr int kKsliceMaxRecords = 24;
// With K beyond kKsliceMaxRecords records and no workspace, a workgroup
// takes the parts of K one after another and keeps each of its tiles'
// running sums in LDS: at most kInMaxTiles tiles per workgroup then.
constexpr int kInMaxTiles = 16;
constexpr int kKsliceBatchLds = kLdsBytes - kInMaxTiles * 1024;
// LDS of the K-slice kernel's partial sums for W waves.
constexpr int kslice_batch(int W) { return kKsliceBatchLds / (W * 1024); }
// M = 17..32: two row tiles, so 2 KiB of partial sums per wave and tile, and
// the sequential parts' running sums (kInMaxTiles tiles) take 2 KiB a tile.
constexpr int kslice_batch2(int W, bool seq) {
  return (kLdsBytes - 1024 - (seq ? kInMaxTiles * 2048 : 0)) / (W * 2048);
}
// At most this many records per part at M = 17..32 (one per wave).
constexpr int kKsliceMaxRecords2 = 12;
// On the planar layout each wave also stages its two records' codes of one
// tile in LDS (4 KiB per wave), and the workgroup the scales and biases of
// the current and the next tile (at most 24 records: 6 KiB per tile); the
// sequential parts then keep at most kInMaxTilesPlanar running sums.
constexpr int kPlanarCodeLds = 4096;
constexpr int kPlanarSbLds = 2 * 16 * kKsliceMaxRecords * 8;
constexpr int kInMaxTilesPlanar = 4;
constexpr int kslice_planar_batch(int W, bool seq) {
  return (kLdsBytes - 2 * kPlanarSbLds - (seq ? kInMaxTilesPlanar * 1024 : 0) -
          W * kPlanarCodeLds) / (W * 1024);
}

// The verify sampling epilogue's argument rules (sizes, parameters, NULL
// pointers) and its second kernel: row m merges the S candidate lists of 32
// keys each at cand[(m * S + s) * 32 ..] and samples (see
// q4verify_sample.hip).  Shared by q4_verify_sample and the LM-head GEMM with
// the fused epilogue.
int check_sample_args(int M, int64_t V, const q4_sample_params *prm,
                      const int32_t *draft_tok, const int32_t *draft_idx,
                      const float *draft_q, const float *u, const float *v,
                      int32_t *top_idx, float *top_val, float *top_prob,
                      int32_t *greedy, int32_t *accept, int32_t *token);
int launch_sample_rows(const uint64_t *cand, int M, int S,
                       const q4_sample_params &p, const int32_t *draft_tok,
                       const int32_t *draft_idx, const float *draft_q,
                       const float *u, const float *v, int32_t *top_idx,
                       float *top_val, float *top_prob, int32_t *greedy,
                       int32_t *accept, int32_t *token, hipStream_t s);
// Candidate lists of the fused LM-head epilogue: 32 keys per workgroup and
// row; a workgroup holds at most kSampleMaxTiles tiles (1024 logits of each
// row) in LDS.
constexpr int kSampleTop = 32;
// Lists per row that the row kernel merges (workgroups of the fused GEMM,
// slices of the standalone epilogue).
constexpr int kSampleMaxLists = 512;
constexpr int kSampleMaxTiles = 64;
constexpr int kSampleMaxCols = kSampleMaxTiles * 16;
constexpr int kSampleLgStride = kSampleMaxCols;  // floats per row in LDS
constexpr int kSampleLgBytes = Q4_MAX_ROWS * kSampleLgStride * 4;
// Tiles per reduction batch of the K-slice kernel with the fused epilogue:
// the rest of the LDS after the logits.
constexpr int kslice_sample_batch(int W) {
  return (kLdsBytes - kSampleLgBytes) / (W * 1024);
}

// Q4_OK when a HIP device is current and it is a gfx950; Q4_EDEVICE
// otherwise.  The answer is cached per device ordinal.
int check_device();

// Compute units of the current device (cached per ordinal); 256, the
// MI355X's count, when no device can be queried.
int device_cus();

}  // namespace q4v
