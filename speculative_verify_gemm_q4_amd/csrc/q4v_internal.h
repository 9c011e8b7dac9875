// q4v_internal.h -- declarations shared by the library's host and device
// translation units (not part of the public ABI).
#pragma once

#include <stdint.h>

#include "q4verify.h"

namespace q4v {

// Argument checks of q4_gemm_verify / q4_dequant that need no device: sizes,
// NULL pointers, alignment and 64-bit overflow.  Return Q4_OK or an error.
int check_matrix_shape(int64_t N, int64_t K);
int check_gemm_args(const void *x, const void *W, const float *y, int M,
                    int64_t N, int64_t K);
int check_dequant_args(const void *W, const float *W_out, int64_t N,
                       int64_t K);
int check_stream_args(const void *a, const void *b, uint64_t bytes);
// Extra shape rule of Q4_LAYOUT_TILED16: N % 16 == 0 and K % 256 == 0.
int check_tiled_shape(int64_t N, int64_t K);

// Launch plans of the two GEMM kernels (see q4_gemm_verify_plan); the shape
// has already been checked.
q4_plan plan_gemm_planar(int M, int64_t N, int64_t K);
q4_plan plan_gemm_tiled(int M, int64_t N, int64_t K);

// Bytes of one record of the tiled layout: 16 rows x 4 groups x 36 bytes.
constexpr int kTileRows = 16;
constexpr int kRecordGroups = 4;
constexpr int kRecordBytes = kTileRows * kRecordGroups * 36;

// Q4_OK when a HIP device is current and it is a gfx950; Q4_EDEVICE
// otherwise.  The answer is cached per device ordinal.
int check_device();

}  // namespace q4v
