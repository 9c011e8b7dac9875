/*
 * q4verify.h -- C ABI of the skinny-M Q4 verify GEMM for AMD MI355X (gfx950).
 *
 * The operation.  A speculative-decoding verify step runs the target model
 * once over a block of M draft rows; every linear layer then multiplies a
 * 4-bit weight matrix by M activation rows, and the step is cheap only if each
 * weight byte is read from memory once for all rows (Splash engine article,
 * "144 tok/s needs 502 GB/s ...", section "Why Apple silicon, and why not the
 * M5": the eight verify rows turn decode into an 8 x K x N GEMM; qwen-spec
 * page, Notes and the figure beside them: a matmul that reads each weight tile
 * once costs 1.02x for 16 rows against 1 row; goinfer page "Faster, with the
 * same words", section "How it works": verify rows run in one pass).
 *
 * The weight format.  Splash engine article, section "The engine hard-codes
 * the model": every group of 64 inputs of one output row holds 32 bytes of
 * unsigned 4-bit codes q, one bf16 scale s and one bf16 bias b, and the weight
 * is w = s * q + b; 16 weights take 9 bytes (q4PackedBytes), with no
 * exceptions per tensor.  The pages do not fix the byte layout; this library
 * reads the planar layout described at q4_pack_layout.
 *
 * Conventions for every entry point:
 *   - Stateless and thread-safe; nothing is allocated, no stream is
 *     synchronised.  Device work is enqueued on `stream` (a hipStream_t passed
 *     as void*, NULL = the null stream) and runs asynchronously.
 *   - All data pointers are device memory owned by the caller; the library
 *     only borrows them for the duration of the enqueued work.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns an error code and enqueues nothing.  Faults inside
 *     enqueued work surface at the caller's next synchronisation.
 *   - Return value: Q4_OK (0) or a negative q4_status.
 */
#ifndef Q4VERIFY_H
#define Q4VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 2u
#define Q4_GROUP 64     /* inputs per scale/bias group                     */
#define Q4_MAX_ROWS 16  /* largest activation block M of q4_gemm_verify     */
#define Q4_MAX_ROWS_TILED 32 /* of the tiled calls: two MFMA row tiles    */
#define Q4_DOT_MAX_ROWS 4    /* of q4_gemm_verify_tiled_dot                */

typedef enum {
  Q4_OK = 0,
  Q4_EINVAL = -1,    /* a size, pointer or layout id is invalid            */
  Q4_EALIGN = -2,    /* a pointer is not aligned as the call requires      */
  Q4_EOVERFLOW = -3, /* a byte count does not fit 64 bits                  */
  Q4_EDEVICE = -4,   /* no HIP device, or the current one is not gfx950    */
  Q4_ELAUNCH = -5,   /* the HIP runtime refused the launch                 */
  Q4_ESCRATCH = -6   /* more scratch than q4_gemm_verify_tiled_noalloc has */
} q4_status;

/* Layout ids accepted by q4_pack_layout. */
#define Q4_LAYOUT_PLANAR 0u  /* planes of codes, scales, biases            */
#define Q4_LAYOUT_TILED16 1u /* records of 16 rows x 4 groups (q4_repack)   */

typedef struct {
  uint32_t abi_version; /* Q4_ABI_VERSION                                  */
  uint32_t layout_id;   /* Q4_LAYOUT_PLANAR                                 */
  int64_t N;            /* output rows                                     */
  int64_t K;            /* inputs per row, a multiple of Q4_GROUP           */
  int64_t group;        /* Q4_GROUP                                        */
  uint64_t total_bytes; /* N*K/16*9 exactly                                 */
  uint64_t code_off, code_bytes;   /* 4-bit codes, N*K/2 bytes              */
  uint64_t scale_off, scale_bytes; /* bf16 scales, N*K/64 values            */
  uint64_t bias_off, bias_bytes;   /* bf16 biases, N*K/64 values            */
  /* Q4_LAYOUT_TILED16 only (0 for the planar layout): */
  uint32_t tile_rows;     /* 16 output rows per tile                        */
  uint32_t record_groups; /* 4 groups (256 inputs) per record               */
  uint64_t record_bytes;  /* 2304 bytes per record                          */
} q4_layout;

/*
 * q4_pack_layout -- byte layout of a packed N x K weight matrix (host only).
 *
 * Follows q4PackedBytes (Splash engine article, section "The engine
 * hard-codes the model"): total = N*K/16*9 bytes, computed with overflow
 * checks.  Layout Q4_LAYOUT_PLANAR, a reading of the pages (they give sizes,
 * not positions):
 *   codes  at 0           : [N][K/2] bytes, row-major; byte n*K/2 + k/2
 *                           holds input k of row n in its low nibble when k
 *                           is even, in its high nibble when k is odd;
 *   scales at N*K/2       : [N][K/64] bf16, row-major (group g of row n at
 *                           index n*K/64 + g);
 *   biases at N*K/2+N*K/32: [N][K/64] bf16, same order.
 * In the planar layout the code/scale/bias offsets and sizes are filled in.
 *
 * Layout Q4_LAYOUT_TILED16 holds the same bytes reordered for the GPU (see
 * q4_repack); it needs N % 16 == 0, K % 256 == 0 and K <= 2^26 and has the same
 * total_bytes.  Output rows are cut into tiles of 16, a tile's K into records
 * of 4 groups; tile t's records follow one another (record r of tile t at
 * byte (t*K/256 + r) * 2304).  A record is
 *   [0, 1024)   groups 0 and 1:  16 bytes per lane l = j + 16*kb (j = row in
 *               tile, kb = 0..3): the 8 code bytes kb*8..kb*8+7 of group 0
 *               of row j, then the same 8 bytes of group 1;
 *   [1024,2048) groups 2 and 3, same arrangement;
 *   [2048,2304) 16 bytes per row j: scale, bias of group 0, scale, bias of
 *               group 1, ... group 3 (bf16 each).
 * Within each 32-bit little-endian code word (8 inputs i = 0..7 of a lane,
 * input i in nibble i of the planar word) the nibbles are reordered to
 * inputs 0, 2, 4, 6, 1, 3, 5, 7: even inputs in the low 16 bits, odd inputs
 * in the high 16 bits.
 * Arguments: N >= 1, K >= 64 with K % 64 == 0, a known layout_id, `out`
 * non-NULL (written only on success).
 * Errors: Q4_EINVAL (bad size, id or NULL), Q4_EOVERFLOW (size > 2^64-1).
 */
int q4_pack_layout(int64_t N, int64_t K, uint32_t layout_id, q4_layout *out);

/*
 * q4_gemm_verify -- y[m][n] = sum_k x[m][k] * (s[n][k/64] * q[n][k] +
 * b[n][k/64]) for 0 <= m < M, 0 <= n < N.
 *
 * The verify matmul of the pages (see the file comment): one pass over the
 * packed weights serves all M rows.
 *   x : device, bf16 [M][K] row-major, contiguous, 16-byte aligned.
 *   W : device, packed N x K matrix in Q4_LAYOUT_PLANAR (total_bytes of
 *       q4_pack_layout), 16-byte aligned.  Read only.
 *   y : device, fp32 [M][N] row-major, contiguous, 4-byte aligned; fully
 *       overwritten (no accumulation into prior contents).  Must not overlap
 *       x or W.
 *   M : 1..Q4_MAX_ROWS.  N : 1..2^31-1.  K : multiple of 64, 64..2^31-64.
 *   stream : hipStream_t or NULL.
 * Kernel (q4_gemm_verify_plan reports it): for K % 256 == 0 the K-slice
 * kernel (Q4_KERNEL_TILED_KSLICE with layout_id Q4_LAYOUT_PLANAR): each
 * wave keeps two 256-input records of the activations in registers and
 * streams those records of every 16-row tile as whole 128-byte row runs
 * through LDS; K beyond 24 records is taken in parts one after another by
 * the same workgroup (k_seq_parts), so no workspace is needed at any K.
 * Other K, K beyond 24 records with more than 4 tiles per workgroup
 * (N > 16384 on 256 CUs), and shapes whose 32-bit offsets would overflow run
 * Q4_KERNEL_PLANAR.
 * Accumulation is fp32; results stay within 2e-3 * sum_k |x*w| + 1e-5 of the
 * exact product.  The plan depends on (N, K) only, never on M, and rows are
 * summed in an order fixed by (N, K): a row's result does not depend on M or
 * on the other rows of the block, and repeated calls are bitwise equal.
 * Errors: Q4_EINVAL, Q4_EALIGN, Q4_EOVERFLOW, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_gemm_verify(const void *x, const void *W, float *y, int M, int64_t N,
                   int64_t K, void *stream);

/*
 * q4_repack -- one-time reorder of a planar packed matrix into
 * Q4_LAYOUT_TILED16, the layout q4_gemm_verify_tiled streams.  A pure
 * permutation of 4-bit codes and bf16 values: the output holds exactly the
 * input's codes, scales and biases, total_bytes of them.  The pages' engine loads weights once and keeps them resident (Splash
 * engine article, section "Why Apple silicon, and why not the M5"); this is
 * the one-time step before that residency, timed apart from the GEMM.
 *   W_planar : device, Q4_LAYOUT_PLANAR, 16-byte aligned, read only.
 *   W_tiled  : device, total_bytes, 16-byte aligned, overwritten, must not
 *              overlap W_planar.
 *   N % 16 == 0, K % 256 == 0, K <= 2^26 (else Q4_EINVAL).
 * Errors: Q4_EINVAL, Q4_EALIGN, Q4_EOVERFLOW, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_repack(const void *W_planar, void *W_tiled, int64_t N, int64_t K,
              void *stream);

/*
 * q4_gemm_verify_tiled -- the product of q4_gemm_verify for weights in
 * Q4_LAYOUT_TILED16 (same x, y, M and results within the same bound).  Each
 * wave streams whole 2304-byte records with 16-byte loads, so every weight
 * byte is fetched once in full cache lines.  Kernels (q4_gemm_verify_plan
 * reports which): M <= 16 runs the K-slice kernel (Q4_KERNEL_TILED_KSLICE;
 * K beyond 24 records in parts taken one after another, no workspace)
 * whenever a workgroup's tiles fit its running sums (at most 16 tiles per
 * workgroup once K is cut in parts), otherwise Q4_KERNEL_TILED_RESIDENT
 * (K <= 5120, activations in LDS) or Q4_KERNEL_TILED_STREAM.  For M <= 16
 * the plan depends on (N, K) only: within M = 1..16 a row's bits do not
 * depend on M, and for the model's shapes (K in {5120, 6144, 17408}) they
 * equal q4_gemm_verify's on the same weights.  M = 17..32 (two MFMA row
 * tiles multiplying the same unpacked weights, the Splash engine's
 * multi-lane shapes) runs another kernel, whose rows agree with the M <= 16
 * rows within the bound, not bit for bit; without a workspace it needs
 * K <= 2560 (larger K at M > 16: q4_gemm_verify_tiled_ws).
 *   x, y, M, stream: as q4_gemm_verify.
 *   W_tiled : device, Q4_LAYOUT_TILED16 of an N x K matrix, 16-byte aligned.
 *   N % 16 == 0, K % 256 == 0, K <= 2^26 (else Q4_EINVAL).
 * Errors: Q4_EINVAL, Q4_EALIGN, Q4_EOVERFLOW, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_gemm_verify_tiled(const void *x, const void *W_tiled, float *y, int M,
                         int64_t N, int64_t K, void *stream);

/*
 * q4_gemm_verify_tiled_dot -- q4_gemm_verify_tiled for M <= 4 on the vector
 * ALU: the same K-slice kernel and weight stream, with the row dot products
 * on v_dot2_f32_bf16 instead of MFMA tiles padded to 16 rows.  The Splash
 * engine article (section "Why Apple silicon, and why not the M5") makes
 * the case for matrix hardware at 8 verify rows; this entry point measures
 * the other side at 1, 2 and 4 rows.  Results within the same bound as
 * q4_gemm_verify (a different summation order: not bit-equal to the MFMA
 * path); the plan depends on (N, K) only.
 *   x, W_tiled, y, N, K, stream: as q4_gemm_verify_tiled.
 *   M : 1..Q4_DOT_MAX_ROWS.  K <= 6144 (one part of K).
 * Errors: as q4_gemm_verify_tiled; Q4_EINVAL for M > 4 or K > 6144.
 */
int q4_gemm_verify_tiled_dot(const void *x, const void *W_tiled, float *y,
                             int M, int64_t N, int64_t K, void *stream);

/*
 * q4_dequant -- W_out[n][k] = fp32(s * q + b), rounded once (test hook that
 * exposes the kernels' reading of the format, same passage as above).
 *   W     : device, packed N x K matrix in Q4_LAYOUT_PLANAR, 16-byte aligned.
 *   W_out : device, fp32 [N][K] row-major, 16-byte aligned, overwritten.
 * Errors: as q4_gemm_verify.
 */
int q4_dequant(const void *W, float *W_out, int64_t N, int64_t K,
               void *stream);

/*
 * q4_stream_read -- measurement probe: read `bytes` bytes at `buf` once with
 * 16-byte non-temporal loads, one contiguous share per CU, and write nothing
 * unless a checksum hits a sentinel (then one uint32 to *sink).  Gives the streaming read rate the GEMM is measured
 * against besides the HBM peak (the prediction-first page, section "What a
 * Measurement Record Contains", keeps both the vendor figure and a measured
 * streaming rate as denominators).
 *   buf : device, 16-byte aligned; bytes a positive multiple of 16.
 *   sink: device, one uint32.
 */
int q4_stream_read(const void *buf, uint64_t bytes, uint32_t *sink,
                   void *stream);

/*
 * q4_stream_copy -- measurement probe: dst[i] = src[i] for `bytes` bytes with
 * 16-byte loads and stores (the reference kernel of known traffic that the
 * hardware byte counters are calibrated against).
 *   src, dst : device, 16-byte aligned, not overlapping; bytes a positive
 *              multiple of 16.
 */
int q4_stream_copy(const void *src, void *dst, uint64_t bytes, void *stream);

/* Launch plan of a verify GEMM for one shape (host only, pure). */
typedef struct {
  uint32_t grid;         /* workgroups launched                            */
  uint32_t block;        /* threads per workgroup (64 per wave)            */
  uint32_t row_tiles;    /* 16-row output tiles per workgroup              */
  uint32_t tiles_per_wave; /* 16-row tiles one wave multiplies at once     */
  uint32_t k_splits;     /* waves per tile set, each taking a contiguous
                            range of K; partial sums are added in split
                            order inside the workgroup                     */
  uint32_t lookahead;    /* groups whose loads are issued ahead of use      */
  uint32_t kernel;       /* Q4_KERNEL_* below                               */
  uint32_t lds_bytes;    /* LDS per workgroup                               */
  uint32_t k_parts;      /* parts of K taken by separate workgroups; > 1
                            only on the workspace path                      */
  uint32_t m_tiles;      /* 16-row MFMA tiles of the activation block (1 for
                            M <= 16, 2 for M <= 32)                         */
  uint64_t workspace_bytes; /* device workspace the call needs (0: none)    */
  uint32_t k_seq_parts;  /* parts of K one workgroup takes one after another,
                            its tiles' running sums kept on chip (1: K in
                            one part)                                       */
  uint32_t layout_id;    /* Q4_LAYOUT_* the plan reads                      */
} q4_plan;

#define Q4_KERNEL_PLANAR 0u          /* q4_gemm_verify                       */
#define Q4_KERNEL_TILED_STREAM 1u    /* tiled; activations loaded per record */
#define Q4_KERNEL_TILED_RESIDENT 2u  /* tiled; activations resident in LDS;
                                        grid = one workgroup per CU (at most
                                        N/16), each owning whole 16-row tiles
                                        split evenly across its waves        */
#define Q4_KERNEL_TILED_KSLICE 3u    /* M <= 16, either layout (layout_id);
                                        grid = about one workgroup per CU
                                        (times k_parts) over whole tiles;
                                        wave w takes records 2w and 2w+1 of
                                        every tile of its part of K and keeps
                                        that slice of the activations in
                                        registers; k_seq_parts parts of K are
                                        taken one after another;
                                        block = 64 * ceil(records/2) of a
                                        part (at most 12 waves)             */

/*
 * q4_gemm_verify_plan -- the plan q4_gemm_verify (layout_id
 * Q4_LAYOUT_PLANAR) or q4_gemm_verify_tiled (Q4_LAYOUT_TILED16) launches for
 * (M, N, K).  Same argument rules as those calls; `out` non-NULL.
 * Errors: Q4_EINVAL, Q4_EOVERFLOW.
 */
int q4_gemm_verify_plan(int M, int64_t N, int64_t K, uint32_t layout_id,
                        q4_plan *out);

/*
 * q4_gemm_verify_tiled_ws -- q4_gemm_verify_tiled with a caller-owned device
 * workspace, which lets workgroups split K for K > 5120 (the output and down
 * projections, whose N = 5120 gives only 320 tiles and whose 16 activation
 * rows exceed one CU's LDS): part 0 writes y, parts 1..P-1 write their
 * partial products into the workspace, and a second kernel adds them to y in
 * part order, so results are deterministic.  Up to 16 rows the split (P = 4
 * or more, a power of two, at most 24 records per part) depends on (N, K)
 * only, so within M = 1..16 a row's bits do not depend on M; M = 17..32
 * splits differently and agrees with those rows within the bound.  For
 * K <= 6144 it runs exactly what q4_gemm_verify_tiled runs.
 *   x, W_tiled, y, M, N, K, stream: as q4_gemm_verify_tiled, with M up to
 *               Q4_MAX_ROWS_TILED for any K.
 *   workspace : device, 16-byte aligned, at least workspace_bytes as
 *               reported by q4_gemm_verify_tiled_ws_plan for (M, N, K); may
 *               be NULL when that is 0.  Overwritten; must not overlap x, W
 *               or y; two calls in flight at once need two workspaces.
 *   workspace_bytes : its size.
 * Errors: as q4_gemm_verify_tiled; Q4_EINVAL if the workspace is too small.
 */
int q4_gemm_verify_tiled_ws(const void *x, const void *W_tiled, float *y,
                            int M, int64_t N, int64_t K, void *workspace,
                            uint64_t workspace_bytes, void *stream);

/*
 * q4_gemm_verify_tiled_noalloc -- q4_gemm_verify_tiled_ws for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the K-split partial products go
 * to a scratch array the library holds in device memory instead of a
 * caller workspace.  Same kernels, plan and results (bit for bit) as
 * q4_gemm_verify_tiled_ws.
 *   x, W_tiled, y, M, N, K, stream: as q4_gemm_verify_tiled_ws.
 * The scratch is Q4_NOALLOC_SCRATCH_BYTES per device, a static array of the
 * library's code object that each GPU it runs on holds until the process
 * ends; nothing is allocated or freed by the call.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (two streams, or
 * two host threads) race, and must be ordered by the caller.  Nothing in the
 * array needs to start at zero (each part writes its whole slice before the
 * reduction reads it), and a later call overwrites what an earlier one left.
 * Shapes whose plan needs more workspace than the array holds (see
 * q4_gemm_verify_tiled_ws_plan) return Q4_ESCRATCH before anything is
 * enqueued.  Every projection of the 27B model fits at every M <= 32 (the
 * largest, 5120 x 17408 at M = 32, needs 4.4 MiB) except the 248320-row LM
 * head at M > 16 (16-30 MiB); at M <= 16 and N <= 5120 every K <= 98304
 * fits.
 * Errors: as q4_gemm_verify_tiled_ws; Q4_ESCRATCH as above.
 */
#define Q4_NOALLOC_SCRATCH_BYTES (8u << 20)
int q4_gemm_verify_tiled_noalloc(const void *x, const void *W_tiled, float *y,
                                 int M, int64_t N, int64_t K, void *stream);

/*
 * q4_gemm_verify_tiled_ws_plan -- the plan q4_gemm_verify_tiled_ws launches
 * for (M, N, K), including its workspace_bytes (for the current device's CU
 * count).  Errors: Q4_EINVAL, Q4_EOVERFLOW.
 */
int q4_gemm_verify_tiled_ws_plan(int M, int64_t N, int64_t K, q4_plan *out);

/* ------------------------------------------------------------------------
 * Verify sampling epilogue: the step after the LM head in a verify pass
 * (Splash engine article, section "Exact, up to top-32"; qwen-spec page, the
 * fused sampling kernel and the paragraph on sampling).  For each of the M
 * verify rows of logits:
 *   1. candidates: the top_k largest logits, larger first, equal logits by
 *      smaller token index;
 *   2. target probabilities p over them: softmax at `temperature`, cut to
 *      the shortest prefix whose mass reaches top_p, renormalised (0 for
 *      tokens outside it); temperature 0 is greedy (p = 1 on the argmax);
 *   3. the drafted token d is accepted when u * q(d) < p(d), q(d) being the
 *      draft's probability of d (0 if d is not among the row's draft
 *      candidates);
 *   4. otherwise the emitted token is drawn from max(p - q, 0), normalised:
 *      the first candidate (in candidate order, skipping zero residuals)
 *      whose cumulative residual exceeds v * R, R the residual mass; with no
 *      residual mass the same rule is applied to p.
 * Arithmetic is fp32; random numbers are inputs.
 * ------------------------------------------------------------------------ */
#define Q4_SAMPLE_MAX_TOPK 32
#define Q4_SAMPLE_MAX_DRAFT 16
#define Q4_SAMPLE_MAX_ROWS 1024
/* Longest row (vocabulary) q4_verify_sample takes: 512 slices of 16384. */
#define Q4_SAMPLE_MAX_VOCAB 8388608

typedef struct {
  float temperature; /* >= 0, finite; 0 = greedy                          */
  float top_p;       /* (0, 1]                                              */
  int32_t top_k;     /* 1 .. Q4_SAMPLE_MAX_TOPK, at most V                 */
  int32_t draft_k;   /* draft candidates per row, 0 .. Q4_SAMPLE_MAX_DRAFT */
} q4_sample_params;

/* Device workspace bytes q4_verify_sample needs for (M, V).
 * Errors: Q4_EINVAL (M outside 1..Q4_SAMPLE_MAX_ROWS, V outside
 * 1..Q4_SAMPLE_MAX_VOCAB). */
int q4_verify_sample_workspace(int M, int64_t V, uint64_t *bytes);

/*
 * q4_verify_sample -- steps 1-4 above for M rows.  Device pointers (caller
 * owned, row-major):
 *   logits [M][V] fp32 (4-byte aligned; must not hold NaN);
 *   draft_tok [M] int32; draft_idx [M][draft_k] int32 and draft_q
 *   [M][draft_k] fp32 (may be NULL when draft_k == 0); u, v [M] fp32 in
 *   [0, 1);
 *   outputs top_idx [M][top_k] int32, top_val [M][top_k] fp32 (the
 *   candidates' logits; -0 reported as +0, the two being equal and tied),
 *   top_prob [M][top_k] fp32 (p), greedy [M] int32 (the
 *   argmax), accept [M] int32 (0/1), token [M] int32 (the emitted token);
 *   workspace of at least q4_verify_sample_workspace bytes, 8-byte aligned.
 * prm is a host pointer, read before the call returns.  Two kernels are
 * enqueued on `stream`.
 * Errors: Q4_EINVAL (sizes, parameters, NULL pointers, small workspace),
 * Q4_EALIGN, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_verify_sample(const float *logits, int M, int64_t V,
                     const q4_sample_params *prm, const int32_t *draft_tok,
                     const int32_t *draft_idx, const float *draft_q,
                     const float *u, const float *v, int32_t *top_idx,
                     float *top_val, float *top_prob, int32_t *greedy,
                     int32_t *accept, int32_t *token, void *workspace,
                     uint64_t workspace_bytes, void *stream);

/*
 * q4_gemm_verify_sample -- the LM head of a verify step with the sampling
 * epilogue fused in: the logits x W^T of the M verify rows are never
 * written to memory.  The product runs as in q4_gemm_verify_tiled, and each
 * workgroup keeps the logits of its run of 16-row tiles on chip and passes
 * on only the best 32 candidates of each verify row among its columns; a
 * second kernel merges those lists per row and applies steps 2-4 above
 * (Splash engine article, section "Exact, up to top-32", and "The decode
 * step is one command buffer": sampling and the accept test follow the LM
 * head in the same step; qwen-spec page, Notes: the fused sampling kernel).
 * The candidates, probabilities and decisions are those of
 * q4_gemm_verify_tiled followed by q4_verify_sample on the same inputs, bit
 * for bit (the logits are the same fp32 values).
 *   x, W_tiled, M (1..Q4_MAX_ROWS), N (the vocabulary, V), K: as
 *     q4_gemm_verify_tiled; K <= 6144 and N <= 1024 * (compute units), the
 *     compute units counted up to 512 (the merge takes at most 512 lists).
 *   prm, draft_tok .. token: as q4_verify_sample with V = N.
 *   workspace: q4_gemm_verify_sample_workspace bytes, 8-byte aligned.
 * Two kernels on `stream`; calls sharing a workspace race.
 * Errors: Q4_EINVAL (sizes, parameters, NULL pointers, small workspace, a
 * shape outside the rule above), Q4_EALIGN, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_gemm_verify_sample(const void *x, const void *W_tiled, int M,
                          int64_t N, int64_t K, const q4_sample_params *prm,
                          const int32_t *draft_tok, const int32_t *draft_idx,
                          const float *draft_q, const float *u, const float *v,
                          int32_t *top_idx, float *top_val, float *top_prob,
                          int32_t *greedy, int32_t *accept, int32_t *token,
                          void *workspace, uint64_t workspace_bytes,
                          void *stream);

/* Workspace bytes of q4_gemm_verify_sample for (M, N, K) on the current
 * device: M * (workgroups) * 32 keys of 8 bytes.  Errors: Q4_EINVAL. */
int q4_gemm_verify_sample_workspace(int M, int64_t N, int64_t K,
                                    uint64_t *bytes);

/* ------------------------------------------------------------------------
 * Gated DeltaNet state commit.
 *
 * A recurrent layer carries one dv x dk fp32 state per value head, read and
 * written back every step (Splash engine article, section on what one step
 * reads: 48 layers x 48 value heads x 128 x 128).  After the check, the
 * accepted tree nodes are written into the state in path order (qwen-spec
 * page, the hybrid-model paragraph), each by the gated delta rule
 *     S <- alpha S (I - beta k k^T) + beta v k^T,
 * k being the node's key for key head h / (H / Hk), v its value for head h,
 * alpha and beta its gate and writing strength for head h.  Arithmetic is
 * fp32; the gate is carried as one running factor per head.
 * ------------------------------------------------------------------------ */
#define Q4_GDN_DK 128
#define Q4_GDN_MAX_NODES 32

/* Dynamic LDS bytes of the commit kernel for M tree nodes (informational).
 * Errors: Q4_EINVAL (M outside 1..Q4_GDN_MAX_NODES, NULL). */
int q4_gdn_commit_lds_bytes(int M, int *bytes);

/*
 * q4_gdn_commit -- apply the accepted nodes to every layer's state, in
 * place.  Device pointers (caller owned, row-major, fp32 unless stated):
 *   S [L][H][dv][dk] (16-byte aligned): row r of a head's state is value
 *     index r, column c key index c; read and overwritten;
 *   k [L][M][Hk][dk] (16-byte aligned), v [L][M][H][dv] (16-byte aligned),
 *   alpha, beta [L][M][H]: every tree node's key, value, gate, strength;
 *   path [M] int32: the accepted nodes, root first (entries past the count
 *     are not read); n_accept: one int32, the count, 0 .. M;
 *   status: NULL or one int32 that receives Q4_OK, or Q4_EINVAL when the
 *     count or a read path entry is out of range -- then S is not written.
 * The count and the path are read on the device: the call may be enqueued
 * right after the step that decides them.  A count of 0 leaves S unread.
 * Sizes: dk == Q4_GDN_DK, dv a multiple of 64, Hk divides H,
 * 1 <= M <= Q4_GDN_MAX_NODES, L * H * dv / 64 < 2^31.  One kernel on
 * `stream`; calls that overlap on the same S race.
 * Errors: Q4_EINVAL, Q4_EALIGN, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_gdn_commit(float *S, int L, int H, int Hk, int dv, int dk, int M,
                  const float *k, const float *v, const float *alpha,
                  const float *beta, const int32_t *path,
                  const int32_t *n_accept, int32_t *status, void *stream);

/*
 * q4_gdn_tree_out -- every tree node's output of one recurrent layer from
 * the shared state (qwen-spec page, the hybrid-model paragraph): node i
 * reads the state after the context plus the updates, by the rule above, of
 * the nodes on its own path root .. i, i included, and its output is
 *     o_i = S_i q_i.
 * Device pointers (caller owned, row-major, fp32 unless stated):
 *   S [H][dv][dk] (16-byte aligned): the layer's state, read only;
 *   q, k [M][Hk][dk] (16-byte aligned): every node's query and key;
 *   v [M][H][dv], alpha, beta [M][H]: value, gate, strength;
 *   parent [M] int32: node i's parent, -1 for a child of the context's last
 *     token; parents precede children (parent[i] < i);
 *   out [M][H][dv] (16-byte aligned): written;
 *   status: NULL or one int32 that receives Q4_OK, or Q4_EINVAL when a
 *     parent entry is out of range -- then out is not written.
 * The tree is read on the device, so the call may follow the step that
 * builds it on the stream.  Sizes: dk == Q4_GDN_DK, dv a multiple of 32, Hk
 * divides H, 1 <= M <= Q4_GDN_MAX_NODES.  Arithmetic is fp32; the updates
 * along a path are applied through their key and query products (the rows
 * of S evolve independently), not by rewriting S.  One kernel on `stream`.
 * Errors: Q4_EINVAL, Q4_EALIGN, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_gdn_tree_out(const float *S, int H, int Hk, int dv, int dk, int M,
                    const float *q, const float *k, const float *v,
                    const float *alpha, const float *beta,
                    const int32_t *parent, float *out, int32_t *status,
                    void *stream);

/* ------------------------------------------------------------------------
 * Tree-verify attention over the paged int8 KV cache.
 *
 * One attention layer of the verify pass.  Every tree node attends to the
 * context and to its own ancestors, reading the cache in place (qwen-spec
 * page, Notes and the hybrid-model paragraph).  The layer has Hq query heads
 * over Hkv KV heads of dimension 256.  A page holds 32 tokens in int8 with
 * an fp32 scale per token per head (Splash engine article, the model listing
 * and the paged KV pool).
 *
 * The tree's own keys and values sit in the cache right after the context:
 * node j at logical position ctx_len + j.  Node i sees positions
 * p < ctx_len, and tree position ctx_len + j when bit j of anc[i] is set
 * (node j is i or one of its ancestors).  Query head h reads KV head
 * h / (Hq / Hkv).  The output is softmax(scale * q k^T) v over the visible
 * positions, with k = k8 * k_scale and v = v8 * v_scale.
 * Arithmetic: scores as bf16 products on MFMA (the int8 keys are exact in
 * bf16), fp32 accumulation; each probability times its value scale, divided
 * by a power of two at or above every value scale seen so far, enters the
 * value product rounded to fp16 (11 significant bits; the int8 values are
 * exact in fp16).
 * ------------------------------------------------------------------------ */
#define Q4_ATTN_HEAD_DIM 256
#define Q4_ATTN_PAGE 32
#define Q4_ATTN_MAX_NODES 16

/* The split of the context a call would use, and the workspace it needs.
 * splits = 0 picks a split for the current device (runs of about 8 pages,
 * at least 16 runs and at most one per CU for each KV head), > 0 asks for
 * that many runs of pages (at most the number of pages).  The shape rules are those of
 * q4_tree_attn.  Errors: Q4_EINVAL. */
int q4_tree_attn_plan(int M, int Hq, int Hkv, int D, int64_t ctx_len,
                      int splits, int *splits_used, uint64_t *workspace_bytes);

/*
 * q4_tree_attn -- out[i][h][:] for every tree node i < M and query head h.
 * Device pointers (caller owned, row-major):
 *   q [M][Hq][D] bf16, 16-byte aligned;
 *   k_pages [pool_pages][Hkv][32][D] int8 (keys, token-major) and
 *   v_pages [pool_pages][Hkv][D][32] int8 (values, stored transposed), both
 *     16-byte aligned;
 *   k_scale, v_scale [pool_pages][Hkv][32] fp32, 16-byte aligned;
 *   page_table [ceil((ctx_len + M) / 32)] int32: logical page -> physical
 *     page; anc [M] uint32 ancestor-or-self sets;
 *   out [M][Hq][D] fp32, 16-byte aligned, overwritten;
 *   workspace: q4_tree_attn_plan's bytes (none when the plan uses one run),
 *     16-byte aligned;
 *   status: NULL, or one int32 that receives Q4_EINVAL when a page id is
 *     outside the pool (it is left as it was otherwise; such a page reads as
 *     zeros).
 * Sizes: D == Q4_ATTN_HEAD_DIM, 1 <= M <= Q4_ATTN_MAX_NODES, Hq / Hkv one of
 * 2, 4, 6, 8; 0 <= ctx_len < 2^31 - 64; scale > 0 and finite.  One or two
 * kernels on `stream`; calls sharing a workspace race.
 * Errors: Q4_EINVAL, Q4_EALIGN, Q4_EDEVICE, Q4_ELAUNCH.
 */
int q4_tree_attn(const void *q, int M, int Hq, int Hkv, int D,
                 const int8_t *k_pages, const int8_t *v_pages,
                 const float *k_scale, const float *v_scale,
                 const int32_t *page_table, int pool_pages, int64_t ctx_len,
                 const uint32_t *anc, float scale, float *out, int splits,
                 void *workspace, uint64_t workspace_bytes, int32_t *status,
                 void *stream);

/* Human-readable name of a q4_status value (static string, never NULL). */
const char *q4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* Q4VERIFY_H */
