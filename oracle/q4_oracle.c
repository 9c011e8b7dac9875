/*
 * q4_oracle.c -- plain, slow CPU oracle for the group-affine Q4 verify GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; it reads the packed weight buffer through its own reading of
 * the format, written out below.
 *
 * What it computes
 * ----------------
 * The packed weight format is the one the Splash engine article ("144 tok/s
 * needs 502 GB/s ...", section "The engine hard-codes the model") describes:
 * for every group of 64 inputs of one output row there are 32 bytes of 4-bit
 * codes, one bf16 scale and one bf16 bias, so 16 weights take 9 bytes
 * (q4PackedBytes = elements / 16 * 9, with a checked 64-bit multiply).  A
 * weight is w = scale * q + bias with q the unsigned code 0..15.
 *
 * The verify step multiplies that matrix W[N][K] (outputs by inputs, the
 * argument order of q4PackedBytes) by a block of M activation rows,
 * y[m][n] = sum_k x[m][k] * w[n][k]; the Splash article (section "Why Apple
 * silicon, and why not the M5") calls the eight verify rows an 8 x K x N GEMM,
 * and the qwen-spec page (Notes) describes the kernel that multiplies all rows
 * with one read of each weight tile.  The fast method reaches exactly this
 * plain product, so the oracle is the product written out:
 *
 *   1. dequantise one output row: w[k] = fp32(s * q + b)   (one rounding);
 *   2. y64[m][n] = sum over k ascending of (double)x[m][k] * (double)w[k],
 *      a64[m][n] = sum over k ascending of |same product|,
 *      y32[m][n] = (float)y64[m][n]   (round to nearest even).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - buffer layout is planar: [nibbles N*K/2 B][scales N*K/64 bf16]
 *     [biases N*K/64 bf16], each plane row-major by output row;
 *   - within a byte the low nibble is the even input k, the high nibble k+1;
 *   - q is unsigned (w = s*q + b, not s*(q - z));
 *   - y is overwritten, not accumulated into.
 *
 * Exactness: s has 8 significant bits and q at most 4, so s*q is exact in
 * fp32 and the only rounding in step 1 is the add.  In step 2 every product of
 * a bf16 and an fp32 value is exact in fp64 (8 + 24 <= 53 bits), so the sum's
 * error is at most (K-1) * 2^-53 * a64 -- negligible against any fp32 check.
 *
 * Threads: rows n are split into contiguous blocks, one per thread; every
 * output element is computed by one thread in ascending k order, so results do
 * not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define Q4O_GROUP 64

/* Status codes of this oracle (independent of the library's). */
#define Q4O_OK 0
#define Q4O_EINVAL (-1)
#define Q4O_EOVERFLOW (-3)
#define Q4O_ENOMEM (-6)

/* bf16 -> fp32: bf16 is the top half of an fp32 bit pattern, so this is
 * exact. */
static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Packed size of an N x K Q4 matrix: elements / 16 * 9 bytes, with every
 * multiply checked for 64-bit overflow (the q4PackedBytes listing of the
 * Splash article does the same with a checked multiply). */
int q4o_packed_bytes(int64_t N, int64_t K, uint64_t *out_bytes) {
    if (out_bytes == NULL) return Q4O_EINVAL;
    if (N < 1 || K < Q4O_GROUP || K % Q4O_GROUP != 0) return Q4O_EINVAL;
    uint64_t elements;
    if (__builtin_mul_overflow((uint64_t)N, (uint64_t)K, &elements))
        return Q4O_EOVERFLOW;
    uint64_t bytes;
    if (__builtin_mul_overflow(elements / 16u, (uint64_t)9u, &bytes))
        return Q4O_EOVERFLOW;
    *out_bytes = bytes;
    return Q4O_OK;
}

/* Where each plane of the planar layout starts (bytes from the buffer
 * start). */
static void plane_offsets(int64_t N, int64_t K, uint64_t *nib_off,
                          uint64_t *scale_off, uint64_t *bias_off) {
    uint64_t elements = (uint64_t)N * (uint64_t)K;
    *nib_off = 0;
    *scale_off = elements / 2;                     /* 4 bits per weight  */
    *bias_off = *scale_off + (elements / 64) * 2;  /* one bf16 per group */
}

/* Step 1 for one output row n: w[k] = s * q + b, rounded once to fp32. */
static void dequant_row(const uint8_t *W, int64_t N, int64_t K, int64_t n,
                        float *w) {
    uint64_t nib_off, scale_off, bias_off;
    plane_offsets(N, K, &nib_off, &scale_off, &bias_off);
    const uint8_t *nib = W + nib_off + (uint64_t)n * (uint64_t)(K / 2);
    const int64_t groups = K / Q4O_GROUP;
    for (int64_t g = 0; g < groups; ++g) {
        uint64_t idx = (uint64_t)n * (uint64_t)groups + (uint64_t)g;
        uint16_t s_bits, b_bits;
        memcpy(&s_bits, W + scale_off + 2 * idx, 2);
        memcpy(&b_bits, W + bias_off + 2 * idx, 2);
        const float s = bf16_bits_to_float(s_bits);
        const float b = bf16_bits_to_float(b_bits);
        for (int64_t k = g * Q4O_GROUP; k < (g + 1) * Q4O_GROUP; ++k) {
            const uint8_t byte = nib[k / 2];
            const unsigned q = (k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
            const float sq = s * (float)q; /* exact: 8 x 4 significant bits */
            w[k] = sq + b;                 /* the one rounding              */
        }
    }
}

int q4o_dequant(const uint8_t *W, int64_t N, int64_t K, float *out) {
    uint64_t bytes;
    int st = q4o_packed_bytes(N, K, &bytes);
    if (st != Q4O_OK) return st;
    if (W == NULL || out == NULL) return Q4O_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        dequant_row(W, N, K, n, out + (uint64_t)n * (uint64_t)K);
    return Q4O_OK;
}

typedef struct {
    const uint16_t *x;
    const uint8_t *W;
    int64_t M, N, K;
    int64_t n_begin, n_end;
    double *y64, *a64;
    float *y32;
    int status;
} gemm_job;

static void *gemm_rows(void *arg) {
    gemm_job *job = (gemm_job *)arg;
    const int64_t K = job->K, M = job->M, N = job->N;
    float *w = (float *)malloc((size_t)K * sizeof(float));
    if (w == NULL) {
        job->status = Q4O_ENOMEM;
        return NULL;
    }
    for (int64_t n = job->n_begin; n < job->n_end; ++n) {
        dequant_row(job->W, N, K, n, w);
        for (int64_t m = 0; m < M; ++m) {
            const uint16_t *xr = job->x + (uint64_t)m * (uint64_t)K;
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p =
                    (double)bf16_bits_to_float(xr[k]) * (double)w[k];
                acc += p;
                acc_abs += fabs(p);
            }
            const uint64_t o = (uint64_t)m * (uint64_t)N + (uint64_t)n;
            if (job->y64) job->y64[o] = acc;
            if (job->a64) job->a64[o] = acc_abs;
            if (job->y32) job->y32[o] = (float)acc;
        }
    }
    free(w);
    job->status = Q4O_OK;
    return NULL;
}

/* y[m][n] = sum_k x[m][k] * w[n][k] for x bf16 [M][K] (raw bits), W packed
 * [N][K].  Outputs are [M][N] row-major; any of them may be NULL.  threads <= 0
 * means one thread per online CPU.  Returns the number of threads used in
 * *threads_used when that pointer is not NULL. */
int q4o_gemm(const uint16_t *x, const uint8_t *W, int64_t M, int64_t N,
             int64_t K, double *y64, double *a64, float *y32, int threads,
             int *threads_used) {
    uint64_t bytes;
    int st = q4o_packed_bytes(N, K, &bytes);
    if (st != Q4O_OK) return st;
    if (M < 1 || x == NULL || W == NULL) return Q4O_EINVAL;
    if (threads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        threads = c > 0 ? (int)c : 1;
    }
    if ((int64_t)threads > N) threads = (int)N;
    gemm_job *jobs = (gemm_job *)calloc((size_t)threads, sizeof(gemm_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (jobs == NULL || tids == NULL) {
        free(jobs);
        free(tids);
        return Q4O_ENOMEM;
    }
    for (int t = 0; t < threads; ++t) {
        jobs[t].x = x;
        jobs[t].W = W;
        jobs[t].M = M;
        jobs[t].N = N;
        jobs[t].K = K;
        jobs[t].n_begin = N * t / threads;
        jobs[t].n_end = N * (t + 1) / threads;
        jobs[t].y64 = y64;
        jobs[t].a64 = a64;
        jobs[t].y32 = y32;
        jobs[t].status = Q4O_EINVAL;
    }
    int started = 0;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tids[t], NULL, gemm_rows, &jobs[t]) != 0) break;
        started = t;
    }
    gemm_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    /* Rows of threads that could not be started are done here, in order. */
    for (int t = started + 1; t < threads; ++t) gemm_rows(&jobs[t]);
    int status = Q4O_OK;
    for (int t = 0; t < threads; ++t)
        if (jobs[t].status != Q4O_OK) status = jobs[t].status;
    free(jobs);
    free(tids);
    if (threads_used) *threads_used = threads;
    return status;
}
