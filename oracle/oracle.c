/*
 * oracle.c -- plain, slow, scalar CPU reference for the 1-bit (Q1_0) and
 * ternary (Q2_0) quantized matrix-vector product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the CPU leg
 * of the benchmark load it.  It shares no code, header, table or constant
 * with the HIP path.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared oracle.c -lm -lpthread
 * (no -ffast-math, no -mfma: every float operation below is one IEEE
 * binary32 operation rounded to nearest-even, and fmaf() is the C library's
 * correctly rounded fused multiply-add).
 *
 * Sources (the bankML documentation pages):
 *   [GPU]  bankML "gpu/ -- the video-card component", section
 *          "kernels.rs -- the Q1_0 kernels" (the dot-product order) and
 *          section "How it is verified" (random weights with -128 quants).
 *   [PAR]  bankML "par.rs -- the persistent thread pool and row scheduler",
 *          sections "Summary" and "Technical usage" (rows are independent;
 *          16-row chunks handed out from an atomic counter).
 *   [VK]   vkML "Shaders and the GLSL layer", section "f16 is storage, never
 *          arithmetic" (an f16 load is an exact widening) and section "Why
 *          f32->f16 narrowing is done in software" (narrowing rounds to
 *          nearest, ties to even).
 *
 * Readings taken where the pages are silent:
 *   R1  Q1_0 block = f16 scale (little-endian) then 16 payload bytes; weight k
 *       of the block is bit (k & 7) of byte (k >> 3); bit 1 -> +1, 0 -> -1.
 *   R2  Q2_0 block = f16 scale then 16 payload bytes of 2-bit codes; weight k
 *       is bits 2(k&3)..2(k&3)+1 of byte (k >> 2); code c means weight c - 1.
 *   R3  lane L of a 32-weight sub-block sums weights 4L .. 4L+3.
 *   R4  activation quantizer: per block of qa values, d = amax / 127 (f32),
 *       q = round-half-away-from-zero(x / d), clamped to [-127, 127]; d == 0
 *       gives q == 0.
 *   R5  the accumulators start at +0; the activation scale of sub-block j is
 *       d[(first element of j) / qa]; Q2_0 follows the same chain over its
 *       two sub-blocks.
 *   R6  the f16-scale flavour of the quantizer (the pages' q8_0 activation
 *       carries f16-valued scales): d = f16(amax / 127), narrowed to nearest
 *       with ties to even, and q = round-half-away(x / d) with that d,
 *       clamped to [-127, 127] (the clamp can bind when d lands in the f16
 *       subnormal range); d == 0 gives q == 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_Q1_0 1
#define ORACLE_Q2_0 2
#define ORACLE_BLOCK_BYTES 18
#define ORACLE_CHUNK_ROWS 16 /* [PAR] "Technical usage": rows claimed 16 at a time */

/* ---------------------------------------------------------------- f16 -> f32
 * [VK] "f16 is storage, never arithmetic": reading an f16 value is an exact
 * widening.  Written out from the binary16 definition: sign, 5-bit exponent
 * with bias 15, 10-bit fraction; exponent 0 encodes subnormals m * 2^-24. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* ---------------------------------------------------------------- f32 -> f16
 * [VK] "Why f32->f16 narrowing is done in software": round to nearest, ties
 * to even.  Written out from the binary16 definition: the value is scaled by
 * a power of two (exact) so that the kept bits form an integer part, which
 * rintf rounds in the default mode (nearest, ties to even).  Normal results
 * keep 11 significant bits (exponent -14 .. 15); below 2^-14 the grid is
 * m * 2^-24 (subnormals; m = 1024 is the smallest normal, same bits);
 * beyond 65504 the value rounds to infinity from 65520 on. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    float a = fabsf(f);
    if (isnan(f))
        return sign | 0x7E00;
    if (a >= 65520.0f)
        return sign | 0x7C00;
    if (a < ldexpf(1.0f, -14))
        return sign | (uint16_t)rintf(ldexpf(a, 24));
    int e;
    frexpf(a, &e); /* a = m * 2^e, m in [0.5, 1): the leading bit has weight 2^(e-1) */
    float m = rintf(ldexpf(a, 11 - e)); /* 11 significant bits: [1024, 2048] */
    int ex = e - 1;
    if (m == 2048.0f) {
        m = 1024.0f;
        ++ex;
    }
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)m - 1024));
}

/* ------------------------------------------------------- activation quantizer
 * Reading R4 (the pages name a q8_0 activation with one scale per block, see
 * [GPU] "kernels.rs": activation scales and int8 quants).  Returns the number
 * of values the clamp had to change (0 for finite input). */
static int64_t quantize(const float *x, int64_t n, int32_t qa, int f16_scale, int8_t *q, float *d)
{
    int64_t clamped = 0;
    for (int64_t b = 0; b * qa < n; ++b) {
        const float *xb = x + b * qa;
        float amax = 0.0f;
        for (int32_t i = 0; i < qa; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        float db = amax / 127.0f;
        if (f16_scale)
            db = oracle_f16_to_f32(oracle_f32_to_f16(db)); /* reading R6 */
        d[b] = db;
        for (int32_t i = 0; i < qa; ++i) {
            int v = 0;
            if (db != 0.0f) {
                float r = roundf(xb[i] / db); /* C roundf: halves away from zero */
                if (r > 127.0f) { r = 127.0f; ++clamped; }
                if (r < -127.0f) { r = -127.0f; ++clamped; }
                v = (int)r;
            }
            q[b * qa + i] = (int8_t)v;
        }
    }
    return clamped;
}

int64_t oracle_quantize_q8(const float *x, int64_t n, int32_t qa, int8_t *q, float *d)
{
    return quantize(x, n, qa, 0, q, d);
}

/* Reading R6: the same with f16-valued scales. */
int64_t oracle_quantize_q8_f16(const float *x, int64_t n, int32_t qa, int8_t *q, float *d)
{
    return quantize(x, n, qa, 1, q, d);
}

/* -------------------------------------------------------------- one Q1_0 row
 * [GPU] "kernels.rs": per 128-weight block, four 32-weight sub-blocks; in each
 * sub-block eight lanes of exact integer sums, where negating an int8 -128
 * gives -128 again; ab = d1*s on the first sub-block and ab = fma(d1, s, ab)
 * on the others; then acc = fma(d0, ab, acc) per lane; at the end the eight
 * lanes are summed as ((a0+a4) + (a2+a6)) + ((a1+a5) + (a3+a7)). */
static int32_t q1_0_product(int bit, int8_t qv)
{
    if (bit)
        return qv;
    return qv == -128 ? -128 : -(int32_t)qv; /* int8 negation wraps -128 */
}

float oracle_q1_0_row(const uint8_t *blocks, int64_t nb, const int8_t *q, const float *d, int32_t qa)
{
    float acc[8];
    for (int L = 0; L < 8; ++L)
        acc[L] = 0.0f;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *blk = blocks + b * ORACLE_BLOCK_BYTES;
        float d0 = oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
        const uint8_t *qs = blk + 2;
        float ab[8];
        for (int j = 0; j < 4; ++j) {
            int64_t e0 = 128 * b + 32 * j; /* first element of sub-block j */
            float d1 = d[e0 / qa];
            for (int L = 0; L < 8; ++L) {
                int32_t s = 0;
                for (int i = 0; i < 4; ++i) {
                    int k = 32 * j + 4 * L + i; /* weight index inside the block */
                    int bit = (qs[k >> 3] >> (k & 7)) & 1;
                    s += q1_0_product(bit, q[e0 + 4 * L + i]);
                }
                if (j == 0)
                    ab[L] = d1 * (float)s;
                else
                    ab[L] = fmaf(d1, (float)s, ab[L]);
            }
        }
        for (int L = 0; L < 8; ++L)
            acc[L] = fmaf(d0, ab[L], acc[L]);
    }
    return ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));
}

/* -------------------------------------------------------------- one Q2_0 row
 * Ternary weights (the pages give only their size and that no GPU kernel for
 * them existed yet); readings R2 and R5: the Q1_0 chain applied to the two
 * 32-weight sub-blocks of a 64-weight block, with exact products (c-1)*q. */
float oracle_q2_0_row(const uint8_t *blocks, int64_t nb, const int8_t *q, const float *d, int32_t qa)
{
    float acc[8];
    for (int L = 0; L < 8; ++L)
        acc[L] = 0.0f;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *blk = blocks + b * ORACLE_BLOCK_BYTES;
        float d0 = oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
        const uint8_t *qs = blk + 2;
        float ab[8];
        for (int j = 0; j < 2; ++j) {
            int64_t e0 = 64 * b + 32 * j;
            float d1 = d[e0 / qa];
            for (int L = 0; L < 8; ++L) {
                int32_t s = 0;
                for (int i = 0; i < 4; ++i) {
                    int k = 32 * j + 4 * L + i;
                    int code = (qs[k >> 2] >> (2 * (k & 3))) & 3;
                    s += (code - 1) * (int32_t)q[e0 + 4 * L + i];
                }
                if (j == 0)
                    ab[L] = d1 * (float)s;
                else
                    ab[L] = fmaf(d1, (float)s, ab[L]);
            }
        }
        for (int L = 0; L < 8; ++L)
            acc[L] = fmaf(d0, ab[L], acc[L]);
    }
    return ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));
}

/* ----------------------------------------------------------- row scheduler
 * [PAR] "Summary" / "Technical usage": each row is computed by the same
 * single-thread routine, so which thread takes a row changes no bit; rows are
 * claimed in chunks of 16 from a shared atomic counter, and the calling thread
 * works too.  This driver exists only to make the full-size checks finish. */
typedef struct {
    int fmt;
    const uint8_t *canon;
    int64_t rows, nb;
    const int8_t *q;
    const float *d;
    int32_t qa;
    int32_t ncols;
    int64_t ld_q, ld_d;
    float *y;
    int *cover; /* optional: per-row write counter (coverage test) */
    atomic_long next;
} oracle_job;

static void *oracle_worker(void *arg)
{
    oracle_job *job = (oracle_job *)arg;
    for (;;) {
        int64_t r0 = atomic_fetch_add(&job->next, ORACLE_CHUNK_ROWS);
        if (r0 >= job->rows)
            break;
        int64_t r1 = r0 + ORACLE_CHUNK_ROWS < job->rows ? r0 + ORACLE_CHUNK_ROWS : job->rows;
        for (int64_t r = r0; r < r1; ++r) {
            if (job->cover) {
                job->cover[r] += 1;
                continue;
            }
            const uint8_t *row = job->canon + r * job->nb * ORACLE_BLOCK_BYTES;
            for (int32_t c = 0; c < job->ncols; ++c) {
                const int8_t *qc = job->q + c * job->ld_q;
                const float *dc = job->d + c * job->ld_d;
                job->y[c * job->rows + r] = job->fmt == ORACLE_Q1_0
                                                ? oracle_q1_0_row(row, job->nb, qc, dc, job->qa)
                                                : oracle_q2_0_row(row, job->nb, qc, dc, job->qa);
            }
        }
    }
    return NULL;
}

static int oracle_run(oracle_job *job, int threads)
{
    if (threads < 1)
        threads = 1;
    atomic_init(&job->next, 0);
    pthread_t *tid = NULL;
    int spawned = 0;
    if (threads > 1) {
        tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)(threads - 1));
        if (!tid)
            return -1;
        for (int t = 0; t < threads - 1; ++t) {
            if (pthread_create(&tid[t], NULL, oracle_worker, job) != 0)
                break;
            ++spawned;
        }
    }
    oracle_worker(job); /* the caller is worker 0 */
    for (int t = 0; t < spawned; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    return 0;
}

/* y holds ncols x rows floats, column c (activation c) contiguous.
 * canon holds rows x (cols / QK) blocks of 18 bytes.  Returns 0, or -1 on a
 * bad argument. */
int oracle_matvec(int fmt, const uint8_t *canon, int64_t rows, int64_t cols, const int8_t *q,
                  const float *d, int32_t qa, int32_t ncols, int64_t ld_q, int64_t ld_d, float *y,
                  int threads)
{
    int64_t qk = fmt == ORACLE_Q1_0 ? 128 : fmt == ORACLE_Q2_0 ? 64 : 0;
    if (qk == 0 || rows < 0 || cols < 0 || cols % qk || qa <= 0 || cols % qa || ncols < 1)
        return -1;
    oracle_job job;
    memset(&job, 0, sizeof job);
    job.fmt = fmt;
    job.canon = canon;
    job.rows = rows;
    job.nb = cols / qk;
    job.q = q;
    job.d = d;
    job.qa = qa;
    job.ncols = ncols;
    job.ld_q = ld_q;
    job.ld_d = ld_d;
    job.y = y;
    return oracle_run(&job, threads);
}

/* Coverage probe for the scheduler: counts how often each row is visited. */
int oracle_cover_rows(int64_t rows, int threads, int *counts)
{
    oracle_job job;
    memset(&job, 0, sizeof job);
    job.rows = rows;
    job.cover = counts;
    return oracle_run(&job, threads);
}
