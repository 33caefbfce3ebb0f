/*
 * bq.h -- C ABI of libbq: 1-bit (Q1_0) and ternary (Q2_0) quantized
 * matrix-vector products on AMD Instinct MI355X (gfx950).
 *
 * The operation (bankML "gpu/ -- the video-card component", section
 * "kernels.rs -- the Q1_0 kernels"): a weight matrix stored as blocks of
 * packed sign bits or ternary codes with one f16 scale per block, times an
 * activation vector quantized to int8 with one f32 scale per block of qa
 * values, gives one f32 dot product per output row.  Every output element is
 * produced in one fixed order:
 *
 *   for each weight block b (Q1_0: 128 weights = 4 sub-blocks of 32;
 *                            Q2_0:  64 weights = 2 sub-blocks of 32):
 *     for each lane L in 0..7 and sub-block j:
 *       s   = exact int32 sum over weights 32j+4L .. 32j+4L+3 of w * q
 *             (Q1_0: w = +1 / -1, and -1 times -128 gives -128 as in an int8
 *              negation; Q2_0: w = code - 1)
 *       ab  = d1(j) * s        (first sub-block)
 *       ab  = fma(d1(j), s, ab) (later sub-blocks)
 *     acc[L] = fma(d0(b), ab, acc[L])        (acc starts at +0)
 *   y = ((acc0+acc4) + (acc2+acc6)) + ((acc1+acc5) + (acc3+acc7))
 *
 * with d0 the block's f16 scale widened exactly and d1(j) the activation
 * scale that covers the first value of sub-block j; every step is one
 * binary32 operation rounded to nearest-even (no flush of subnormals).  The
 * results do not depend on the grid, on how rows are split, or on which call
 * (matvec or sweep) computes them.
 *
 * Conventions for every entry point:
 *   - Return BQ_OK (0) on success or a BQ_E* code; the text of the last
 *     error of the calling thread, naming the call and the argument, is
 *     returned by bq_last_error().  No exception crosses this boundary, no
 *     call aborts, and there is no CPU fallback: a call that cannot run on
 *     the GPU fails.
 *   - Arguments are validated before anything is launched.  A GPU fault
 *     inside a kernel is reported by the caller's next synchronisation of
 *     the stream, not by the launching call.
 *   - "device" pointers are HIP device allocations (for example the
 *     data_ptr() of a torch tensor on a ROCm device); "host" pointers are
 *     ordinary process memory.  The caller allocates and owns every buffer;
 *     the library keeps no pointer after a call returns, except that a sweep
 *     plan keeps the pointers it was created with until it is destroyed.
 *   - GPU work is enqueued on the given stream (a hipStream_t, NULL = the
 *     null stream) and runs asynchronously; calls are reentrant and are
 *     ordered only by their streams.
 */
#ifndef BQ_H
#define BQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQ_ABI_VERSION 8

/* Weight formats (one canonical block = 18 bytes: f16 scale, little-endian,
 * then 16 payload bytes).
 *   BQ_Q1_0: 128 weights; weight k is bit (k & 7) of payload byte (k >> 3);
 *            bit 1 means +1, bit 0 means -1.
 *   BQ_Q2_0: 64 weights; weight k is bits 2(k&3)..2(k&3)+1 of payload byte
 *            (k >> 2); code c means weight c - 1 (codes 0, 1, 2 are -1, 0, +1;
 *            code 3 decodes as +2 on both the CPU and the GPU). */
#define BQ_Q1_0 1
#define BQ_Q2_0 2

/* Return codes. */
#define BQ_OK 0
#define BQ_EARG 1   /* null pointer, bad shape, unsupported qa / ncols / format */
#define BQ_EALIGN 2 /* a pointer or a leading dimension is not aligned as required */
#define BQ_EHIP 3   /* the HIP runtime reported an error (its text is kept) */
#define BQ_ENOMEM 4 /* a plan could not allocate its device table */

typedef void *bq_stream; /* hipStream_t */

/* A packed weight matrix as laid out by bq_pack (device pointers). */
typedef struct bq_weights {
    int32_t fmt;            /* BQ_Q1_0 or BQ_Q2_0 */
    int32_t reserved;       /* must be 0 */
    int64_t rows;           /* M >= 1 */
    int64_t cols;           /* K >= 1, a multiple of the block length (128 or 64) */
    const void *bits;       /* device, 16-byte aligned: payload plane from bq_pack */
    const uint16_t *scales; /* device, 16-byte aligned: scale plane from bq_pack */
} bq_weights;

/* ncols quantized activation vectors (device pointers), as written by
 * bq_quantize_act_q8: column c is q[c*ld_q .. c*ld_q + n) with scales
 * d[c*ld_d .. c*ld_d + n/qa). */
typedef struct bq_act {
    const int8_t *q; /* device, 16-byte aligned */
    const float *d;  /* device, 4-byte aligned */
    int64_t n;       /* values per column; must equal the weights' cols */
    int32_t qa;      /* values per scale: 32, 64 or 128 (n % qa == 0) */
    int32_t ncols;   /* number of activation columns, 1..16 */
    int64_t ld_q;    /* int8 elements between columns, >= n, multiple of 16 */
    int64_t ld_d;    /* floats between columns, >= n / qa */
} bq_act;

/* One product of a sweep: y = W x for one activation vector. */
typedef struct bq_gemv {
    bq_weights w;
    bq_act a; /* a.ncols must be 1 */
    float *y; /* device, 4-byte aligned: w.rows floats */
} bq_gemv;

/* One product of a sweep that quantizes in the launch: y = W q(x), with q
 * the activation quantizer's output for the f32 vector x. */
typedef struct bq_gemv_x {
    bq_weights w;
    const float *x; /* device, 16-byte aligned: w.cols floats */
    float *y;       /* device, 4-byte aligned: w.rows floats */
} bq_gemv_x;

typedef struct bq_sweep bq_sweep; /* opaque plan */

/* BQ_ABI_VERSION of the loaded library, so that a binding can refuse a
 * library built for another version of this interface instead of passing it
 * structs of another layout (bankML "gpu/ -- the video-card component",
 * section "Advantages and efficiency": checks fail closed).  Host only. */
int bq_abi_version(void);

/* Text of the calling thread's last error ("" if none): the failing call,
 * the argument and why (bankML "gpu/ -- the video-card component", section
 * "Advantages and efficiency": errors name the failing call; OneModel GPU
 * docs, section "Errors": a failure names what was being done).  Owned by
 * the library, thread-local, valid until the thread's next failing call.
 * Host only. */
const char *bq_last_error(void);

/* Sizes in bytes of the two device planes that bq_pack writes for a packed
 * rows x cols matrix of format fmt (bankML "gpu/ -- the video-card
 * component", section "kernels.rs -- the Q1_0 kernels": weights are
 * repacked once into the card's layout, bits as 32-bit words).  Writes
 * *bits_bytes and *scale_bytes (host pointers) and returns BQ_OK, or BQ_EARG
 * (unknown fmt; rows or cols not in [1, 2^31); cols not a multiple of the
 * block length; a 64-row tile's payload above 2^31 - 16 bytes; a null output
 * pointer) with nothing written.  The sizes come back through pointers so
 * that the result is a return code like every other call.  The planes'
 * layout belongs to the library and changes with BQ_ABI_VERSION (the
 * payload plane may hold unused zero padding between groups of row tiles):
 * size buffers with this call, not with a formula.  Host only; touches no
 * GPU. */
int bq_packed_bytes(int32_t fmt, int64_t rows, int64_t cols, size_t *bits_bytes, size_t *scale_bytes);

/* Repack canonical blocks into the device layout (bankML "gpu/", section
 * "kernels.rs": weights are repacked once, numbers unchanged, only
 * re-ordered).  Host only: canon (host) holds rows x (cols / block length)
 * canonical 18-byte blocks, row-major; bits_out and scales_out (host) must
 * hold the sizes bq_packed_bytes reports.  The caller copies both planes to
 * the device once.  Padding is written as zeros. */
int bq_pack(int32_t fmt, const uint8_t *canon, int64_t rows, int64_t cols, void *bits_out,
            uint16_t *scales_out);

/* Inverse of bq_pack: bits and scales (host, the planes bq_pack wrote for
 * the same fmt, rows, cols) give back the canonical blocks in canon_out
 * (host, rows x (cols / block length) x 18 bytes), byte for byte -- the
 * repacking changes no number, it only re-orders them (bankML "gpu/ -- the
 * video-card component", section "kernels.rs -- the Q1_0 kernels").
 * Returns BQ_OK, or BQ_EARG (shape as bq_packed_bytes, null pointer).
 * Host only. */
int bq_unpack(int32_t fmt, const void *bits, const uint16_t *scales, int64_t rows, int64_t cols,
              uint8_t *canon_out);

/* The activation quantizer: the int8 activation with one scale per block
 * that the products read (bankML "gpu/ -- the video-card component",
 * section "kernels.rs -- the Q1_0 kernels": the activation binding holds
 * f32 scales, one per 32 values, and int8 quants, and the activation is
 * repacked per call; here the block length qa is a parameter, 128 in the
 * configured workloads).  Quantize n floats x (device, 16-byte aligned) in
 * blocks of qa values: d = amax / 127 (f32, correctly rounded), q = x / d
 * (correctly rounded) rounded half away from zero into [-127, 127]; an
 * all-zero block gives d = 0 and q = 0.  q (device, 4-byte aligned)
 * receives n int8 values and d (device, 4-byte aligned) n / qa floats.  qa
 * is 32, 64 or 128; n % qa == 0 (n = 0 does nothing).  Non-finite inputs are
 * outside the contract.  Returns BQ_EARG / BQ_EALIGN before any launch, or
 * BQ_EHIP if the launch fails.  Allocates nothing.  Asynchronous on s. */
int bq_quantize_act_q8(const float *x, int64_t n, int32_t qa, int8_t *q, float *d, bq_stream s);

/* The same quantizer with f16-valued scales, the flavour of the pages' q8_0
 * activation (bankML "gpu/", section "kernels.rs -- the Q1_0 kernels": the
 * activation binding holds one scale per 32 values; section "Advantages and
 * efficiency": d1*s is exact in f32, which holds when d1 has at most 11
 * significant bits).  Per block of qa values: d = amax / 127 (correctly
 * rounded), then narrowed to the nearest f16 value (ties to even) and stored
 * widened in d; q = x / d (correctly rounded) rounded half away from zero,
 * clamped to [-127, 127] -- the clamp can bind when d falls in the f16
 * subnormal range (amax < 127 * 2^-14).  d == 0 (also when amax / 127
 * narrows to 0) gives q = 0.  Blocks with amax / 127 >= 65520 (d = +inf)
 * are outside the contract, as are non-finite inputs.  Arguments, alignment
 * and errors as bq_quantize_act_q8.  Asynchronous on s. */
int bq_quantize_act_q8_f16(const float *x, int64_t n, int32_t qa, int8_t *q, float *d, bq_stream s);

/* The product itself (bankML "gpu/ -- the video-card component", section
 * "kernels.rs -- the Q1_0 kernels": one f32 dot product per row, in the
 * order given at the top of this file; Q2_0 by the same order, readings of
 * the format noted above).  y (device, 4-byte aligned, a.ncols * w->rows
 * floats; column c at y + c * rows) = W times each activation column.
 * w (host struct, device planes) must have fmt BQ_Q1_0 (resp. BQ_Q2_0 for
 * the second call); a (host struct, device arrays) must have a->n ==
 * w->cols.  Returns BQ_EARG / BQ_EALIGN before any launch, or BQ_EHIP if the
 * launch fails.  Allocates nothing.  Asynchronous on s. */
int bq_q1_0_matvec(const bq_weights *w, const bq_act *a, float *y, bq_stream s);
int bq_q2_0_matvec(const bq_weights *w, const bq_act *a, float *y, bq_stream s);

/* Which kernels compute the lane-group sums of bq_q1_0_matvec /
 * bq_q2_0_matvec for 2 to 16 activation columns: BQ_BATCH_AUTO (the path
 * measured faster for the shape and column count), BQ_BATCH_TABLES (LDS
 * lookup tables of the activation, the VALU path) or BQ_BATCH_MFMA (exact
 * integer sums on the matrix cores, as products with a block-diagonal
 * activation matrix; the f32 chain of the order above stays on the VALU).  Both paths give the same
 * bits; the choice affects only speed.  The sums are the integer part of
 * bankML "gpu/ -- the video-card component", section "kernels.rs -- the
 * Q1_0 kernels" (exact lane-group sums before the chain).  Process-wide,
 * atomic; calls already launched keep their path.  Returns the previous
 * setting, or -1 (with BQ_EARG's message) for an unknown path.  Host only. */
#define BQ_BATCH_AUTO 0
#define BQ_BATCH_TABLES 1
#define BQ_BATCH_MFMA 2
int bq_set_batch_path(int path);

/* One group of a dependency-ordered decode step in ONE launch: the count
 * products (1..4) that read the same activation -- bankML "gpu/ -- the
 * video-card component", section "Limitations": Q/K/V, and gate/up, are
 * submitted together with one wait per group.  x (device, 16-byte aligned)
 * holds the f32 activation of length w[0].cols; it is quantized in blocks of
 * qa exactly as bq_quantize_act_q8 would (the quants stay on chip) and
 * y[i] (device, 4-byte aligned, w[i].rows floats) receives what
 * bq_q1_0_matvec / bq_q2_0_matvec would write for w[i] and those quants.
 * Every w[i] must share w[0]'s format and cols (a multiple of qa); qa is
 * 32, 64 or 128.  No y[i] may overlap x.  w and y are host arrays of count
 * entries, read during the call.  Allocates nothing.  Asynchronous on s. */
int bq_group_matvec(const bq_weights *w, int32_t count, const float *x, int32_t qa, float *const *y,
                    bq_stream s);

/* A plan for many independent products run by ONE kernel launch (the 253
 * products of one decode token: bankML "par.rs -- the persistent thread pool
 * and row scheduler", section "Summary").  All entries must share one format
 * and one qa, with ncols == 1.  Validates every entry, balances the work
 * over the GPU and copies a descriptor table to the device (the plan's only
 * allocation, freed by bq_sweep_destroy).  Must be called with the device of
 * the pointers current.  *plan receives the plan, or NULL on failure. */
int bq_sweep_create(const bq_gemv *list, int32_t count, bq_sweep **plan);

/* As bq_sweep_create, for products whose activations are f32 vectors that
 * the launch itself quantizes: every workgroup quantizes the blocks of x it
 * needs into on-chip memory, with bq_quantize_act_q8's rule and block length
 * qa (32, 64 or 128; every w.cols a multiple of qa), before building its
 * tables, so a decode token's products run from their f32 inputs in one
 * launch and the int8 vectors never go to memory (bankML "par.rs -- the
 * persistent thread pool and row scheduler", section "Summary": one token's
 * 253 products; bankML "gpu/ -- the video-card component", section
 * "kernels.rs -- the Q1_0 kernels": the activation is quantized per call).
 * Each y equals what bq_quantize_act_q8 followed by bq_q1_0_matvec /
 * bq_q2_0_matvec would give.  No y may overlap an x.  Allocation, errors and
 * ownership as bq_sweep_create; run and release the plan with
 * bq_token_sweep and bq_sweep_destroy. */
int bq_sweep_create_x(const bq_gemv_x *list, int32_t count, int32_t qa, bq_sweep **plan);

/* Enqueue the whole plan on s as ONE kernel launch (bankML "gpu/ -- the
 * video-card component", section "Limitations": each of the token's 253
 * matrix calls paid one submit and wait there; here the token is one
 * submission).  Each entry's y equals what bq_q1_0_matvec / bq_q2_0_matvec
 * would write for it; the plan's pointers must still be valid.  Returns
 * BQ_EARG (null plan) or BQ_EHIP if the launch fails.  Allocates nothing.
 * Asynchronous on s. */
int bq_token_sweep(const bq_sweep *plan, bq_stream s);

/* The sweep of bq_sweep_create + bq_token_sweep in ONE call that allocates
 * nothing, for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  The
 * list (host array of count bq_gemv, rules as bq_sweep_create) is validated
 * and planned on fixed host storage, and the plan (descriptors and work
 * items) is copied on s into a fixed device array of the library: 320 KiB
 * per GPU, held until the process ends, room for up to 1024 products and
 * 16384 work items (the 253 products of a decode token need 1,743 in Q1_0,
 * 2,029 in Q2_0).
 * Larger lists are refused with BQ_EARG, as is every invalid entry, before
 * anything is copied or launched.  The copy is from pageable memory, so the
 * call returns once the table is staged; it may wait for earlier work on s.
 * Each entry's y equals what bq_token_sweep of a bq_sweep_create plan of the
 * same list writes.  All calls on one GPU share that GPU's array: calls on
 * one stream are ordered, but calls that overlap on one GPU (several streams
 * or threads with launches in flight together) race on it.  Calls from
 * several host threads are serialised while they plan.  Returns BQ_OK,
 * BQ_EARG / BQ_EALIGN, or BQ_EHIP if the copy or the launch fails.
 * Asynchronous on s. */
int bq_token_sweep_noalloc(const bq_gemv *list, int32_t count, bq_stream s);

/* Release a plan and its device table (NULL is allowed): resources are
 * released only by an explicit call, never behind the caller's back (bankML
 * "gpu/ -- the video-card component", section "compute.rs -- Vulkan
 * compute": a buffer is released only by the free call).  Synchronises the
 * device first, so launches of the plan still in flight finish. */
void bq_sweep_destroy(bq_sweep *plan);

/* The streaming-read floor, a measurement aid and not a step of the
 * product (bankML "par.rs -- the persistent thread pool and row scheduler",
 * sections "How it is verified" and "Advantages and efficiency": the memory
 * floor a token's weight stream is compared against).  Reads every byte of
 * p (device, 16-byte aligned, bytes a positive multiple of 16) once with
 * plain 16-byte loads from a fixed grid and writes BQ_FLOOR_SINK_WORDS
 * uint32 to sink (device, 4-byte aligned): the XOR of all of them equals
 * the XOR of all 32-bit words of the buffer.  Time it with events to get
 * the read bandwidth a kernel can reach on this GPU.  Allocates nothing.
 * Asynchronous on s. */
#define BQ_FLOOR_SINK_WORDS 8192
int bq_read_floor(const void *p, int64_t bytes, uint32_t *sink, bq_stream s);

#ifdef __cplusplus
}
#endif

#endif /* BQ_H */
