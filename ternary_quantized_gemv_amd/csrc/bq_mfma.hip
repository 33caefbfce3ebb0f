// bq_mfma.hip -- 8 to 16 activation columns against one matrix, with the
// integer part of the dot product on the matrix cores.
//
// The dot-product order (bankML "gpu/ -- the video-card component", section
// "kernels.rs -- the Q1_0 kernels") needs, per row, column, block and
// 32-weight sub-block, eight exact integer sums s over four consecutive
// weights (the lane groups), and then a sequential f32 chain over them.  The
// sums are a product with a block-diagonal matrix: for a 16-weight slice of
// a sub-block (four lane groups),
//
//     S[(lane group, column)][row] = sum_k A[(lane group, column)][k] * W[k][row]
//
// where W holds the weights (+1/-1 for Q1_0, code - 1 for Q2_0) and
// A[(g, c)][k] is column c's int8 quant when weight k belongs to lane group
// g and 0 otherwise.  One v_mfma_f32_32x32x16_bf16 takes 32 (lane group,
// column) pairs (four lane groups x eight columns) against 32 rows.  Every
// operand is a small integer held exactly in bf16 (|q| <= 128, weights in
// {-1, 0, 1, 2}) and every partial sum is an integer below 2^12, so the f32
// results are the exact sums whatever order the matrix core adds in.
//
// Q1_0 multiplies -1 by -128 to -128 (int8 negation); a quant of -128 thus
// contributes -128 whatever the weight.  Such quants enter A as 0 and their
// contribution (-128 per occurrence) is added through the accumulator input
// of the MFMA; a chunk without them (always, for activations from the
// quantizer) takes the plain path.
//
// The chain then runs on the VALU exactly as in the table kernels: ab = d1*s
// on sub-block 0, fma(d1, s, ab) on the later ones, acc = fma(d0, ab, acc)
// per block, and the tree ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)) per row and
// column.
//
// Operand layout of v_mfma_f32_32x32x16_bf16 (measured on gfx950): lane l
// supplies row l%32 of A (column l%32 of B) and eight k values, slot i of
// lane half h pairing with slot i of the same half of the other operand;
// result register r of lane l holds element (8*(r/4) + 4*(l/32) + r%4,
// l%32).  Here element m of a result column is the pair (lane group
// g' = 2*((m/4)%2) + m%2, column 2*(m/8) + (m%4)/2) of the slice, so a
// register's column is the same in every lane (its d1 is one value) and a
// lane half holds the lane groups the tree adds first.
//
// Slice s (0 or 1) of a sub-block takes lane groups s, s+4 (lane half 0)
// and s+2, s+6 (lane half 1): the pairs a_k + a_(k+4) of the tree sit in one
// lane, and p_k + p_(k+2) across the two halves.
//
// A wavefront owns 32 rows and eight columns (lanes l and l + 32 read the
// same row's payload, each taking its half's nibbles); a workgroup of four
// wavefronts stages the activation fragments of a 4-block chunk in LDS (1 KiB
// per slice; zeros included) once for all its rows, the next chunk's quants
// already loaded into registers while the current chunk runs.
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMfChunk = 4;  // blocks per staged chunk
constexpr int kMfWaves = 4;  // wavefronts per workgroup
constexpr int kMfCols = 8;   // activation columns per workgroup

// bf16 bits of a small integer (exact: at most 8 significant bits).
__device__ __forceinline__ uint32_t bf16_of_int(int v)
{
    return __builtin_bit_cast(uint32_t, (float)v) >> 16;
}

// One chunk's activation for the workgroup's NC columns (8, or 4 in the
// whole-sub-block form), loaded into registers ahead of its staging: thread t
// holds 16 consecutive quants (four lane groups) of one column, and one d1.
template <int FMT, int QA, int NC>
struct MfChunk {
    static constexpr int JS = FMT == BQ_Q1_0 ? 4 : 2;     // sub-blocks per block
    static constexpr int BL = FMT == BQ_Q1_0 ? 128 : 64;  // weights per block
    static constexpr int kPieces = kMfChunk * BL / 16;    // 16-quant pieces of one column's chunk
    static constexpr int kDBlocks = (kMfChunk * BL + QA - 1) / QA;
    static_assert(NC * kPieces <= kMfWaves * 64, "one piece per thread");
    static_assert(kDBlocks * NC <= kMfWaves * 64, "one d1 per thread");
    u32x4 qv;
    float dv;
    int nbc;

    __device__ __forceinline__ void load(const GemvDesc &g, int64_t ld_q, int64_t ld_d, int c0, int ncols, int k0,
                                         int nblocks)
    {
        nbc = nblocks;
        // the column varies fastest across threads: the fragment stores of a
        // wavefront then spread over the LDS banks (eight consecutive pieces
        // of a column are still one 128-byte run of its quants)
        const int c = threadIdx.x % NC, p = threadIdx.x / NC;
        const bool ok = p < kPieces && p < nbc * BL / 16 && c0 + c < ncols;
        qv = ok ? *reinterpret_cast<const u32x4 *>(g.q + (int64_t)(c0 + c) * ld_q + k0 + 16 * p)
                : u32x4{0u, 0u, 0u, 0u};
        // d1 per activation-scale block of the chunk (k0 is a multiple of QA) and column
        const int dc = threadIdx.x % NC, db = threadIdx.x / NC;
        const bool dok = db < (nbc * BL + QA - 1) / QA && c0 + dc < ncols;
        dv = dok ? g.d[(int64_t)(c0 + dc) * ld_d + k0 / QA + db] : 0.0f;
    }

    // The nonzero halves of the A fragments of every (block, sub-block,
    // slice), the -128 corrections (Q1_0), and d1 per (scale block, column).
    // The other halves, and the fragments of lanes whose lane group lies in
    // the other half of the slice, stay zero from the kernel's start.  Sets
    // *wrap if a quant is -128 (Q1_0).
    //
    // NC = 8: fragment (block, sub-block j, slice s) holds lane groups s, s+4
    // (lane half 0) and s+2, s+6 (half 1) of eight columns; element m of a
    // result column is (lane group position 2((m/4)%2) + m%2, column
    // 2(m/8) + (m%4)/2).  NC = 4: fragments (block, j, t) for the two
    // 16-weight halves t of sub-block j, accumulated into one result whose
    // element m is (lane group m % 8, column m / 8); the correction of a
    // (block, j) goes in with t = 0.
    __device__ __forceinline__ void store(u32x4 *Afr, float *Bias, float *D1s, int *wrap) const
    {
        const int c = threadIdx.x % NC, p = threadIdx.x / NC;
        if (p < kPieces && p < nbc * BL / 16) {
            const int b = 16 * p / BL, o = 16 * p % BL, j = o / 32, L0 = (o % 32) / 4;
            bool any = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int L = L0 + e;
                int kh, m, fi, half, bi;
                if (NC == 8) {
                    // lane group L of slice s = L % 2 sits at local position gl: lane half
                    // kh = gl / 2, fragment half gl % 2 (slice s: groups s, s+4 | s+2, s+6)
                    const int sl = L & 1, gl = (L & 2) | ((L >> 2) & 1);
                    kh = gl >> 1;
                    m = 8 * (c >> 1) + 4 * kh + 2 * (c & 1) + (gl & 1);
                    fi = (b * JS + j) * 2 + sl;
                    half = gl & 1;
                    bi = fi * 32 + m;
                } else {
                    // weight k of half t = L / 4 in slot k % 8 of lane half (k % 16) / 8
                    kh = (L & 3) >> 1;
                    m = 8 * c + L;
                    fi = (b * JS + j) * 2 + (L >> 2);
                    half = L & 1;
                    bi = (b * JS + j) * 32 + m;
                }
                int cnt = 0;
                uint32_t h[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    int v = (int8_t)(qv[e] >> (8 * k));
                    if (FMT == BQ_Q1_0 && v == -128) {
                        ++cnt;
                        v = 0;
                    }
                    h[k] = bf16_of_int(v);
                }
                reinterpret_cast<u32x2 *>(&Afr[fi * 64 + 32 * kh + m])[half] =
                    u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                if (FMT == BQ_Q1_0) {
                    Bias[bi] = -128.0f * (float)cnt;
                    any |= cnt > 0;
                }
            }
            if (FMT == BQ_Q1_0 && any)
                *wrap = 1;
        }
        if (threadIdx.x < kDBlocks * NC)
            D1s[threadIdx.x] = dv;
    }
};

// The B fragment (eight weights of this lane's row) of slice s of sub-block
// j, from the 16-entry tables TB: Q1_0 entry n = four bf16 of nibble n's
// signs (8 bytes); Q2_0 entry n = two bf16 of nibble n's codes (4 bytes).
// xr: the block's words rotated for this lane half (see mf_block).
template <int FMT>
__device__ __forceinline__ bf16x8 mf_bfrag(const char *TB, const uint32_t (&xr)[8], int j, int s)
{
    u32x4 f;
    if (FMT == BQ_Q1_0) {
        // nibble of lane group s + 2h (byte 0) and s + 2h + 4 (byte 2) at bits 3..6: nibble * 8
        const uint32_t x = xr[2 * j + s];
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(TB + (x & 0x78u));
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(TB + ((x >> 16) & 0x78u));
        f = u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
        // lane group s + 2h: byte s of word 2j (low and high nibble), s + 2h + 4: byte s of word 2j + 1
        f[0] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[4 * j + 0], s));
        f[1] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[4 * j + 1], s));
        f[2] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[4 * j + 2], s));
        f[3] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[4 * j + 3], s));
    }
    return __builtin_bit_cast(bf16x8, f);
}

// The B fragment of 16-weight half t of sub-block j in the whole-sub-block
// form: lane groups 4t + 2h (slots 0-3) and 4t + 2h + 1 (slots 4-7).
template <int FMT>
__device__ __forceinline__ bf16x8 mf_bfrag4(const char *TB, const uint32_t (&xr)[8], int j, int t)
{
    u32x4 f;
    if (FMT == BQ_Q1_0) {
        // even nibble 4t + 2h of word j at bits 3..6 of byte 2t of xr[2j], the odd one of xr[2j + 1]
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(TB + ((xr[2 * j] >> (16 * t)) & 0x78u));
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(TB + ((xr[2 * j + 1] >> (16 * t)) & 0x78u));
        f = u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
        // bytes 2h and 2h + 1 of word 2j + t, moved to bytes 0 and 1 (low and high nibbles)
        const int m = 2 * j + t;
        f[0] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[2 * m], 0));
        f[1] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[2 * m + 1], 0));
        f[2] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[2 * m], 1));
        f[3] = *reinterpret_cast<const uint32_t *>(TB + nib4(xr[2 * m + 1], 1));
    }
    return __builtin_bit_cast(bf16x8, f);
}

// One block of this wavefront's 32 rows in the whole-sub-block form (four
// columns): per sub-block two MFMAs accumulate the sums of all eight lane
// groups; the pair of sub-block j + 1 is issued before the chain of j.
template <int FMT, int QA, bool WRAP>
__device__ __forceinline__ void mf_block4(const u32x4 *__restrict__ Afr, const float *__restrict__ Bias,
                                          const float *__restrict__ D1s, const char *TB, int b, u32x4 w, float d0,
                                          uint32_t rot0, uint32_t rot1, f32x16 &acc)
{
    constexpr int JS = FMT == BQ_Q1_0 ? 4 : 2;
    constexpr int BL = FMT == BQ_Q1_0 ? 128 : 64;
    const int lane = threadIdx.x & 63;
    uint32_t xr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xr[2 * i] = __builtin_amdgcn_alignbit(w[i], w[i], rot0);
        xr[2 * i + 1] = __builtin_amdgcn_alignbit(w[i], w[i], rot1);
    }
    auto issue = [&](int j) -> f32x16 {
        const int fi = (b * JS + j) * 2;
        f32x16 c = {};
        if (WRAP) {
            const f32x4 *bp = reinterpret_cast<const f32x4 *>(Bias + (b * JS + j) * 32 + 4 * (lane >> 5));
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 v = bp[2 * a];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    c[4 * a + e] = v[e];
            }
        }
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, Afr[fi * 64 + lane]),
                                                    mf_bfrag4<FMT>(TB, xr, j, 0), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, Afr[(fi + 1) * 64 + lane]),
                                                       mf_bfrag4<FMT>(TB, xr, j, 1), c, 0, 0, 0);
    };
    f32x16 ab;
    f32x16 cur = issue(0);
#pragma unroll
    for (int j = 0; j < JS; ++j) {
        f32x16 nxt = {};
        if (!WRAP && j + 1 < JS)
            nxt = issue(j + 1);
        // register r holds column r / 4
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(D1s + (b * BL + 32 * j) / QA * 4);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ab[r] = j == 0 ? d1[r >> 2] * cur[r] : __builtin_fmaf(d1[r >> 2], cur[r], ab[r]);
        if (WRAP) {
            if (j + 1 < JS)
                cur = issue(j + 1);
        } else {
            cur = nxt;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = __builtin_fmaf(d0, ab[r], acc[r]);
}

// One block of this wavefront's 32 rows: slice halves S0 .. S0 + HALVES - 1.
// The wavefront's MFMAs form a list of items (half, sub-block j) in chain
// order; the MFMA of item t + 1 is issued before the chain of item t
// consumes its result, so the matrix core works while the VALU runs the
// chain.
template <int FMT, int QA, int HALVES, int S0, bool WRAP>
__device__ __forceinline__ void mf_block(const u32x4 *__restrict__ Afr, const float *__restrict__ Bias,
                                         const float *__restrict__ D1s, const char *TB, int b, u32x4 w, float d0,
                                         uint32_t rot0, uint32_t rot1, f32x16 (&acc)[HALVES])
{
    constexpr int JS = FMT == BQ_Q1_0 ? 4 : 2;
    constexpr int BL = FMT == BQ_Q1_0 ? 128 : 64;
    constexpr int T = HALVES * JS;
    const int lane = threadIdx.x & 63;
    // Q1_0: xr[2j] = word j with the nibbles of even lane groups 2h, 2h + 4 at
    // bits 3..6 of bytes 0 and 2, xr[2j+1] the same for odd lane groups.
    // Q2_0: xr[4j + 2t + e] = word 2j + t with byte h*2 + s moved to byte s,
    // e = 1 after a further rotation by 4 (high nibbles).
    uint32_t xr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xr[2 * i] = __builtin_amdgcn_alignbit(w[i], w[i], rot0);
        xr[2 * i + 1] = __builtin_amdgcn_alignbit(w[i], w[i], rot1);
    }
    auto issue = [&](int t) -> f32x16 {
        const int j = t % JS, s = S0 + t / JS;
        const int fi = (b * JS + j) * 2 + s;
        const bf16x8 bf = mf_bfrag<FMT>(TB, xr, j, s);
        const bf16x8 af = __builtin_bit_cast(bf16x8, Afr[fi * 64 + lane]);
        f32x16 c = {};
        if (WRAP) {
            const f32x4 *bp = reinterpret_cast<const f32x4 *>(Bias + fi * 32 + 4 * (lane >> 5));
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 v = bp[2 * a];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    c[4 * a + e] = v[e];
            }
        }
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, c, 0, 0, 0);
    };
    f32x16 ab;
    f32x16 cur = issue(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int j = t % JS, hs = t / JS;
        f32x16 nxt = {};
        if (!WRAP && t + 1 < T)
            nxt = issue(t + 1);  // the -128 path (rare) keeps one MFMA in flight
        const f32x4 *dp = reinterpret_cast<const f32x4 *>(D1s + (b * BL + 32 * j) / QA * kMfCols);
        const f32x4 dlo = dp[0], dhi = dp[1];
        const float d1[8] = {dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float d = d1[2 * (r >> 2) + ((r >> 1) & 1)];
            ab[r] = j == 0 ? d * cur[r] : __builtin_fmaf(d, cur[r], ab[r]);
        }
        if (j == JS - 1) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[hs][r] = __builtin_fmaf(d0, ab[r], acc[hs][r]);
        }
        if (WRAP) {
            if (t + 1 < T)
                cur = issue(t + 1);
        } else {
            cur = nxt;
        }
    }
}

// Workgroup id -> (row group of 32-row tiles, group of NC columns); ids 8
// apart share an XCD, so the column groups of one row group read its weights
// through one L2.  NC = 8, HALVES = 2: a wavefront takes both slice halves of
// its 32 rows, four tiles per workgroup; HALVES = 1: the two halves of a tile
// in two wavefronts, two tiles per workgroup, joined through LDS at the end.
// NC = 4 (HALVES = 2): the whole-sub-block form, a wavefront per 32 rows.
template <int FMT, int QA, int HALVES, int NC>
__global__ __launch_bounds__(kMfWaves * 64) __attribute__((amdgpu_waves_per_eu(3))) void mfma_kernel(
    GemvDesc g, int64_t ld_q, int64_t ld_d, int ncols, int ntiles, int cgroups)
{
    static_assert(NC == 8 || (NC == 4 && HALVES == 2), "forms");
    using Chunk = MfChunk<FMT, QA, NC>;
    constexpr int JS = Chunk::JS;
    constexpr int BL = Chunk::BL;
    constexpr int TASKS = 2 / HALVES;       // wavefronts per 32-row tile
    constexpr int NTW = kMfWaves / TASKS;   // 32-row tiles per workgroup
    __shared__ u32x4 Afr[kMfChunk * JS * 2 * 64];
    __shared__ f32x4 Bias4[FMT == BQ_Q1_0 ? kMfChunk * JS * 2 * 8 : 1];
    __shared__ f32x4 D1s4[Chunk::kDBlocks * NC / 4];
    float *Bias = reinterpret_cast<float *>(Bias4);
    float *D1s = reinterpret_cast<float *>(D1s4);
    __shared__ u32x2 TB[16];
    __shared__ int Wrap[2];

    const int id = blockIdx.x, slot = id & 7, rest = id >> 3;
    const int cg = rest % cgroups, rg = (rest / cgroups) * 8 + slot;
    if (rg * NTW >= ntiles)
        return;  // padding workgroup (the grid is a multiple of 8 row groups)
    const int c0 = cg * NC;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nt = rg * NTW + wave / TASKS, sh = HALVES == 2 ? 0 : wave % 2;
    const bool live = nt < ntiles;
    const int ntc = live ? nt : rg * NTW;  // a wavefront past the last tile repeats the first and stores nothing
    const int kh = lane >> 5;
    const rsrc_t wp = rsrc_of(g.bits + tile_block0(FMT, ntc >> 1, g.nb) * kTileRows);
    const rsrc_t sp = rsrc_of(g.scales + (int64_t)(ntc >> 1) * g.ng * kTileRows);
    const uint32_t lo = (uint32_t)((ntc & 1) * 32 + (lane & 31)) * 16;
    // Q1_0: rotate right by 8h - 1 (even lane groups) and 8h + 3 (odd); Q2_0: 16h and 16h + 4.
    const uint32_t rot0 = FMT == BQ_Q1_0 ? (8u * kh + 31u) & 31u : 16u * kh;
    const uint32_t rot1 = FMT == BQ_Q1_0 ? 8u * kh + 3u : 16u * kh + 4u;

    Chunk next;
    next.load(g, ld_q, ld_d, c0, ncols, 0, min(kMfChunk, g.nb));
    if (threadIdx.x < 16) {
        const uint32_t n = threadIdx.x;
        if (FMT == BQ_Q1_0) {
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                h[i] = ((n >> i) & 1) ? 0x3F80u : 0xBF80u;  // bf16 +1 / -1
            TB[n] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        } else {
            // Q2_0 entries are 4 bytes: entry n at byte 4n
            reinterpret_cast<uint32_t *>(TB)[n] = bf16_of_int((int)(n & 3) - 1) | (bf16_of_int((int)(n >> 2) - 1) << 16);
        }
    }
    if (threadIdx.x == 0)
        Wrap[0] = 0;
    for (int i = threadIdx.x; i < kMfChunk * JS * 2 * 64; i += kMfWaves * 64)
        Afr[i] = u32x4{0u, 0u, 0u, 0u};
    if (FMT == BQ_Q1_0)
        for (int i = threadIdx.x; i < kMfChunk * JS * 2 * 8; i += kMfWaves * 64)
            Bias4[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    __syncthreads();

    f32x16 acc[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
        acc[h] = f32x16{};
    u32x4 ring[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        ring[i] = bload(wp, lo, (uint32_t)min(i, g.nb - 1) * kStep);
    // the weight scales of a chunk's four blocks: 8 bytes of the lane's 16-byte scale group
    auto scales4 = [&](int cb) {
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             sp, lo + (uint32_t)(cb % 8) * 2, (uint32_t)(cb / 8) * kStep, 2));
    };
    u32x2 sc = scales4(0);

    for (int cb = 0; cb < g.nb; cb += kMfChunk) {
        const int nbc = min(kMfChunk, g.nb - cb), par = (cb / kMfChunk) & 1;
        if (cb > 0)
            __syncthreads();  // every wavefront is done with the previous chunk
        if (threadIdx.x == 0)
            Wrap[par ^ 1] = 0;
        next.store(Afr, Bias, D1s, &Wrap[par]);
        __syncthreads();
        if (cb + kMfChunk < g.nb)
            next.load(g, ld_q, ld_d, c0, ncols, (cb + kMfChunk) * BL, min(kMfChunk, g.nb - cb - kMfChunk));
        const bool wrap = __builtin_amdgcn_readfirstlane(Wrap[par]) != 0;
        const u32x2 sc_next = scales4(min(cb + kMfChunk, (g.nb - 1) & ~(kMfChunk - 1)));
#pragma unroll
        for (int i = 0; i < kMfChunk; ++i) {
            const u32x4 w = ring[i];
            ring[i] = bload(wp, lo, (uint32_t)min(cb + i + 4, g.nb - 1) * kStep);
            if (i < nbc) {
                float d0 = f16_bits_to_f32((i & 1) ? (sc[i >> 1] >> 16) : (sc[i >> 1] & 0xFFFFu));
                asm volatile("" : "+v"(d0));
                const char *tb = reinterpret_cast<const char *>(TB);
                if constexpr (NC == 4) {
                    if (FMT == BQ_Q1_0 && wrap)
                        mf_block4<FMT, QA, true>(Afr, Bias, D1s, tb, i, w, d0, rot0, rot1, acc[0]);
                    else
                        mf_block4<FMT, QA, false>(Afr, Bias, D1s, tb, i, w, d0, rot0, rot1, acc[0]);
                } else if (FMT == BQ_Q1_0 && wrap) {
                    if (sh == 0)
                        mf_block<FMT, QA, HALVES, 0, true>(Afr, Bias, D1s, tb, i, w, d0, rot0, rot1, acc);
                    else
                        mf_block<FMT, QA, HALVES, 1, true>(Afr, Bias, D1s, tb, i, w, d0, rot0, rot1, acc);
                } else {
                    if (sh == 0)
                        mf_block<FMT, QA, HALVES, 0, false>(Afr, Bias, D1s, tb, i, w, d0, rot0, rot1, acc);
                    else
                        mf_block<FMT, QA, HALVES, 1, false>(Afr, Bias, D1s, tb, i, w, d0, rot0, rot1, acc);
                }
            }
        }
        sc = sc_next;
    }

    const int row = nt * 32 + (lane & 31);
    if constexpr (NC == 4) {
        // The tree: register 4c + k of lane half h holds lane group 4h + k of
        // column c; p_k = a_k + a_(k+4) across the halves, then
        // (p0 + p2) + (p1 + p3) within the lane.
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float o = __shfl_xor(acc[0][r], 32, 64);
            p[r] = acc[0][r] + o;
        }
        if (live && kh == 0 && row < g.rows) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (c0 + c < ncols)
                    g.y[(int64_t)(c0 + c) * g.rows + row] = (p[4 * c] + p[4 * c + 2]) + (p[4 * c + 1] + p[4 * c + 3]);
        }
        return;
    }
    // The tree: in lane half h, registers 2k and 2k + 1 of slice half s hold
    // lane groups s + 2h and s + 2h + 4 of column k.
    float P[HALVES][kMfCols];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int k = 0; k < kMfCols; ++k) {
            const float p = acc[h][2 * k] + acc[h][2 * k + 1];  // a_(s+2h) + a_(s+2h+4)
            const float o = __shfl_xor(p, 32, 64);
            P[h][k] = kh == 0 ? p + o : o + p;  // p_s + p_(s+2)
        }
    if (HALVES == 2) {
        if (live && kh == 0 && row < g.rows) {
#pragma unroll
            for (int k = 0; k < kMfCols; ++k)
                if (c0 + k < ncols)
                    g.y[(int64_t)(c0 + k) * g.rows + row] = P[0][k] + P[1][k];
        }
    } else {
        // the wavefront of slice half 1 hands its partial to that of half 0 through LDS
        float *X = reinterpret_cast<float *>(Afr);
        __syncthreads();
        const int t2 = wave / TASKS;  // tile of this wavefront within the workgroup
        if (sh == 1 && kh == 0) {
#pragma unroll
            for (int k = 0; k < kMfCols; ++k)
                X[(t2 * kMfCols + k) * 32 + (lane & 31)] = P[0][k];
        }
        __syncthreads();
        if (sh == 0 && live && kh == 0 && row < g.rows) {
#pragma unroll
            for (int k = 0; k < kMfCols; ++k)
                if (c0 + k < ncols)
                    g.y[(int64_t)(c0 + k) * g.rows + row] = P[0][k] + X[(t2 * kMfCols + k) * 32 + (lane & 31)];
        }
    }
}

template <int FMT, int HALVES, int NC>
static void mfma_shape(int qa, dim3 grid, hipStream_t st, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int ncols,
                       int ntiles, int cgroups)
{
    switch (qa) {
    case 32: hipLaunchKernelGGL((mfma_kernel<FMT, 32, HALVES, NC>), grid, dim3(kMfWaves * 64), 0, st, g, ld_q, ld_d, ncols, ntiles, cgroups); break;
    case 64: hipLaunchKernelGGL((mfma_kernel<FMT, 64, HALVES, NC>), grid, dim3(kMfWaves * 64), 0, st, g, ld_q, ld_d, ncols, ntiles, cgroups); break;
    default: hipLaunchKernelGGL((mfma_kernel<FMT, 128, HALVES, NC>), grid, dim3(kMfWaves * 64), 0, st, g, ld_q, ld_d, ncols, ntiles, cgroups); break;
    }
}

template <int FMT>
static hipError_t mfma_fmt(int shape, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int ncols,
                           hipStream_t st)
{
    const int nc = shape == 2 ? 4 : kMfCols;
    const int cgroups = (ncols + nc - 1) / nc;
    const int ntiles = (g.rows + 31) / 32;
    const int ntw = shape == 1 ? kMfWaves / 2 : kMfWaves;  // 32-row tiles per workgroup
    const int rgroups = (ntiles + ntw - 1) / ntw;
    const dim3 grid((unsigned)(((rgroups + 7) / 8) * 8 * cgroups));
    if (shape == 0)
        mfma_shape<FMT, 2, 8>(qa, grid, st, g, ld_q, ld_d, ncols, ntiles, cgroups);
    else if (shape == 1)
        mfma_shape<FMT, 1, 8>(qa, grid, st, g, ld_q, ld_d, ncols, ntiles, cgroups);
    else
        mfma_shape<FMT, 2, 4>(qa, grid, st, g, ld_q, ld_d, ncols, ntiles, cgroups);
    return hipGetLastError();
}

hipError_t launch_mfma(int fmt, int shape, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int ncols,
                       hipStream_t st)
{
    return fmt == BQ_Q1_0 ? mfma_fmt<BQ_Q1_0>(shape, qa, g, ld_q, ld_d, ncols, st)
                          : mfma_fmt<BQ_Q2_0>(shape, qa, g, ld_q, ld_d, ncols, st);
}

}  // namespace bq
