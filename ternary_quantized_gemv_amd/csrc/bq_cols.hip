// bq_cols.hip -- several activation columns against one tall matrix, four
// columns per workgroup, one row per lane.
//
// The table key of a lane group is its weight nibble, which is the same for
// every activation column.  So the LDS tables of four columns are
// interleaved: entry n of a slot holds the four columns' values side by side
// (16 bytes), and one ds_read_b128 serves all four.  Per lane group and
// column what remains is the chain of the dot-product order (bankML "gpu/ --
// the video-card component", section "kernels.rs -- the Q1_0 kernels"),
// exactly as in the single-column kernels: for Q1_0 the sub-block-0 entries
// already hold d1*s (the same single rounding), then fma(d1, s, ab) per later
// sub-block and fma(d0, ab, acc) per block; the final tree per column.
//
// Tables cover a chunk of 4 blocks: 4 x 32 slots x 16 entries x 16 bytes
// (34 KiB with the slot padding below), rebuilt between barriers.  A workgroup is four wavefronts, one
// 64-row tile each, so three workgroups share a CU (registers allow three
// wavefronts per SIMD).
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

constexpr int kColsNC = 4;     // activation columns per workgroup
constexpr int kColsChunk = 4;  // blocks per table chunk
// the walk steps through a chunk four blocks at a time with a four-block
// payload ring, so a full chunk must be a multiple of four blocks
static_assert(kColsChunk % 4 == 0, "chunk of whole ring turns");
constexpr int kColsWaves = 4;  // wavefronts (tiles) per workgroup
// A slot's 16 entries take 256 bytes, padded to 272: the table builds store
// single floats (entry n, column c) from lanes that differ in slot and
// column, and a 256-byte slot stride would put sixteen of a wavefront's
// stores in each LDS bank (a 272-byte one: two).  Lookups of one slot stay
// within its 256 bytes.
constexpr int kColsSlotBytes = 16 * kColsNC * 4 + 16;
constexpr int kColsSlotVecs = kColsSlotBytes / 16;  // f32x4 per slot
constexpr int kColsSlotFloats = kColsSlotBytes / 4;
constexpr int kColsD1 = kColsChunk * 4 * kColsNC;  // activation scales per chunk [sub-block][column]

// Byte m of x masked to bits 4..7: nibble * 16, the byte offset of a
// four-column table entry.  (Byte 1 is spelled out as one SDWA instruction.)
__device__ __forceinline__ uint32_t nib16(uint32_t x, int m)
{
    if (m == 1) {
        uint32_t r;
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
            : "=v"(r)
            : "v"(x), "v"(0xF0u));
        return r;
    }
    return (x >> (8 * m)) & 0xF0u;
}

__device__ __forceinline__ f32x4 tab4(const f32x4 *T, int slot, uint32_t idx16)
{
    return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const char *>(T) + slot * kColsSlotBytes + idx16);
}

// The 16 table entries of one slot and column from its packed quants
// (Q1_0: four, Q2_0: two): Q1_0 entry n = sum_i (bit i of n ? q_i :
// wrap8(-q_i)); Q2_0 entry 4h + e = (e-1) q_0 + (h-1) q_1.  Formed in f32
// from converted quants: every partial sum is an integer of magnitude at
// most 512, so each addition is exact, and negation is a subtraction from
// +0 so that a zero entry is +0 as the integer sum's conversion would be.
// Q1_0 shares its pair sums: entry 4h + e = lo[e] + hi[h].
template <int FMT>
__device__ __forceinline__ void slot_entries(uint32_t wq, float (&v)[16])
{
    if (FMT == BQ_Q1_0) {
        float p[4], n[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int x = (int8_t)(wq >> (8 * i));
            p[i] = (float)x;
            n[i] = x == -128 ? -128.0f : 0.0f - p[i];
        }
        float lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo[e] = ((e & 1) ? p[0] : n[0]) + ((e & 2) ? p[1] : n[1]);
            hi[e] = ((e & 1) ? p[2] : n[2]) + ((e & 2) ? p[3] : n[3]);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[4 * h + e] = lo[e] + hi[h];
    } else {
        const float a = (float)(int8_t)(wq & 0xFF), b = (float)(int8_t)(wq >> 8);
        const float A[4] = {0.0f - a, 0.0f, a, a + a}, B[4] = {0.0f - b, 0.0f, b, b + b};
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[4 * h + e] = A[e] + B[h];
    }
}

// Tables of one chunk for columns c0 .. c0+3 (zeros for columns >= ncols).
// Q1_0 slot t covers chunk values 4t..4t+3 (block t/32, sub-block (t/8)%4,
// lane group t%8); entries as slot_entries, times d1 on sub-block 0.  Q2_0
// slot t covers values 2t, 2t+1.
template <int FMT, int QA, int CHUNK = kColsChunk, int THREADS = kColsWaves * 64>
__device__ void build_cols(f32x4 *T, float *D1, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int c0, int ncols,
                           int k0, int nbc)
{
    constexpr int S = FMT == BQ_Q1_0 ? 4 : 2;
    constexpr int kThreadsHere = THREADS;
    constexpr int kIters = CHUNK * kSlotsPerBlock * kColsNC / kThreadsHere;
    static_assert(kIters * kThreadsHere == CHUNK * kSlotsPerBlock * kColsNC, "whole slots per thread");
    // unit u = (slot t, column c): the slot's 16 entries of column c.  All of
    // a thread's loads are issued before any is used.
    const int nunits = nbc * kSlotsPerBlock * kColsNC;
    float *Tf = reinterpret_cast<float *>(T);
    uint32_t wq[kIters];
    float d1[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int u = threadIdx.x + it * kThreadsHere;
        const int c = u % kColsNC, t = u / kColsNC;
        const bool ok = u < nunits && c0 + c < ncols;
        const int cc = ok ? c0 + c : c0;
        const int8_t *q = g.q + (int64_t)cc * ld_q + k0;
        if (FMT == BQ_Q1_0) {
            wq[it] = ok ? *reinterpret_cast<const uint32_t *>(q + 4 * t) : 0u;
            d1[it] = ok && ((t >> 3) & 3) == 0 ? g.d[(int64_t)cc * ld_d + (k0 + 4 * t) / QA] : 0.0f;
        } else {
            wq[it] = ok ? *reinterpret_cast<const uint16_t *>(q + 2 * t) : 0u;
            d1[it] = 0.0f;
        }
    }
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int u = threadIdx.x + it * kThreadsHere;
        if (u >= nunits)
            break;
        const int c = u % kColsNC, t = u / kColsNC;
        float v[16];
        slot_entries<FMT>(wq[it], v);
        // a column past ncols loaded zeros: its entries are 0 (Q1_0 d1 = 0 on sub-block 0, and
        // the integer sums of zero quants are 0)
        const bool first = FMT == BQ_Q1_0 && ((t >> 3) & 3) == 0;
#pragma unroll
        for (int n = 0; n < 16; ++n)
            Tf[t * kColsSlotFloats + n * kColsNC + c] = first ? d1[it] * v[n] : v[n];
    }
    for (int i = threadIdx.x; i < nbc * S * kColsNC; i += kThreadsHere) {
        const int sb = i / kColsNC, c = i % kColsNC;
        const bool ok = c0 + c < ncols;
        D1[i] = ok ? g.d[(int64_t)(c0 + c) * ld_d + (k0 + 32 * sb) / QA] : 0.0f;
    }
}

// The chains of one block (index b within the chunk) of this lane's row for
// four columns, taken in two halves of four lane groups (each lane group's
// chain is independent of the others, so this only bounds the registers in
// use).
template <int FMT>
__device__ __forceinline__ void block_cols(const f32x4 *__restrict__ T, const float *__restrict__ D1, int b, u32x4 w,
                                           float d0, float acc[8][kColsNC])
{
    // even nibbles of a word at bits 4..7 of each byte after a left rotation
    // by 2, odd nibbles after a right rotation by 2
    uint32_t xe[4], xo[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        xe[m] = __builtin_amdgcn_alignbit(w[m], w[m], 30);
        xo[m] = __builtin_amdgcn_alignbit(w[m], w[m], 2);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float ab[4][kColsNC];
        if (FMT == BQ_Q1_0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 d1 = *reinterpret_cast<const f32x4 *>(D1 + (b * 4 + j) * kColsNC);
#pragma unroll
                for (int l = 0; l < 4; ++l) {
                    const int L = 4 * half + l;
                    const f32x4 v = tab4(T, b * kSlotsPerBlock + j * 8 + L, nib16((L & 1) ? xo[j] : xe[j], L >> 1));
#pragma unroll
                    for (int c = 0; c < kColsNC; ++c)
                        ab[l][c] = j == 0 ? v[c] : __builtin_fmaf(d1[c], v[c], ab[l][c]);
                }
                __builtin_amdgcn_sched_barrier(0);  // four lookups in flight at a time
            }
        } else {
            // lane group L = 4 * (word & 1) + byte of sub-block word / 2: this half's words are half, half + 2
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int m = 2 * j + half;
                const f32x4 d1 = *reinterpret_cast<const f32x4 *>(D1 + (b * 2 + j) * kColsNC);
#pragma unroll
                for (int beta = 0; beta < 4; ++beta) {
                    const int slot = b * kSlotsPerBlock + m * 8 + 2 * beta;
                    const f32x4 lo = tab4(T, slot, nib16(xe[m], beta));
                    const f32x4 hi = tab4(T, slot + 1, nib16(xo[m], beta));
#pragma unroll
                    for (int c = 0; c < kColsNC; ++c) {
                        const float s = lo[c] + hi[c];
                        ab[beta][c] = j == 0 ? d1[c] * s : __builtin_fmaf(d1[c], s, ab[beta][c]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // one word of lookups in flight at a time
            }
        }
#pragma unroll
        for (int l = 0; l < 4; ++l)
#pragma unroll
            for (int c = 0; c < kColsNC; ++c)
                acc[4 * half + l][c] = __builtin_fmaf(d0, ab[l][c], acc[4 * half + l][c]);
    }
}

// Workgroup id -> (row block of kColsWaves tiles, column group); ids 8 apart
// share an XCD, so the column groups of one row block read its weights from
// one L2.
template <int FMT, int QA>
__global__ __launch_bounds__(kColsWaves * 64) __attribute__((amdgpu_waves_per_eu(3))) void cols_kernel(GemvDesc g, int64_t ld_q, int64_t ld_d, int ncols, int tiles,
                                                        int cgroups)
{
    __shared__ f32x4 T[kColsChunk * kSlotsPerBlock * kColsSlotVecs];
    __shared__ float D1[kColsD1];
    const int id = blockIdx.x, slot = id & 7, rest = id >> 3;
    const int cg = rest % cgroups, rb = (rest / cgroups) * 8 + slot;
    if (rb * kColsWaves >= tiles)
        return;  // padding workgroup (the grid is a multiple of 8 row blocks)
    const int c0 = cg * kColsNC;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int tile = rb * kColsWaves + wave;
    const bool live = tile < tiles;
    // a wavefront past the last tile reads the workgroup's first tile and stores nothing
    const rsrc_t wp = rsrc_of(g.bits + tile_block0(FMT, live ? tile : rb * kColsWaves, g.nb) * kTileRows);
    const rsrc_t sp = rsrc_of(g.scales + (int64_t)(live ? tile : rb * kColsWaves) * g.ng * kTileRows);
    const uint32_t lo = (uint32_t)lane * 16;
    const int bl = FMT == BQ_Q1_0 ? 128 : 64;

    float acc[8][kColsNC];
#pragma unroll
    for (int L = 0; L < 8; ++L)
#pragma unroll
        for (int c = 0; c < kColsNC; ++c)
            acc[L][c] = 0.0f;
    // payload ring four blocks ahead (continuing across chunks); one scale group per chunk
    u32x4 ring[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        ring[i] = bload(wp, lo, (uint32_t)min(i, g.nb - 1) * kStep);
    u32x4 sc = bload(sp, lo, 0);

    for (int cb = 0; cb < g.nb; cb += kColsChunk) {
        const int nbc = min(kColsChunk, g.nb - cb);
        if (cb > 0)
            __syncthreads();  // every wavefront is done with the previous tables
        build_cols<FMT, QA>(T, D1, g, ld_q, ld_d, c0, ncols, cb * bl, nbc);
        __syncthreads();
        const u32x4 sc_next = bload(sp, lo, (uint32_t)min((cb + kColsChunk) / 8, g.ng - 1) * kStep);
        for (int i0 = 0; i0 < nbc; i0 += 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 w = ring[i];
                ring[i] = bload(wp, lo, (uint32_t)min(cb + i0 + i + 4, g.nb - 1) * kStep);
                if (i0 + i < nbc) {
                    float d0 = scale_of(sc, cb + i0 + i);
                    asm volatile("" : "+v"(d0));
                    block_cols<FMT>(T, D1, i0 + i, w, d0, acc);
                }
            }
        }
        if (kColsChunk == 8 || (cb + kColsChunk) % 8 == 0)
            sc = sc_next;
    }
    const int row = tile * kTileRows + lane;
    if (live && row < g.rows) {
#pragma unroll
        for (int c = 0; c < kColsNC; ++c) {
            if (c0 + c < ncols) {
                const float y = ((acc[0][c] + acc[4][c]) + (acc[2][c] + acc[6][c])) +
                                ((acc[1][c] + acc[5][c]) + (acc[3][c] + acc[7][c]));
                g.y[(int64_t)(c0 + c) * g.rows + row] = y;
            }
        }
    }
}

template <int FMT>
static hipError_t cols_fmt(int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                           hipStream_t st)
{
    const int cgroups = (ncols + kColsNC - 1) / kColsNC;
    const int rblocks = (tiles + kColsWaves - 1) / kColsWaves;
    const dim3 grid((unsigned)(((rblocks + 7) / 8) * 8 * cgroups));
    switch (qa) {
    case 32: hipLaunchKernelGGL((cols_kernel<FMT, 32>), grid, dim3(kColsWaves * 64), 0, st, g, ld_q, ld_d, ncols, tiles, cgroups); break;
    case 64: hipLaunchKernelGGL((cols_kernel<FMT, 64>), grid, dim3(kColsWaves * 64), 0, st, g, ld_q, ld_d, ncols, tiles, cgroups); break;
    default: hipLaunchKernelGGL((cols_kernel<FMT, 128>), grid, dim3(kColsWaves * 64), 0, st, g, ld_q, ld_d, ncols, tiles, cgroups); break;
    }
    return hipGetLastError();
}

hipError_t launch_cols(int fmt, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                       hipStream_t st)
{
    return fmt == BQ_Q1_0 ? cols_fmt<BQ_Q1_0>(qa, g, ld_q, ld_d, tiles, ncols, st)
                          : cols_fmt<BQ_Q2_0>(qa, g, ld_q, ld_d, tiles, ncols, st);
}

// ------------------------------------------------------------ split columns
// Several activation columns against a matrix of few row tiles (too few for
// cols_kernel's one row per lane to fill the GPU): W wavefronts share a
// 64-row tile, wavefront k carrying the chains of lane groups
// L = k, k + W, ... (LG = 8 / W of them) of every row, for four columns at
// once from the interleaved tables above (one ds_read_b128 serves the four).
// The lane groups of a wavefront are ones the final tree joins first --
// W = 4: a_k + a_(k+4); W = 2: (a_k + a_(k+4)) + (a_(k+2) + a_(k+6)) -- so a
// wavefront adds them in the tree's order and the remaining additions of
// the tree go through LDS.  Tables cover chunks of CH blocks: 16 (136 KiB,
// one workgroup per CU) when the launch's workgroups fit one round of the
// GPU and rows have more than 8 blocks, halving the chunks' table builds
// and barriers, else 8 (68 KiB, two workgroups per CU).  The wavefronts of
// a tile read the same payload (one HBM stream, the rest from the caches),
// each rotating a word once so that its lane groups' nibbles sit at bits
// 4..7 of bytes (nibble * 16: an entry of four floats).
constexpr int kScRing = 4;  // payload blocks loaded ahead

// The partial of a wavefront's lane groups, in the tree's order.
template <int LG>
__device__ __forceinline__ float sc_part(const float (&acc)[LG][kColsNC], int c)
{
    if constexpr (LG == 1)
        return acc[0][c];
    else if constexpr (LG == 2)
        return acc[0][c] + acc[1][c];
    else
        return (acc[0][c] + acc[2][c]) + (acc[1][c] + acc[3][c]);
}

// The inputs of one chunk's interleaved tables, read a chunk ahead into
// registers so that the build after the next barrier does not wait for
// memory: unit u = (slot t, column c) of the table.  Unlike
// build_cols, every entry holds the integer sum s (sub-block 0 too); the
// walk forms d1 * s itself, the same single rounding.
template <int FMT, int QA, int CHUNK, int THREADS>
struct ColsInputs {
    static constexpr int kIters = (CHUNK * kSlotsPerBlock * kColsNC + THREADS - 1) / THREADS;
    static constexpr int S = FMT == BQ_Q1_0 ? 4 : 2;
    static constexpr int kD1 = (CHUNK * S * kColsNC + THREADS - 1) / THREADS;
    uint32_t wq[kIters];
    float dd[kD1];

    __device__ __forceinline__ void load(const GemvDesc &g, int64_t ld_q, int64_t ld_d, int c0, int ncols, int k0,
                                         int nbc)
    {
        const int nunits = nbc * kSlotsPerBlock * kColsNC;
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int u = threadIdx.x + it * THREADS;
            const int c = u % kColsNC, t = u / kColsNC;
            const bool ok = u < nunits && c0 + c < ncols;
            const int cc = ok ? c0 + c : c0;
            const int8_t *q = g.q + (int64_t)cc * ld_q + k0;
            if (FMT == BQ_Q1_0)
                wq[it] = ok ? *reinterpret_cast<const uint32_t *>(q + 4 * t) : 0u;
            else
                wq[it] = ok ? *reinterpret_cast<const uint16_t *>(q + 2 * t) : 0u;
        }
#pragma unroll
        for (int r = 0; r < kD1; ++r) {
            const int i = threadIdx.x + r * THREADS;
            const int sb = i / kColsNC, c = i % kColsNC;
            const bool ok = i < nbc * S * kColsNC && c0 + c < ncols;
            dd[r] = ok ? g.d[(int64_t)(c0 + c) * ld_d + (k0 + 32 * sb) / QA] : 0.0f;
        }
    }

    // the tables of the loaded chunk: unit u = (slot t, column c), the
    // slot's 16 entries of column c (slot_entries)
    __device__ __forceinline__ void store(f32x4 *T, float *D1, int nbc) const
    {
        const int nunits = nbc * kSlotsPerBlock * kColsNC;
        float *Tf = reinterpret_cast<float *>(T);
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int u = threadIdx.x + it * THREADS;
            if (u >= nunits)
                break;
            const int c = u % kColsNC, t = u / kColsNC;
            float v[16];
            slot_entries<FMT>(wq[it], v);
#pragma unroll
            for (int n = 0; n < 16; ++n)
                Tf[t * kColsSlotFloats + n * kColsNC + c] = v[n];
        }
#pragma unroll
        for (int r = 0; r < kD1; ++r) {
            const int i = threadIdx.x + r * THREADS;
            if (i < nbc * S * kColsNC)
                D1[i] = dd[r];
        }
    }
};

// One block (index b within the chunk) of the calling lane's row: the chains
// of lane groups k + W*i, four columns each.
template <int FMT, int W>
__device__ __forceinline__ void sc_block(const f32x4 *__restrict__ T, const float *__restrict__ D1, int b, u32x4 w,
                                         float d0, int k, float (&acc)[8 / W][kColsNC])
{
    constexpr int LG = 8 / W;
    float ab[LG][kColsNC];
    if (FMT == BQ_Q1_0) {
        // nibble L sits at bits 4L+2 .. 4L+5; a right rotation by 4k - 2 brings
        // nibble k + W*i to bits 4..7 of byte i*W/2
        const uint32_t rot = (uint32_t)(4 * k + 30) & 31u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = __builtin_amdgcn_alignbit(w[j], w[j], rot);
            const f32x4 d1 = *reinterpret_cast<const f32x4 *>(D1 + (b * 4 + j) * kColsNC);
#pragma unroll
            for (int i = 0; i < LG; ++i) {
                const int L = k + W * i;
                const f32x4 v = tab4(T, b * kSlotsPerBlock + j * 8 + L, nib16(x, i * W / 2));
#pragma unroll
                for (int c = 0; c < kColsNC; ++c)
                    ab[i][c] = j == 0 ? d1[c] * v[c] : __builtin_fmaf(d1[c], v[c], ab[i][c]);
            }
        }
    } else {
        // lane group L of sub-block j is byte L & 3 of word 2j + (L >> 2); its low
        // nibble after a right rotation by 8(k & 3) - 2, its high nibble after
        // one by 8(k & 3) + 2, at bits 4..7 of byte (L & 3) - (k & 3)
        const uint32_t rlo = (uint32_t)(8 * (k & 3) + 30) & 31u, rhi = (uint32_t)(8 * (k & 3) + 2) & 31u;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const f32x4 d1 = *reinterpret_cast<const f32x4 *>(D1 + (b * 2 + j) * kColsNC);
#pragma unroll
            for (int i = 0; i < LG; ++i) {
                const int L = k + W * i;
                const int m = 2 * j + (L >> 2), beta = L & 3, byte = beta - (k & 3);
                const uint32_t xl = __builtin_amdgcn_alignbit(w[m], w[m], rlo);
                const uint32_t xh = __builtin_amdgcn_alignbit(w[m], w[m], rhi);
                const int slot = b * kSlotsPerBlock + m * 8 + 2 * beta;
                const f32x4 lo = tab4(T, slot, nib16(xl, byte));
                const f32x4 hi = tab4(T, slot + 1, nib16(xh, byte));
#pragma unroll
                for (int c = 0; c < kColsNC; ++c) {
                    const float sv = lo[c] + hi[c];
                    ab[i][c] = j == 0 ? d1[c] * sv : __builtin_fmaf(d1[c], sv, ab[i][c]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < LG; ++i)
#pragma unroll
        for (int c = 0; c < kColsNC; ++c)
            acc[i][c] = __builtin_fmaf(d0, ab[i][c], acc[i][c]);
}

// Workgroup id -> (row block of TPW tiles, column group); ids 8 apart share
// an XCD, so the column groups of one row block read its weights from one L2.
template <int FMT, int QA, int W, int TPW, int CH>
__global__ __launch_bounds__(W * TPW * 64) void splitcols_kernel(GemvDesc g, int64_t ld_q, int64_t ld_d, int ncols,
                                                                 int tiles, int cgroups)
{
    constexpr int kThreadsHere = W * TPW * 64;
    constexpr int LG = 8 / W;
    constexpr int kScChunk = CH;                          // blocks per table chunk
    constexpr int kScGroups = CH / kScalesPerGroup;      // scale groups per chunk
    static_assert(CH % kScalesPerGroup == 0 && CH % kScRing == 0, "whole scale groups and ring turns");
    __shared__ f32x4 T[kScChunk * kSlotsPerBlock * kColsSlotVecs];
    __shared__ float D1[kScChunk * 4 * kColsNC];
    __shared__ float P[TPW][W][kColsNC][64];
    const int id = blockIdx.x, slot = id & 7, rest = id >> 3;
    const int cg = rest % cgroups, rb = (rest / cgroups) * 8 + slot;
    if (rb * TPW >= tiles)
        return;  // padding workgroup (the grid is a multiple of 8 row blocks)
    const int c0 = cg * kColsNC;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int tl = wave / W, k = wave % W;
    const int tile = rb * TPW + tl;
    const bool live = tile < tiles;
    // a wavefront past the last tile reads the workgroup's first tile and stores nothing
    const int rt = live ? tile : rb * TPW;
    const rsrc_t wp = rsrc_of(g.bits + tile_block0(FMT, rt, g.nb) * kTileRows);
    const rsrc_t sp = rsrc_of(g.scales + (int64_t)rt * g.ng * kTileRows);
    const uint32_t lo = (uint32_t)lane * 16;
    const int bl = FMT == BQ_Q1_0 ? 128 : 64;

    float acc[LG][kColsNC];
#pragma unroll
    for (int i = 0; i < LG; ++i)
#pragma unroll
        for (int c = 0; c < kColsNC; ++c)
            acc[i][c] = 0.0f;
    // payload ring kScRing blocks ahead (continuing across chunks); the
    // chunk's scale groups, and the next chunk's requested during its walk
    u32x4 ring[kScRing];
#pragma unroll
    for (int i = 0; i < kScRing; ++i)
        ring[i] = bload(wp, lo, (uint32_t)min(i, g.nb - 1) * kStep);
    u32x4 sc[kScGroups];
#pragma unroll
    for (int s = 0; s < kScGroups; ++s)
        sc[s] = bload(sp, lo, (uint32_t)min(s, g.ng - 1) * kStep);

    ColsInputs<FMT, QA, kScChunk, kThreadsHere> in;
    in.load(g, ld_q, ld_d, c0, ncols, 0, min(kScChunk, g.nb));
    for (int cb = 0; cb < g.nb; cb += kScChunk) {
        const int nbc = min(kScChunk, g.nb - cb);
        if (cb > 0)
            __syncthreads();  // every wavefront is done with the previous tables
        in.store(T, D1, nbc);
        __syncthreads();
        if (cb + kScChunk < g.nb)  // the next chunk's table inputs, read during this walk
            in.load(g, ld_q, ld_d, c0, ncols, (cb + kScChunk) * bl, min(kScChunk, g.nb - cb - kScChunk));
        u32x4 sc_next[kScGroups];
#pragma unroll
        for (int s = 0; s < kScGroups; ++s)
            sc_next[s] = bload(sp, lo, (uint32_t)min(cb / kScalesPerGroup + kScGroups + s, g.ng - 1) * kStep);
#pragma unroll
        for (int i0 = 0; i0 < kScChunk; i0 += kScRing) {
#pragma unroll
            for (int i = 0; i < kScRing; ++i) {
                const u32x4 w = ring[i];
                ring[i] = bload(wp, lo, (uint32_t)min(cb + i0 + i + kScRing, g.nb - 1) * kStep);
                if (i0 + i < nbc) {
                    float d0 = scale_of(sc[(i0 + i) / kScalesPerGroup], i0 + i);
                    asm volatile("" : "+v"(d0));
                    sc_block<FMT, W>(T, D1, i0 + i, w, d0, k, acc);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < kScGroups; ++s)
            sc[s] = sc_next[s];
    }
#pragma unroll
    for (int c = 0; c < kColsNC; ++c)
        P[tl][k][c][lane] = sc_part<LG>(acc, c);
    __syncthreads();
    const int row = tile * kTileRows + lane;
    if (k == 0 && live && row < g.rows) {
#pragma unroll
        for (int c = 0; c < kColsNC; ++c) {
            if (c0 + c < ncols) {
                float y;
                if constexpr (W == 8)
                    y = ((P[tl][0][c][lane] + P[tl][4][c][lane]) + (P[tl][2][c][lane] + P[tl][6][c][lane])) +
                        ((P[tl][1][c][lane] + P[tl][5][c][lane]) + (P[tl][3][c][lane] + P[tl][7][c][lane]));
                else if constexpr (W == 4)
                    y = (P[tl][0][c][lane] + P[tl][2][c][lane]) + (P[tl][1][c][lane] + P[tl][3][c][lane]);
                else
                    y = P[tl][0][c][lane] + P[tl][1][c][lane];
                g.y[(int64_t)(c0 + c) * g.rows + row] = y;
            }
        }
    }
}

template <int FMT, int W, int TPW>
static hipError_t splitcols_shape(int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                                  hipStream_t st)
{
    const int cgroups = (ncols + kColsNC - 1) / kColsNC;
    const int rblocks = (tiles + TPW - 1) / TPW;
    const dim3 grid((unsigned)(((rblocks + 7) / 8) * 8 * cgroups)), block(W * TPW * 64);
    // 16-block chunks when the workgroups fit one per compute unit and the
    // rows are longer than one 8-block chunk
    const bool wide = (int64_t)rblocks * cgroups <= 256 && g.nb > 8;
#define BQ_SPLITCOLS(Q)                                                                                            \
    if (wide)                                                                                                      \
        hipLaunchKernelGGL((splitcols_kernel<FMT, Q, W, TPW, 16>), grid, block, 0, st, g, ld_q, ld_d, ncols, tiles, \
                           cgroups);                                                                               \
    else                                                                                                           \
        hipLaunchKernelGGL((splitcols_kernel<FMT, Q, W, TPW, 8>), grid, block, 0, st, g, ld_q, ld_d, ncols, tiles,  \
                           cgroups)
    switch (qa) {
    case 32: BQ_SPLITCOLS(32); break;
    case 64: BQ_SPLITCOLS(64); break;
    default: BQ_SPLITCOLS(128); break;
    }
#undef BQ_SPLITCOLS
    return hipGetLastError();
}

template <int FMT>
static hipError_t splitcols_fmt(int shape, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                                hipStream_t st)
{
    static_assert(kSplitColsShapes == 4, "one case per shape");
    switch (shape) {
    case 0: return splitcols_shape<FMT, 8, 1>(qa, g, ld_q, ld_d, tiles, ncols, st);
    case 1: return splitcols_shape<FMT, 4, 2>(qa, g, ld_q, ld_d, tiles, ncols, st);
    case 2: return splitcols_shape<FMT, 4, 3>(qa, g, ld_q, ld_d, tiles, ncols, st);
    default: return splitcols_shape<FMT, 4, 4>(qa, g, ld_q, ld_d, tiles, ncols, st);
    }
}

hipError_t launch_splitcols(int fmt, int shape, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles,
                            int ncols, hipStream_t st)
{
    return fmt == BQ_Q1_0 ? splitcols_fmt<BQ_Q1_0>(shape, qa, g, ld_q, ld_d, tiles, ncols, st)
                          : splitcols_fmt<BQ_Q2_0>(shape, qa, g, ld_q, ld_d, tiles, ncols, st);
}

}  // namespace bq
