// bq_kernels.hip -- gfx950 kernels of libbq and the GPU entry points of the
// C ABI (include/bq.h).
//
// The product computed for every output row is the dot-product order of
// bankML's GPU page ("gpu/ -- the video-card component", section "kernels.rs
// -- the Q1_0 kernels"): per block, eight lanes of exact integer sums over
// four consecutive weights of each 32-weight sub-block; ab = d1*s on the
// first sub-block, ab = fma(d1, s, ab) on the others; acc = fma(d0, ab, acc);
// then the tree ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)).  Everything is built
// with -ffp-contract=off and every fused step is an explicit fma, so the
// compiler neither fuses nor splits what that order prescribes.
//
// How the work maps onto CDNA4
// ----------------------------
// * One wavefront owns 64 rows (lane i = row 64t+i) and carries all eight
//   lane accumulators of its row in registers.  Rows never split across
//   threads, so the result does not depend on the grid.
// * The weights stream from HBM once: per block each lane issues one 16-byte
//   load of its row's payload, and the layout (bq_layout.h) makes the 64
//   loads of a wavefront one contiguous KiB.  Loads run kPrefetch blocks
//   ahead of the arithmetic.
// * The activation never meets the weights as bytes.  For each group of
//   weights that shares one 4-bit nibble of packed weights (Q1_0: 4 signs;
//   Q2_0: 2 codes) the workgroup first tabulates, in LDS, the partial sum for
//   all 16 nibble values (exact small integers held as floats; for Q1_0's
//   first sub-block the table already holds the rounded product d1*s, which
//   is the same single rounding the order prescribes).  The inner loop is
//   then: byte-select the nibble (SDWA), one LDS read, one fma.  All 64
//   lanes of a wavefront read the same 16-entry table, so reads never
//   conflict on LDS banks.
// * A table covers a chunk of 32 blocks (64 KiB); longer rows walk several
//   chunks, rebuilding the table between barriers while the accumulators
//   stay in registers.
// * The sweep runs all products of a decode token in one launch: one
//   workgroup per work item (up to 8 tiles of one matrix), ordered from the
//   most to the least work so the hardware's in-order dispatch balances the
//   GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "../../include/bq.h"
#include "bq_layout.h"

namespace bq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkBlocks = 32;                                     // blocks per LDS table
constexpr int kSlotsPerBlock = 32;                                   // nibbles per block
constexpr int kSlotFloats = 16;                                      // entries per nibble table
constexpr int kTableFloats = kChunkBlocks * kSlotsPerBlock * kSlotFloats;  // 64 KiB
constexpr int kScaleFloats = kChunkBlocks * 4;                       // d1 per sub-block
#ifndef BQ_WAVES
#define BQ_WAVES 8
#endif
#ifndef BQ_PREFETCH
#define BQ_PREFETCH 4
#endif
#ifndef BQ_PIPE
#define BQ_PIPE 1
#endif
constexpr int kWaves = BQ_WAVES;                                     // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kPrefetch = BQ_PREFETCH;                               // blocks loaded ahead
#ifdef BQ_WPE
#define BQ_KATTR __attribute__((amdgpu_waves_per_eu(BQ_WPE, BQ_WPE)))
#else
#define BQ_KATTR
#endif
#ifndef BQ_MAX_ROUNDS
#define BQ_MAX_ROUNDS 3
#endif
#ifndef BQ_TAIL_ITEMS
#define BQ_TAIL_ITEMS 1024
#endif
// Sweep work items of single-chunk products hold up to kMaxRounds tiles per
// wavefront, all served by one table; the last kTailItems items of the
// dispatch order are cut back to one tile per wavefront so the end of the
// launch drains in small pieces.
constexpr int kMaxRounds = BQ_MAX_ROUNDS;
static_assert(kChunkBlocks % kPrefetch == 0, "a chunk must hold a whole number of prefetch rounds");
constexpr int kTailItems = BQ_TAIL_ITEMS;

struct GemvDesc {
    const u32x4 *bits;    // payload plane
    const u32x4 *scales;  // scale plane: 8 f16 per lane per 16 bytes
    const int8_t *q;      // activation quants of this product
    const float *d;       // activation scales
    float *y;             // output
    int32_t rows;
    int32_t nb;  // blocks per row
    int32_t ng;  // scale groups (of 8 blocks) per row
    int32_t pad;
};

struct WorkItem {
    int32_t gemv;
    int32_t tile0;
    int32_t ntiles;  // tiles tile0 .. tile0+ntiles-1; wavefront w takes tile0+w, tile0+w+kWaves, ...
    int32_t pad;
};

typedef const float __attribute__((address_space(4))) *cfptr;

// Weight planes are read through buffer resources: the wave-uniform base of
// a tile sits in scalar registers, each lane adds its 16-byte offset, and the
// block offset is a scalar constant, so a load costs no vector address math.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t rsrc_of(const u32x4 *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(base), (short)0, 0x7FFFFFF0, 0x00020000);
}

// 16 bytes at base + voff + soff, streamed (non-temporal).
__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// --------------------------------------------------------------- tables
// Each thread writes one quarter (4 entries, 16 bytes) of a slot's table per
// step, so a wavefront's stores cover 1 KiB of consecutive LDS addresses.
//
// Q1_0: slot t of a chunk covers chunk values 4t..4t+3 (block t/32, sub-block
// (t/8)%4, lane t%8).  Entry n = 4h + e: s = sum_i (bit i of n ? q_i : -q_i),
// where the negation of -128 stays -128; on sub-block 0 the entry is d1*s.
template <int QA>
__device__ void build_table_q1(float *T, float *D1, const int8_t *q, const float *d, int k0, int nbc)
{
    const int nquarters = nbc * kSlotsPerBlock * 4;
    for (int u = threadIdx.x; u < nquarters; u += blockDim.x) {
        const int t = u >> 2, h = u & 3;
        const uint32_t w4 = *reinterpret_cast<const uint32_t *>(q + k0 + 4 * t);
        int p1[4], p0[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = (int8_t)(w4 >> (8 * i));
            p1[i] = v;
            p0[i] = v == -128 ? -128 : -v;
        }
        const int hi = ((h & 1) ? p1[2] : p0[2]) + ((h & 2) ? p1[3] : p0[3]);
        const bool first = ((t >> 3) & 3) == 0;
        const float d1 = first ? d[(k0 + 4 * t) / QA] : 0.0f;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int lo = ((e & 1) ? p1[0] : p0[0]) + ((e & 2) ? p1[1] : p0[1]);
            const float sf = (float)(lo + hi);
            v[e] = first ? d1 * sf : sf;
        }
        reinterpret_cast<f32x4 *>(T + t * kSlotFloats)[h] = v;
    }
    for (int i = threadIdx.x; i < nbc * 4; i += blockDim.x)
        D1[i] = d[(k0 + 32 * i) / QA];
}

// Q2_0: slot t of a chunk covers chunk values 2t and 2t+1 (the low or high
// nibble of payload byte t/2 of its block).  Entry n = 4h + e holds the codes
// (e, h): (e-1)*q_2t + (h-1)*q_2t+1.
template <int QA>
__device__ void build_table_q2(float *T, float *D1, const int8_t *q, const float *d, int k0, int nbc)
{
    const int nquarters = nbc * kSlotsPerBlock * 4;
    for (int u = threadIdx.x; u < nquarters; u += blockDim.x) {
        const int t = u >> 2, h = u & 3;
        const uint32_t w2 = *reinterpret_cast<const uint16_t *>(q + k0 + 2 * t);
        const int qa0 = (int8_t)(w2 & 0xFF), qa1 = (int8_t)(w2 >> 8);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (float)((e - 1) * qa0 + (h - 1) * qa1);
        reinterpret_cast<f32x4 *>(T + t * kSlotFloats)[h] = v;
    }
    // d1 per (block, sub-block): D1[4b + j], j = 0, 1.
    for (int i = threadIdx.x; i < nbc * 4; i += blockDim.x) {
        const int b = i >> 2, j = i & 3;
        D1[i] = j < 2 ? d[(k0 + 64 * b + 32 * j) / QA] : 0.0f;
    }
}

// LDS read of entry (byte offset idx4 = nibble*4) of the table at slot `slot`.
__device__ __forceinline__ float tab(const float *T, int slot, uint32_t idx4)
{
    return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(T) + slot * (kSlotFloats * 4) + idx4);
}

// Byte m of w masked to bits 2..5: the byte offset of a nibble's table entry.
// The compiler selects bytes 0, 2 and 3 with SDWA on its own; byte 1 is
// spelled out so that it also costs a single instruction.
__device__ __forceinline__ uint32_t nib4(uint32_t w, int m)
{
#ifdef BQ_NO_SDWA
    if (m > 0) {
        uint32_t t = w >> (8 * m);
        asm volatile("" : "+v"(t));
        return t & 0x3Cu;
    }
#endif
    if (m == 1) {
        uint32_t r;
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
            : "=v"(r)
            : "v"(w), "v"(0x3Cu));
        return r;
    }
    return (w >> (8 * m)) & 0x3Cu;
}

// ------------------------------------------------------- activation scales
// d1 of the four sub-blocks of block b of a chunk.  When a full chunk has at
// most 32 distinct activation scales they sit in scalar registers for the
// whole chunk (loaded once, wave-uniform); otherwise they are read from the
// chunk's LDS copy.
template <int FMT, int QA>
struct ChunkScales {
    static constexpr int BL = FMT == BQ_Q1_0 ? 128 : 64;
    static constexpr int ND = kChunkBlocks * BL / QA;
    static constexpr bool kScalar = ND <= 32;
    float dv[kScalar ? ND : 1];

    __device__ __forceinline__ void load(const float *d_chunk)
    {
        if (kScalar) {
            // the address is wave-uniform; say so, so that the loads are scalar
            const uint64_t a = (uint64_t)d_chunk;
            const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
            const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
            const cfptr gc = (cfptr)(const float *)((hi << 32) | lo);
#pragma unroll
            for (int i = 0; i < (kScalar ? ND : 1); ++i) {
                dv[i] = gc[i];
                asm volatile("" : "+s"(dv[i]));  // load all of them here, once per chunk
            }
        }
    }

    __device__ __forceinline__ f32x4 get(const float *__restrict__ D1, int b) const
    {
        f32x4 r;
        if (kScalar) {
            constexpr int sub = FMT == BQ_Q1_0 ? 4 : 2;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                r[j] = j < sub ? dv[((BL * b + 32 * j) / QA) % (kScalar ? ND : 1)] : 0.0f;
        } else {
            r = *reinterpret_cast<const f32x4 *>(D1 + 4 * b);
        }
        return r;
    }
};

// ------------------------------------------------------------ block math
// The eight lane chains of one block of the calling lane's row.  `b` is the
// block's index inside the table chunk; v its four payload words; d0 its
// widened scale.
template <int FMT>
__device__ __forceinline__ void block_math(const float *__restrict__ T, const f32x4 d1, int b, u32x4 v, float d0,
                                           float acc[8])
{
    float ab[8];
    if (FMT == BQ_Q1_0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t wa = v[j];
            const uint32_t wb = __builtin_amdgcn_alignbit(wa, wa, 4);
#pragma unroll
            for (int L = 0; L < 8; ++L) {
                const uint32_t idx = nib4((L & 1) ? wb : wa, L >> 1);
                const float t = tab(T, b * kSlotsPerBlock + j * 8 + L, idx);
                ab[L] = j == 0 ? t : __builtin_fmaf(d1[j], t, ab[L]);
            }
#ifdef BQ_SPLIT
            if (j % BQ_SPLIT == BQ_SPLIT - 1)
                __builtin_amdgcn_sched_barrier(0);
#endif
        }
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t wa = v[m];
            const uint32_t wb = __builtin_amdgcn_alignbit(wa, wa, 4);
            const int j = m >> 1;
#pragma unroll
            for (int beta = 0; beta < 4; ++beta) {
                const int L = 4 * (m & 1) + beta;
                const int slot = b * kSlotsPerBlock + m * 8 + 2 * beta;
                const float s = tab(T, slot, nib4(wa, beta)) + tab(T, slot + 1, nib4(wb, beta));
                ab[L] = j == 0 ? d1[0] * s : __builtin_fmaf(d1[1], s, ab[L]);
            }
        }
    }
#pragma unroll
    for (int L = 0; L < 8; ++L) {
        acc[L] = __builtin_fmaf(d0, ab[L], acc[L]);
        asm volatile("" : "+v"(acc[L]));  // keep each block's chain inside its own code
    }
}

// The eight table reads of sub-block j of a Q1_0 block.
__device__ __forceinline__ void lookups_q1(const float *__restrict__ T, int b, int j, uint32_t wa, float t[8])
{
    const uint32_t wb = __builtin_amdgcn_alignbit(wa, wa, 4);
#pragma unroll
    for (int L = 0; L < 8; ++L)
        t[L] = tab(T, b * kSlotsPerBlock + j * 8 + L, nib4((L & 1) ? wb : wa, L >> 1));
}

__device__ __forceinline__ float scale_of(u32x4 sc, int b)
{
    const uint32_t sw = sc[(b & 7) >> 1];
    return f16_bits_to_f32((b & 1) ? (sw >> 16) : (sw & 0xFFFFu));
}

// Payload words of the first kPrefetch blocks of a full chunk, plus its first
// two scale groups.
struct Prefetch {
    u32x4 buf[kPrefetch];
    u32x4 sc0, sc1;
};

constexpr uint32_t kStep = kTileRows * 16;  // bytes of one block (or scale group) of a tile

__device__ __forceinline__ void prefetch_chunk(Prefetch &pf, rsrc_t w, rsrc_t sc, uint32_t lo)
{
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i)
        pf.buf[i] = bload(w, lo, i * kStep);
    pf.sc0 = bload(sc, lo, 0);
    pf.sc1 = bload(sc, lo, kStep);
}

// A full chunk of 32 blocks.  Loads run kPrefetch blocks ahead; the last
// iterations already load the first blocks and scale groups of the next full
// chunk this wavefront will run (wn, sn), if has_next.  Every index is a
// compile-time constant, so each table read carries its slot as an immediate
// LDS offset.  For Q1_0 the table reads of block b+1 are issued, sub-block by
// sub-block, between the fma steps of block b.
template <int FMT, int QA>
__device__ __forceinline__ void run_full_chunk(const float *__restrict__ T, const float *__restrict__ D1,
                                               const ChunkScales<FMT, QA> &cs, rsrc_t wp, rsrc_t sp, rsrc_t wn,
                                               rsrc_t sn, bool has_next, uint32_t lo, Prefetch &pf, float acc[8])
{
    u32x4 sc = pf.sc0, sc_next = pf.sc1;
    float tc[32], tn[32];
    if (FMT == BQ_Q1_0 && BQ_PIPE) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            lookups_q1(T, 0, j, pf.buf[0][j], tc + 8 * j);
    }
#pragma unroll
    for (int b = 0; b < kChunkBlocks; ++b) {
        if ((b & 7) == 0 && b > 0) {
            sc = sc_next;
            if (b / 8 + 1 < kChunkBlocks / 8)
                sc_next = bload(sp, lo, (b / 8 + 1) * kStep);
            else if (has_next)
                sc_next = bload(sn, lo, 0);
        }
        const u32x4 v = pf.buf[b % kPrefetch];
        if (b + kPrefetch < kChunkBlocks)
            pf.buf[b % kPrefetch] = bload(wp, lo, (b + kPrefetch) * kStep);
        else if (has_next)
            pf.buf[b % kPrefetch] = bload(wn, lo, (b + kPrefetch - kChunkBlocks) * kStep);
        const f32x4 d1 = cs.get(D1, b);
        float d0 = scale_of(sc, b);
        // widen once: eight v_fmac_f32 then run at full rate, where v_fma_mix_f32
        // (the compiler's choice for an f16 operand) runs at half rate
        asm volatile("" : "+v"(d0));
        if (FMT == BQ_Q1_0 && BQ_PIPE) {
            const u32x4 vn = pf.buf[(b + 1) % kPrefetch];
            float ab[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (b + 1 < kChunkBlocks)
                    lookups_q1(T, b + 1, j, vn[j], tn + 8 * j);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int L = 0; L < 8; ++L)
                    ab[L] = j == 0 ? tc[L] : __builtin_fmaf(d1[j], tc[8 * j + L], ab[L]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int L = 0; L < 8; ++L) {
                acc[L] = __builtin_fmaf(d0, ab[L], acc[L]);
                asm volatile("" : "+v"(acc[L]));
            }
#pragma unroll
            for (int i = 0; i < 32; ++i)
                tc[i] = tn[i];
        } else {
            block_math<FMT>(T, d1, b, v, d0, acc);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    pf.sc0 = sc_next;
    if (has_next)
        pf.sc1 = bload(sn, lo, kStep);
}

// A partial chunk (rows whose length is not a multiple of 32 blocks): plain
// loop, no prefetch.
template <int FMT>
__device__ void run_tail_chunk(const float *__restrict__ T, const float *__restrict__ D1, rsrc_t wp, rsrc_t sp,
                               uint32_t lo, int nbc, float acc[8])
{
    for (int b = 0; b < nbc; ++b) {
        const u32x4 v = bload(wp, lo, b * kStep);
        const u32x4 sc = bload(sp, lo, (b / 8) * kStep);
        block_math<FMT>(T, *reinterpret_cast<const f32x4 *>(D1 + 4 * b), b, v, scale_of(sc, b), acc);
    }
}

__device__ __forceinline__ void store_row(const GemvDesc &g, int tile, int lane, const float acc[8])
{
    const int row = tile * kTileRows + lane;
    const float y = ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));
    if (row < g.rows)
        g.y[row] = y;
}

// Rows [64*tile0, 64*(tile0+ntiles)) of one product; wavefront w takes tiles
// tile0 + w, tile0 + w + kWaves, ...  Rows of at most one chunk share one
// table for every tile of the item; longer rows (ntiles <= kWaves) walk the
// chunks with a table rebuild between barriers.
template <int FMT, int QA>
__device__ __forceinline__ void run_item(const GemvDesc &g, int tile0, int ntiles, float *T, float *D1)
{
    // the wavefront index is wave-uniform: say so, so that tile addresses live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int per_chunk = FMT == BQ_Q1_0 ? 128 * kChunkBlocks : 64 * kChunkBlocks;
    const int tend = tile0 + ntiles;
    const uint32_t lo = (uint32_t)lane * 16;
    auto wtile = [&](int tile, int cb) { return rsrc_of(g.bits + ((int64_t)tile * g.nb + cb) * kTileRows); };
    auto stile = [&](int tile, int cb) { return rsrc_of(g.scales + ((int64_t)tile * g.ng + cb / 8) * kTileRows); };
    float acc[8];
    Prefetch pf;

    if (g.nb <= kChunkBlocks) {
        const int nbc = g.nb;
        int tile = tile0 + wave;
        if (tile < tend && nbc == kChunkBlocks)
            prefetch_chunk(pf, wtile(tile, 0), stile(tile, 0), lo);
        if (FMT == BQ_Q1_0)
            build_table_q1<QA>(T, D1, g.q, g.d, 0, nbc);
        else
            build_table_q2<QA>(T, D1, g.q, g.d, 0, nbc);
        __syncthreads();
        ChunkScales<FMT, QA> cs;
        if (nbc == kChunkBlocks)
            cs.load(g.d);
        for (; tile < tend; tile += kWaves) {
#pragma unroll
            for (int L = 0; L < 8; ++L)
                acc[L] = 0.0f;
            const bool has_next = tile + kWaves < tend;
            if (nbc == kChunkBlocks)
                run_full_chunk<FMT, QA>(T, D1, cs, wtile(tile, 0), stile(tile, 0), wtile(tile + kWaves, 0),
                                        stile(tile + kWaves, 0), has_next, lo, pf, acc);
            else
                run_tail_chunk<FMT>(T, D1, wtile(tile, 0), stile(tile, 0), lo, nbc, acc);
            store_row(g, tile, lane, acc);
        }
        return;
    }

    const int tile = tile0 + wave;
    const bool active = tile < tend;
#pragma unroll
    for (int L = 0; L < 8; ++L)
        acc[L] = 0.0f;
    if (active)
        prefetch_chunk(pf, wtile(tile, 0), stile(tile, 0), lo);
    for (int cb = 0; cb < g.nb; cb += kChunkBlocks) {
        const int nbc = min(kChunkBlocks, g.nb - cb);
        const int k0 = (cb / kChunkBlocks) * per_chunk;
        if (cb > 0)
            __syncthreads();  // every wavefront is done with the previous table
        if (FMT == BQ_Q1_0)
            build_table_q1<QA>(T, D1, g.q, g.d, k0, nbc);
        else
            build_table_q2<QA>(T, D1, g.q, g.d, k0, nbc);
        __syncthreads();
        if (active) {
            if (nbc == kChunkBlocks) {
                ChunkScales<FMT, QA> cs;
                cs.load(g.d + k0 / QA);
                const bool has_next = cb + 2 * kChunkBlocks <= g.nb;
                run_full_chunk<FMT, QA>(T, D1, cs, wtile(tile, cb), stile(tile, cb), wtile(tile, cb + kChunkBlocks),
                                        stile(tile, cb + kChunkBlocks), has_next, lo, pf, acc);
            } else {
                run_tail_chunk<FMT>(T, D1, wtile(tile, cb), stile(tile, cb), lo, nbc, acc);
            }
        }
    }
    if (active)
        store_row(g, tile, lane, acc);
}

template <int FMT, int QA>
__global__ __launch_bounds__(kThreads) BQ_KATTR void matvec_kernel(GemvDesc g, int64_t ld_q, int64_t ld_d, int tiles)
{
    __shared__ float T[kTableFloats];
    __shared__ float D1[kScaleFloats];
    const int c = blockIdx.y;  // activation column
    g.q += c * ld_q;
    g.d += c * ld_d;
    g.y += (int64_t)c * g.rows;
    const int tile0 = blockIdx.x * kWaves;
    run_item<FMT, QA>(g, tile0, min(kWaves, tiles - tile0), T, D1);
}

template <int FMT, int QA>
__global__ __launch_bounds__(kThreads) BQ_KATTR void sweep_kernel(const GemvDesc *__restrict__ descs,
                                                         const WorkItem *__restrict__ items)
{
    __shared__ float T[kTableFloats];
    __shared__ float D1[kScaleFloats];
    const WorkItem it = items[blockIdx.x];
    const GemvDesc g = descs[it.gemv];
    run_item<FMT, QA>(g, it.tile0, it.ntiles, T, D1);
}

// ------------------------------------------------------- split single column
// For matrices with few row tiles the one-row-per-lane kernel leaves most of
// the GPU idle.  Here four wavefronts share a 64-row tile: wavefront k carries
// the chains of lane groups L = k and L = k + 4 of every row, which is the
// first pairing of the final tree, so p_k = a_k + a_(k+4) is formed in
// registers and y = (p0 + p2) + (p1 + p3) is added through LDS.  Same tables,
// same chain, same bits; each wavefront reads the whole tile payload (the four
// reads of a block hit the CU's cache) and does a quarter of the table work.
#ifndef BQ_SPLIT_MAX_TILES
#define BQ_SPLIT_MAX_TILES 1024
#endif
constexpr int kSplitMaxTiles = BQ_SPLIT_MAX_TILES;  // single-column products up to this many tiles split
constexpr int kSplit = 4;                          // wavefronts per tile
constexpr int kSplitTiles = kWaves / kSplit;       // tiles per workgroup
constexpr int kGroup = 8;                          // blocks per scale group (one 16-byte scale load)

template <int FMT>
__device__ __forceinline__ void split_block(const float *__restrict__ T, const float *__restrict__ D1, int b,
                                            u32x4 v, float d0, int k, uint32_t sh, float &acc0, float &acc1)
{
    const f32x4 d1 = *reinterpret_cast<const f32x4 *>(D1 + 4 * b);
    float ab0, ab1;
    if (FMT == BQ_Q1_0) {
        // nibble k of each word sits in byte k/2 (odd k: after a rotation by 4);
        // nibble k + 4 two bytes higher
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = __builtin_amdgcn_alignbit(v[j], v[j], sh);
            const float t0 = tab(T, b * kSlotsPerBlock + j * 8 + k, x & 0x3Cu);
            const float t1 = tab(T, b * kSlotsPerBlock + j * 8 + k + 4, (x >> 16) & 0x3Cu);
            ab0 = j == 0 ? t0 : __builtin_fmaf(d1[j], t0, ab0);
            ab1 = j == 0 ? t1 : __builtin_fmaf(d1[j], t1, ab1);
        }
    } else {
        // lane group k of sub-block j is byte k of word 2j, lane group k + 4 byte k of word 2j + 1
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float sv[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int m = 2 * j + hh;
                const uint32_t x = __builtin_amdgcn_alignbit(v[m], v[m], sh);
                const uint32_t x4 = __builtin_amdgcn_alignbit(v[m], v[m], sh + 4);
                const int slot = b * kSlotsPerBlock + m * 8 + 2 * k;
                sv[hh] = tab(T, slot, x & 0x3Cu) + tab(T, slot + 1, x4 & 0x3Cu);
            }
            ab0 = j == 0 ? d1[0] * sv[0] : __builtin_fmaf(d1[1], sv[0], ab0);
            ab1 = j == 0 ? d1[0] * sv[1] : __builtin_fmaf(d1[1], sv[1], ab1);
        }
    }
    acc0 = __builtin_fmaf(d0, ab0, acc0);
    acc1 = __builtin_fmaf(d0, ab1, acc1);
}

template <int FMT, int QA>
__global__ __launch_bounds__(kThreads) void split_kernel(GemvDesc g, int64_t ld_q, int64_t ld_d, int tiles)
{
    __shared__ float T[kTableFloats];
    __shared__ float D1[kScaleFloats];
    __shared__ float P[kSplitTiles][kSplit][64];
    const int c = blockIdx.y;  // activation column
    g.q += c * ld_q;
    g.d += c * ld_d;
    g.y += (int64_t)c * g.rows;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int tl = wave / kSplit, k = wave % kSplit;
    const int tile = blockIdx.x * kSplitTiles + tl;
    const bool live = tile < tiles;
    // a wavefront past the last tile reads tile 0 and stores nothing
    const rsrc_t wp = rsrc_of(g.bits + (int64_t)(live ? tile : 0) * g.nb * kTileRows);
    const rsrc_t sp = rsrc_of(g.scales + (int64_t)(live ? tile : 0) * g.ng * kTileRows);
    const uint32_t lo = (uint32_t)lane * 16;
    const uint32_t sh = FMT == BQ_Q1_0 ? 8u * (k >> 1) + 4u * (k & 1) : 8u * k;
    const int per_chunk = FMT == BQ_Q1_0 ? 128 * kChunkBlocks : 64 * kChunkBlocks;
    float acc0 = 0.0f, acc1 = 0.0f;

    for (int cb = 0; cb < g.nb; cb += kChunkBlocks) {
        const int nbc = min(kChunkBlocks, g.nb - cb);
        // two scale groups of payload in flight: group gi is processed while gi + 1 loads
        u32x4 pa[kGroup], pb[kGroup], sa, sb;
        auto load = [&](u32x4 (&p)[kGroup], u32x4 &s, int g0) {
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
                p[i] = bload(wp, lo, (uint32_t)min(cb + g0 + i, g.nb - 1) * kStep);
            s = bload(sp, lo, (uint32_t)((min(cb + g0, g.nb - 1)) / kGroup) * kStep);
        };
        auto run = [&](const u32x4 (&p)[kGroup], const u32x4 &s, int g0) {
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
                if (g0 + i < nbc)
                    split_block<FMT>(T, D1, g0 + i, p[i], scale_of(s, cb + g0 + i), k, sh, acc0, acc1);
        };
        load(pa, sa, 0);
        if (cb > 0)
            __syncthreads();  // every wavefront is done with the previous table
        if (FMT == BQ_Q1_0)
            build_table_q1<QA>(T, D1, g.q, g.d, (cb / kChunkBlocks) * per_chunk, nbc);
        else
            build_table_q2<QA>(T, D1, g.q, g.d, (cb / kChunkBlocks) * per_chunk, nbc);
        __syncthreads();
        for (int g0 = 0; g0 < nbc; g0 += 2 * kGroup) {
            load(pb, sb, g0 + kGroup);
            run(pa, sa, g0);
            load(pa, sa, g0 + 2 * kGroup);
            run(pb, sb, g0 + kGroup);
        }
    }
    P[tl][k][lane] = acc0 + acc1;  // p_k = a_k + a_(k+4)
    __syncthreads();
    if (k == 0 && live) {
        const int row = tile * kTileRows + lane;
        const float y = (P[tl][0][lane] + P[tl][2][lane]) + (P[tl][1][lane] + P[tl][3][lane]);
        if (row < g.rows)
            g.y[row] = y;
    }
}

// ------------------------------------------------------------ small batch
// ncols in [2, 16] activation columns against one matrix, on the matrix
// cores.  For each 32-row tile, each 16-value slice of a sub-block and each
// group of 8 columns, one v_mfma_f32_32x32x16_f16 yields the lane-group sums
// of all 32 rows x 4 lane groups x 8 columns.  A holds the slice's weights as
// f16 (Q1_0: +-1; Q2_0: -1, 0, +1, and 2 for code 3).  B is block diagonal:
// its column n = 8g + c holds column c's four activation values of lane group
// g of the slice and zeros elsewhere.  Every product and partial sum is an
// integer of magnitude at most 1024, so the f32 result is the exact integer
// sum whatever order the matrix core adds in.  The f32 chain of the
// dot-product order then runs on the vector ALU exactly as in the
// single-column kernels.
//
// Lane l of a 32x32 product holds column n = l % 32 and rows
// 8(i/4) + 4(l/32) + i%4, i = 0..15.  So lane (g, c) carries, for its 16 rows
// and column c, the chain of lane group g (slice 0) or g + 4 (slice 1).  A
// workgroup has 8 wavefronts, four 32-row tiles times the two slices; the
// pair (L, L + 4) is the first pairing of the final tree and is added across
// the two wavefronts of a tile, then ((p0 + p2) + (p1 + p3)) across lanes.
//
// Q1_0 and the int8 wrap: the order takes P(-1, -128) = -128 (int8 negation
// wraps), which no product of +-1 and -128 gives.  A -128 therefore enters B
// as 0, and -128 per such element is added back to the exact sum (still an
// exact small integer) before the chain; chunks without a -128 skip the add.
//
// Activation data reaches LDS one chunk (4 blocks) at a time and is loaded
// from global memory one chunk ahead; the weight payload is prefetched one
// chunk ahead as well.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef BQ_MF_WPE
#define BQ_MF_WPE 4  // wavefronts per SIMD the register budget is cut for
#endif
#ifndef BQ_MF_MIN_COLS
#define BQ_MF_MIN_COLS 5
#endif
// Fewer columns than this run the single-column kernel once per column (one
// grid row each): the matrix-core kernel computes 8 columns per product.
constexpr int kMfMinCols = BQ_MF_MIN_COLS;
constexpr int kMfWaves = 8;                 // 4 row tiles x 2 slices
constexpr int kMfThreads = kMfWaves * 64;
constexpr int kMfRows = 128;                // rows per workgroup (four 32-row tiles)
constexpr int kMfCols = 8;                  // activation columns per workgroup
constexpr int kMfChunk = 4;                 // blocks per LDS chunk

template <int FMT>
struct MfShape {
    static constexpr int S = FMT == BQ_Q1_0 ? 4 : 2;  // sub-blocks per block
    static constexpr int BL = 32 * S;                 // values per block
    static constexpr int CS = kMfChunk * S;           // sub-blocks per chunk
    static constexpr int TRIPLES = CS * 2 * 32;       // (sub-block, slice, column n) per chunk
    static constexpr int PER_THREAD = TRIPLES / kMfThreads;
};

// Row block and column group of this workgroup.  The launch has 8 * ceil(rb/8)
// * cgroups workgroups; ids that differ by a multiple of 8 share an XCD, so the
// column groups of one row block read its weights from one L2.
__device__ __forceinline__ void batch_place(int cgroups, int &rb, int &cg)
{
    const int id = blockIdx.x, slot = id & 7, rest = id >> 3;
    cg = rest % cgroups;
    rb = (rest / cgroups) * 8 + slot;
}

__device__ __forceinline__ uint32_t lds_word(const uint32_t *base, uint32_t byte_off)
{
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(base) + byte_off);
}

// Activation data of one chunk held by one thread between its global load
// and its LDS store.
template <int FMT>
struct MfStage {
    uint32_t q4[MfShape<FMT>::PER_THREAD];  // four int8 activation values per triple
    float d1;                               // one activation scale
    uint32_t d0;                            // one weight scale (f16 bits)
};

// Buffer resources of one workgroup's inputs.  Every load of the pipeline is
// issued unconditionally, so that the compiler can count outstanding loads
// instead of waiting for all of them; a value that does not exist is loaded
// from a valid address (offset 0) and replaced by 0.
struct MfSrc {
    rsrc_t q;   // this column group's activation quants, from column c0
    rsrc_t d;   // its activation scales
    rsrc_t sc;  // the weight scale plane from this workgroup's first 64-row tile
};

template <int FMT, int QA>
__device__ __forceinline__ void mf_stage_load(MfStage<FMT> &st, const MfSrc &src, const GemvDesc &g, int64_t ld_q,
                                              int64_t ld_d, int ncols, int c0, int row0, int cb)
{
    using S = MfShape<FMT>;
    const int tid = threadIdx.x;
    const int nsub = min(kMfChunk, g.nb - cb) * S::S;  // sub-blocks present in this chunk (may be <= 0)
    const uint32_t k0 = (uint32_t)cb * S::BL;
#pragma unroll
    for (int k = 0; k < S::PER_THREAD; ++k) {
        const int u = tid + k * kMfThreads, sb = u >> 6, t = (u >> 5) & 1, n = u & 31;
        const int gq = n >> 3, c = n & 7;
        const bool ok = c0 + c < ncols && sb < nsub;
        const uint32_t off = (uint32_t)(c * ld_q) + k0 + 32 * sb + 16 * t + 4 * gq;
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(src.q, ok ? off : 0u, 0, 0);
        st.q4[k] = ok ? v : 0u;
    }
    {
        const int sb = (tid >> 3) % S::CS, c = tid & 7;
        const bool ok = tid < S::CS * kMfCols && c0 + c < ncols && sb < nsub;
        const uint32_t off = 4 * ((uint32_t)(c * ld_d) + (k0 + 32 * sb) / QA);
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(src.d, ok ? off : 0u, 0, 0);
        st.d1 = ok ? __builtin_bit_cast(float, v) : 0.0f;
    }
    {
        // weight scale of row r of the workgroup, block cb + blk: tile r / 64 of
        // the workgroup, lane r % 64, scale group b / 8, entry b % 8
        const int blk = tid >> 7, r = tid & 127, b = cb + blk;
        const int tiles = (g.rows + kTileRows - 1) / kTileRows;
        const bool ok = b < g.nb && (row0 >> 6) + (r >> 6) < tiles;
        const uint32_t off = (((uint32_t)(r >> 6) * g.ng + b / 8) * kTileRows + (r & 63)) * 16 + (b % 8) * 2;
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(src.sc, ok ? off : 0u, 0, 0);
        st.d0 = ok ? v : 0u;
    }
}

// Writes a staged chunk into LDS; returns whether this thread saw a -128.
template <int FMT>
__device__ __forceinline__ bool mf_stage_store(const MfStage<FMT> &st, u32x4 *BF, float *WR, float *D1, float *D0)
{
    using S = MfShape<FMT>;
    const int tid = threadIdx.x;
    bool saw = false;
#pragma unroll
    for (int k = 0; k < S::PER_THREAD; ++k) {
        const int u = tid + k * kMfThreads, sb = u >> 6, t = (u >> 5) & 1, n = u & 31;
        const int gq = n >> 3;
        f16x4 v;
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int x = (int8_t)(st.q4[k] >> (8 * e));
            if (FMT == BQ_Q1_0 && x == -128) {
                x = 0;
                ++cnt;
            }
            v[e] = (_Float16)(float)x;
        }
        // the active lane of column n holds the slice's values 8(g/2)..8(g/2)+7; lane group g is half g%2
        const int lane = 32 * (gq >> 1) + n;
        char *dst = reinterpret_cast<char *>(BF + (sb * 2 + t) * 64 + lane) + 8 * (gq & 1);
        *reinterpret_cast<u32x2 *>(dst) = __builtin_bit_cast(u32x2, v);
        if (FMT == BQ_Q1_0) {
            WR[(sb * 2 + t) * 32 + n] = -128.0f * (float)cnt;
            saw |= cnt > 0;
        }
    }
    if (tid < S::CS * kMfCols)
        D1[tid] = st.d1;
    D0[tid] = f16_bits_to_f32(st.d0);
    return saw;
}

// One matrix-core product: lane-group sums of sub-block sb (of the chunk),
// slice t, for this wavefront's 32 rows and the 8 columns.  `w` holds the
// block's four payload words; `sh` the lane's byte position within a word.
template <int FMT>
__device__ __forceinline__ f32x16 mf_product(const uint32_t *XT, const u32x4 *BF, u32x4 w, int sb, int t, int lane,
                                             uint32_t sh)
{
    const int j = FMT == BQ_Q1_0 ? sb % 4 : sb % 2;  // sub-block within its block
    const uint32_t word = FMT == BQ_Q1_0 ? w[j] : (t ? w[2 * j + 1] : w[2 * j]);
    const uint32_t x = __builtin_amdgcn_alignbit(word, word, sh);
    const uint32_t x4 = __builtin_amdgcn_alignbit(word, word, sh + 4);
    u32x4 a;
    if (FMT == BQ_Q1_0) {
        // byte 2t + h of word j: its low nibble gives weights 0..3, its high nibble 4..7
        const uint32_t lo = x & 0x3Cu, hi = x4 & 0x3Cu;
        a[0] = lds_word(XT, lo);
        a[1] = lds_word(XT + 16, lo);
        a[2] = lds_word(XT, hi);
        a[3] = lds_word(XT + 16, hi);
    } else {
        // bytes 2h and 2h + 1 of word 2j + t: four nibbles of two codes each
        a[0] = lds_word(XT, x & 0x3Cu);
        a[1] = lds_word(XT, x4 & 0x3Cu);
        a[2] = lds_word(XT, (x >> 8) & 0x3Cu);
        a[3] = lds_word(XT, (x4 >> 8) & 0x3Cu);
    }
    const u32x4 bfrag = BF[(sb * 2 + t) * 64 + lane];
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, bfrag),
                                                  f32x16{}, 0, 0, 0);
}

// LDS of the small-batch kernel; the nibble tables come first so that their
// reads need no base address.
template <int FMT>
struct MfLds {
    uint32_t XT[32];                                              // nibble -> f16 weights (Q1_0: two words each)
    u32x4 BF[MfShape<FMT>::CS * 2 * 64];                          // B fragments [sub-block][slice][lane]
    float WR[FMT == BQ_Q1_0 ? MfShape<FMT>::CS * 2 * 32 : 1];     // Q1_0: -128 per wrapped element [sb][slice][n]
    float D1[MfShape<FMT>::CS * kMfCols];                         // activation scales [sb][column]
    float D0[kMfChunk * kMfRows];                                 // weight scales [block][row]
};
static_assert(sizeof(MfLds<BQ_Q2_0>::BF) >= 4 * 64 * 16 * sizeof(float), "the final reduction reuses BF");
static_assert(kMfChunk * kMfRows == kMfThreads, "one weight scale per thread and chunk");

template <int FMT, int QA>
__global__ __launch_bounds__(kMfThreads) __attribute__((amdgpu_waves_per_eu(BQ_MF_WPE))) void batch_kernel(GemvDesc g, int64_t ld_q, int64_t ld_d, int ncols,
                                                           int cgroups)
{
    using S = MfShape<FMT>;
    __shared__ MfLds<FMT> sh_;
    uint32_t *XT = sh_.XT;
    u32x4 *BF = sh_.BF;
    float *WR = sh_.WR, *D1 = sh_.D1, *D0 = sh_.D0;

    int rb, cg;
    batch_place(cgroups, rb, cg);
    const int row0 = rb * kMfRows;
    if (row0 >= g.rows)
        return;  // padding workgroup (the grid is a multiple of 8 row blocks)
    const int c0 = cg * kMfCols;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int mt = wave >> 1, t = wave & 1;
    const int h = lane >> 5, n = lane & 31, gq = n >> 3, cc = n & 7;
    const int trow0 = row0 + 32 * mt;  // first row of this wavefront's tile
    const bool live = trow0 < g.rows;
    // a wavefront past the last row reads tile 0 (any valid payload) and stores nothing
    const rsrc_t wr = rsrc_of(g.bits + (int64_t)(live ? trow0 / kTileRows : 0) * g.nb * kTileRows);
    const uint32_t voff = (uint32_t)(32 * (mt & 1) + (lane & 31)) * 16;
    MfSrc src;
    src.q = rsrc_of(reinterpret_cast<const u32x4 *>(g.q + c0 * ld_q));
    src.d = rsrc_of(reinterpret_cast<const u32x4 *>(g.d + c0 * ld_d));
    src.sc = rsrc_of(g.scales + (int64_t)(row0 / kTileRows) * g.ng * kTileRows);

    // B fragments are zero outside the active halves, which every chunk rewrites
    for (int i = tid; i < S::CS * 2 * 64; i += kMfThreads)
        BF[i] = u32x4{0u, 0u, 0u, 0u};
    if (tid < 16) {
        uint32_t lo = 0, hi = 0;
        if (FMT == BQ_Q1_0) {
            auto one = [&](int b) { return ((tid >> b) & 1) ? 0x3C00u : 0xBC00u; };
            lo = one(0) | one(1) << 16;
            hi = one(2) | one(3) << 16;
        } else {
            auto code = [&](int c) { return c == 0 ? 0xBC00u : c == 1 ? 0u : c == 2 ? 0x3C00u : 0x4000u; };
            lo = code(tid & 3) | code(tid >> 2) << 16;
        }
        XT[tid] = lo;
        XT[16 + tid] = hi;
    }

    // Activation data is staged two chunks ahead in two register sets that
    // alternate (the chunk loop is unrolled by two), and is issued before the
    // payload loads, so storing a chunk into LDS waits for neither.
    MfStage<FMT> sa, sb2;
    mf_stage_load<FMT, QA>(sa, src, g, ld_q, ld_d, ncols, c0, row0, 0);
    mf_stage_load<FMT, QA>(sb2, src, g, ld_q, ld_d, ncols, c0, row0, kMfChunk);
    u32x4 cur[kMfChunk];  // payload of the chunk; block i is reloaded for the next chunk once used
#pragma unroll
    for (int i = 0; i < kMfChunk; ++i)
        cur[i] = bload(wr, voff, (uint32_t)min(i, g.nb - 1) * kStep);
    __syncthreads();  // the zero fill is complete
    bool wrap = __syncthreads_or(mf_stage_store<FMT>(sa, BF, WR, D1, D0));
    mf_stage_load<FMT, QA>(sa, src, g, ld_q, ld_d, ncols, c0, row0, 2 * kMfChunk);

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = 0.0f;
    const uint32_t sh = FMT == BQ_Q1_0 ? 8u * (2 * t + h) : 16u * h;  // A's byte within its payload word

    // The products of chunk cb (LDS) and the payload reload for chunk cb + 1.
    auto compute = [&](int cb) {
        const int nbc = min(kMfChunk, g.nb - cb);
#pragma unroll
        for (int blk = 0; blk < kMfChunk; ++blk) {
            const u32x4 w = cur[blk];
            if (blk < nbc) {
                float ab[16];
                // products of sub-block j + 1 are issued before the chain of j
                // consumes the result of sub-block j (two results in flight)
                f32x16 s = mf_product<FMT>(XT, BF, w, blk * S::S, t, lane, sh);
#pragma unroll
                for (int j = 0; j < S::S; ++j) {
                    const int sb = blk * S::S + j;
                    f32x16 s_next;
                    if (j + 1 < S::S)
                        s_next = mf_product<FMT>(XT, BF, w, sb + 1, t, lane, sh);
                    __builtin_amdgcn_sched_barrier(0);
                    if (FMT == BQ_Q1_0 && wrap) {
                        const float wc = WR[(sb * 2 + t) * 32 + n];
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            s[i] = s[i] + wc;
                    }
                    const float d1 = D1[sb * kMfCols + cc];
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        ab[i] = j == 0 ? d1 * s[i] : __builtin_fmaf(d1, s[i], ab[i]);
                    if (j + 1 < S::S)
                        s = s_next;
                }
                // this lane's rows 8(i/4) + 4h + i%4 of the tile
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4 d0 = *reinterpret_cast<const f32x4 *>(D0 + blk * kMfRows + 32 * mt + 8 * qd + 4 * h);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[4 * qd + r] = __builtin_fmaf(d0[r], ab[4 * qd + r], acc[4 * qd + r]);
                }
            }
            // the same block of the next chunk (past the last block: the last block again, unused)
            cur[blk] = bload(wr, voff, (uint32_t)min(cb + kMfChunk + blk, g.nb - 1) * kStep);
        }
    };
    // Chunk cb + 1 goes from its register set into LDS; that set then loads chunk cb + 3.
    auto advance = [&](int cb, MfStage<FMT> &stage) {
        __syncthreads();  // every wavefront is done with chunk cb's LDS data
        wrap = __syncthreads_or(mf_stage_store<FMT>(stage, BF, WR, D1, D0));
        mf_stage_load<FMT, QA>(stage, src, g, ld_q, ld_d, ncols, c0, row0, cb + 3 * kMfChunk);
    };
    for (int cb = 0;;) {
        compute(cb);
        if (cb + kMfChunk >= g.nb)
            break;
        advance(cb, sb2);  // chunk cb + 1 was staged in sb2
        cb += kMfChunk;
        compute(cb);
        if (cb + kMfChunk >= g.nb)
            break;
        advance(cb, sa);   // chunk cb + 1 was staged in sa
        cb += kMfChunk;
    }

    // y = ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)): the slice-1 wavefront hands its
    // chains (L = g + 4) to the slice-0 wavefront of the same tile.
    __syncthreads();
    float *red = reinterpret_cast<float *>(BF) + (mt * 64 + lane) * 16;
    if (t == 1) {
#pragma unroll
        for (int i = 0; i < 16; i += 4)
            *reinterpret_cast<f32x4 *>(red + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
    }
    __syncthreads();
    if (t == 0 && live) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float p = acc[i] + red[i];     // p_g = a_g + a_(g+4)
            p = p + __shfl_xor(p, 16, 64);  // lanes g and g^2: p0 + p2, p1 + p3
            p = p + __shfl_xor(p, 8, 64);   // lanes g and g^1: (p0 + p2) + (p1 + p3)
            const int row = trow0 + 8 * (i >> 2) + 4 * h + (i & 3);
            if (gq == 0 && c0 + cc < ncols && row < g.rows)
                g.y[(int64_t)(c0 + cc) * g.rows + row] = p;
        }
    }
}

// ------------------------------------------------------------ quantizer
// Each thread quantizes 4 consecutive values; QA/4 threads share a block and
// combine their |x| maxima with butterfly shuffles (max is exact in any order).
template <int QA>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ x, int64_t n4, int8_t *__restrict__ q,
                                                       float *__restrict__ d)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (i < n4)
        v = reinterpret_cast<const f32x4 *>(x)[i];
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int off = 1; off < QA / 4; off <<= 1)
        m = fmaxf(m, __shfl_xor(m, off, 64));
    if (i >= n4)
        return;
    const float db = m / 127.0f;
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int qv = 0;
        if (db != 0.0f) {
            float r = __builtin_roundf(v[e] / db);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            qv = (int)r;
        }
        packed |= (uint32_t)(qv & 0xFF) << (8 * e);
    }
    reinterpret_cast<uint32_t *>(q)[i] = packed;
    if ((i & (QA / 4 - 1)) == 0)
        d[i / (QA / 4)] = db;
}

// ------------------------------------------------------------ validation
static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

static int hip_check(const char *fn, hipError_t e)
{
    if (e != hipSuccess)
        return set_error(BQ_EHIP, "%s: %s", fn, hipGetErrorString(e));
    return BQ_OK;
}

static int check_weights(const char *fn, const bq_weights *w, int fmt)
{
    if (!w)
        return set_error(BQ_EARG, "%s: null weights", fn);
    if (w->fmt != fmt)
        return set_error(BQ_EARG, "%s: weights format %d, expected %d", fn, (int)w->fmt, fmt);
    if (w->reserved != 0)
        return set_error(BQ_EARG, "%s: weights.reserved must be 0", fn);
    if (w->rows < 1 || w->rows >= (int64_t(1) << 31) || w->cols < 1 || w->cols >= (int64_t(1) << 31))
        return set_error(BQ_EARG, "%s: rows %lld / cols %lld out of range", fn, (long long)w->rows,
                         (long long)w->cols);
    if (w->cols % block_len(fmt))
        return set_error(BQ_EARG, "%s: cols %lld not a multiple of %d", fn, (long long)w->cols, block_len(fmt));
    if (!w->bits || !w->scales)
        return set_error(BQ_EARG, "%s: null weight plane", fn);
    if (!aligned(w->bits, 16) || !aligned(w->scales, 16))
        return set_error(BQ_EALIGN, "%s: weight planes must be 16-byte aligned", fn);
    return BQ_OK;
}

static int check_act(const char *fn, const bq_act *a, int64_t cols, int max_cols)
{
    if (!a)
        return set_error(BQ_EARG, "%s: null activation", fn);
    if (a->n != cols)
        return set_error(BQ_EARG, "%s: activation length %lld != weight cols %lld", fn, (long long)a->n,
                         (long long)cols);
    if (a->qa != 32 && a->qa != 64 && a->qa != 128)
        return set_error(BQ_EARG, "%s: qa %d not in {32, 64, 128}", fn, (int)a->qa);
    if (a->n % a->qa)
        return set_error(BQ_EARG, "%s: n %lld not a multiple of qa %d", fn, (long long)a->n, (int)a->qa);
    if (a->ncols < 1 || a->ncols > max_cols)
        return set_error(BQ_EARG, "%s: ncols %d not in [1, %d]", fn, (int)a->ncols, max_cols);
    if (!a->q || !a->d)
        return set_error(BQ_EARG, "%s: null activation pointer", fn);
    if (a->ncols > 1 && (a->ld_q < a->n || a->ld_d < a->n / a->qa))
        return set_error(BQ_EARG, "%s: leading dimensions too small", fn);
    if (!aligned(a->q, 16) || (a->ncols > 1 && a->ld_q % 16) || !aligned(a->d, 4))
        return set_error(BQ_EALIGN, "%s: q must be 16-byte aligned (ld_q a multiple of 16), d 4-byte aligned", fn);
    return BQ_OK;
}

static GemvDesc make_desc(const bq_weights *w, const bq_act *a, float *y)
{
    GemvDesc g;
    memset(&g, 0, sizeof g);
    const int64_t nb = w->cols / block_len(w->fmt);
    g.bits = static_cast<const u32x4 *>(w->bits);
    g.scales = reinterpret_cast<const u32x4 *>(w->scales);
    g.q = a->q;
    g.d = a->d;
    g.y = y;
    g.rows = (int32_t)w->rows;
    g.nb = (int32_t)nb;
    g.ng = (int32_t)groups_of(nb);
    return g;
}

template <int FMT>
static int launch_matvec(const char *fn, const bq_weights *w, const bq_act *a, float *y, bq_stream s)
{
    int rc = check_weights(fn, w, FMT);
    if (!rc)
        rc = check_act(fn, a, w->cols, 16);
    if (rc)
        return rc;
    if (!y)
        return set_error(BQ_EARG, "%s: null y", fn);
    if (!aligned(y, 4))
        return set_error(BQ_EALIGN, "%s: y must be 4-byte aligned", fn);
    const GemvDesc g = make_desc(w, a, y);
    const int tiles = (int)tiles_of(w->rows);
    hipStream_t st = static_cast<hipStream_t>(s);
    if (a->ncols >= kMfMinCols) {
        const int nc = a->ncols;
        const int cgroups = (nc + kMfCols - 1) / kMfCols;
        const int64_t rblocks = (w->rows + kMfRows - 1) / kMfRows;
        const dim3 grid((unsigned)(((rblocks + 7) / 8) * 8 * cgroups));
        switch (a->qa) {
        case 32: hipLaunchKernelGGL((batch_kernel<FMT, 32>), grid, dim3(kMfThreads), 0, st, g, a->ld_q, a->ld_d, nc, cgroups); break;
        case 64: hipLaunchKernelGGL((batch_kernel<FMT, 64>), grid, dim3(kMfThreads), 0, st, g, a->ld_q, a->ld_d, nc, cgroups); break;
        default: hipLaunchKernelGGL((batch_kernel<FMT, 128>), grid, dim3(kMfThreads), 0, st, g, a->ld_q, a->ld_d, nc, cgroups); break;
        }
        return hip_check(fn, hipGetLastError());
    }
    if (tiles <= kSplitMaxTiles) {
        const dim3 grid((tiles + kSplitTiles - 1) / kSplitTiles, a->ncols);
        switch (a->qa) {
        case 32: hipLaunchKernelGGL((split_kernel<FMT, 32>), grid, dim3(kThreads), 0, st, g, a->ld_q, a->ld_d, tiles); break;
        case 64: hipLaunchKernelGGL((split_kernel<FMT, 64>), grid, dim3(kThreads), 0, st, g, a->ld_q, a->ld_d, tiles); break;
        default: hipLaunchKernelGGL((split_kernel<FMT, 128>), grid, dim3(kThreads), 0, st, g, a->ld_q, a->ld_d, tiles); break;
        }
        return hip_check(fn, hipGetLastError());
    }
    // one grid row of workgroups per activation column
    const dim3 grid((tiles + kWaves - 1) / kWaves, a->ncols);
    switch (a->qa) {
    case 32: hipLaunchKernelGGL((matvec_kernel<FMT, 32>), grid, dim3(kThreads), 0, st, g, a->ld_q, a->ld_d, tiles); break;
    case 64: hipLaunchKernelGGL((matvec_kernel<FMT, 64>), grid, dim3(kThreads), 0, st, g, a->ld_q, a->ld_d, tiles); break;
    default: hipLaunchKernelGGL((matvec_kernel<FMT, 128>), grid, dim3(kThreads), 0, st, g, a->ld_q, a->ld_d, tiles); break;
    }
    return hip_check(fn, hipGetLastError());
}

}  // namespace bq

using namespace bq;

struct bq_sweep {
    int fmt;
    int qa;
    int nitems;
    int count;
    void *dev;  // descriptors, then work items
    const GemvDesc *descs;
    const WorkItem *items;
};

BQ_EXPORT int bq_quantize_act_q8(const float *x, int64_t n, int32_t qa, int8_t *q, float *d, bq_stream s)
{
    const char *fn = "bq_quantize_act_q8";
    if (qa != 32 && qa != 64 && qa != 128)
        return set_error(BQ_EARG, "%s: qa %d not in {32, 64, 128}", fn, (int)qa);
    if (n < 0 || n % qa)
        return set_error(BQ_EARG, "%s: n %lld is not a non-negative multiple of qa %d", fn, (long long)n, (int)qa);
    if (!x || !q || !d)
        return set_error(BQ_EARG, "%s: null pointer", fn);
    if (!aligned(x, 16) || !aligned(q, 4) || !aligned(d, 4))
        return set_error(BQ_EALIGN, "%s: x must be 16-byte aligned, q and d 4-byte aligned", fn);
    if (n == 0)
        return BQ_OK;
    const int64_t n4 = n / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    hipStream_t st = static_cast<hipStream_t>(s);
    switch (qa) {
    case 32: hipLaunchKernelGGL((quantize_kernel<32>), grid, dim3(256), 0, st, x, n4, q, d); break;
    case 64: hipLaunchKernelGGL((quantize_kernel<64>), grid, dim3(256), 0, st, x, n4, q, d); break;
    default: hipLaunchKernelGGL((quantize_kernel<128>), grid, dim3(256), 0, st, x, n4, q, d); break;
    }
    return hip_check(fn, hipGetLastError());
}

BQ_EXPORT int bq_q1_0_matvec(const bq_weights *w, const bq_act *a, float *y, bq_stream s)
{
    return launch_matvec<BQ_Q1_0>("bq_q1_0_matvec", w, a, y, s);
}

BQ_EXPORT int bq_q2_0_matvec(const bq_weights *w, const bq_act *a, float *y, bq_stream s)
{
    return launch_matvec<BQ_Q2_0>("bq_q2_0_matvec", w, a, y, s);
}

BQ_EXPORT int bq_sweep_create(const bq_gemv *list, int32_t count, bq_sweep **plan)
{
    const char *fn = "bq_sweep_create";
    if (!plan)
        return set_error(BQ_EARG, "%s: null plan pointer", fn);
    *plan = nullptr;
    if (!list || count < 1)
        return set_error(BQ_EARG, "%s: empty list", fn);
    const int fmt = list[0].w.fmt, qa = list[0].a.qa;
    std::vector<GemvDesc> descs((size_t)count);
    std::vector<WorkItem> items;
    for (int i = 0; i < count; ++i) {
        const bq_gemv &e = list[i];
        char where[96];
        snprintf(where, sizeof where, "%s: entry %d", fn, i);
        if (e.w.fmt != fmt || e.a.qa != qa)
            return set_error(BQ_EARG, "%s: every entry must share the format and qa of entry 0", where);
        int rc = check_weights(where, &e.w, fmt);
        if (!rc)
            rc = check_act(where, &e.a, e.w.cols, 1);
        if (rc)
            return rc;
        if (!e.y)
            return set_error(BQ_EARG, "%s: null y", where);
        if (!aligned(e.y, 4))
            return set_error(BQ_EALIGN, "%s: y must be 4-byte aligned", where);
        descs[(size_t)i] = make_desc(&e.w, &e.a, e.y);
        const int tiles = (int)tiles_of(e.w.rows);
        const int per_item = descs[(size_t)i].nb <= kChunkBlocks ? kWaves * kMaxRounds : kWaves;
        for (int t = 0; t < tiles; t += per_item) {
            WorkItem it;
            it.gemv = i;
            it.tile0 = t;
            it.ntiles = std::min(per_item, tiles - t);
            it.pad = 0;
            items.push_back(it);
        }
    }
    // Most work first: the hardware dispatches workgroups in order, so the
    // short items fill the tail.  The last kTailItems are cut to one tile per
    // wavefront.
    auto cost = [&](const WorkItem &w) { return (int64_t)w.ntiles * descs[(size_t)w.gemv].nb; };
    auto by_cost = [&](const WorkItem &a, const WorkItem &b) { return cost(a) > cost(b); };
    std::stable_sort(items.begin(), items.end(), by_cost);
    std::vector<WorkItem> tail;
    size_t head = items.size();
    while (head > 0 && tail.size() < (size_t)kTailItems) {
        const WorkItem w = items[--head];
        if (descs[(size_t)w.gemv].nb > kChunkBlocks || w.ntiles <= kWaves) {
            tail.push_back(w);
            continue;
        }
        for (int t = 0; t < w.ntiles; t += kWaves) {
            WorkItem piece = w;
            piece.tile0 = w.tile0 + t;
            piece.ntiles = std::min(kWaves, w.ntiles - t);
            tail.push_back(piece);
        }
    }
    std::stable_sort(tail.begin(), tail.end(), by_cost);
    std::vector<WorkItem> sorted(items.begin(), items.begin() + (ptrdiff_t)head);
    sorted.insert(sorted.end(), tail.begin(), tail.end());

    const size_t dbytes = descs.size() * sizeof(GemvDesc);
    const size_t ibytes = sorted.size() * sizeof(WorkItem);
    void *dev = nullptr;
    if (hipMalloc(&dev, dbytes + ibytes) != hipSuccess)
        return set_error(BQ_ENOMEM, "%s: hipMalloc of %zu bytes failed", fn, dbytes + ibytes);
    hipError_t e = hipMemcpy(dev, descs.data(), dbytes, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(static_cast<char *>(dev) + dbytes, sorted.data(), ibytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(dev);
        return set_error(BQ_EHIP, "%s: %s", fn, hipGetErrorString(e));
    }
    bq_sweep *p = new (std::nothrow) bq_sweep;
    if (!p) {
        (void)hipFree(dev);
        return set_error(BQ_ENOMEM, "%s: out of host memory", fn);
    }
    p->fmt = fmt;
    p->qa = qa;
    p->count = count;
    p->nitems = (int)sorted.size();
    p->dev = dev;
    p->descs = static_cast<const GemvDesc *>(dev);
    p->items = reinterpret_cast<const WorkItem *>(static_cast<char *>(dev) + dbytes);
    *plan = p;
    return BQ_OK;
}

BQ_EXPORT int bq_token_sweep(const bq_sweep *plan, bq_stream s)
{
    const char *fn = "bq_token_sweep";
    if (!plan)
        return set_error(BQ_EARG, "%s: null plan", fn);
    hipStream_t st = static_cast<hipStream_t>(s);
    const dim3 grid((unsigned)plan->nitems);
#define BQ_SWEEP(F, Q) hipLaunchKernelGGL((sweep_kernel<F, Q>), grid, dim3(kThreads), 0, st, plan->descs, plan->items)
    if (plan->fmt == BQ_Q1_0) {
        if (plan->qa == 32) BQ_SWEEP(BQ_Q1_0, 32);
        else if (plan->qa == 64) BQ_SWEEP(BQ_Q1_0, 64);
        else BQ_SWEEP(BQ_Q1_0, 128);
    } else {
        if (plan->qa == 32) BQ_SWEEP(BQ_Q2_0, 32);
        else if (plan->qa == 64) BQ_SWEEP(BQ_Q2_0, 64);
        else BQ_SWEEP(BQ_Q2_0, 128);
    }
#undef BQ_SWEEP
    return hip_check(fn, hipGetLastError());
}

BQ_EXPORT void bq_sweep_destroy(bq_sweep *plan)
{
    if (!plan)
        return;
    (void)hipDeviceSynchronize();
    (void)hipFree(plan->dev);
    delete plan;
}
