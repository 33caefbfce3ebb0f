// bq_sweep.hip -- the single-column kernels: one row per lane
// (matvec_kernel, one grid row per activation column), four wavefronts per
// 64-row tile (split_kernel, for matrices with few tiles), and the sweep of
// many products in one launch (sweep_kernel, one row per lane; its X form
// quantizes f32 activations chunk by chunk into LDS before each table build).
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
#include <mutex>

#include "bq_device.h"
#include "bq_launch.h"
#include "bq_split.h"

namespace bq {

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

    // the same from the chunk's scales in LDS (wave-uniform reads, then
    // scalar registers)
    __device__ __forceinline__ void load_lds(const float *d_chunk)
    {
        if (kScalar) {
#pragma unroll
            for (int i = 0; i < (kScalar ? ND : 1); ++i) {
                dv[i] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, d_chunk[i])));
                asm volatile("" : "+s"(dv[i]));
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

// The eight table reads of word m of a Q2_0 block: for lane groups beta of
// that word, the entries of its low and its high nibble, in t[2 beta] and
// t[2 beta + 1].
__device__ __forceinline__ void lookups_q2(const float *__restrict__ T, int b, int m, uint32_t wa, float t[8])
{
    const uint32_t wb = __builtin_amdgcn_alignbit(wa, wa, 4);
#pragma unroll
    for (int beta = 0; beta < 4; ++beta) {
        const int slot = b * kSlotsPerBlock + m * 8 + 2 * beta;
        t[2 * beta] = tab(T, slot, nib4(wa, beta));
        t[2 * beta + 1] = tab(T, slot + 1, nib4(wb, beta));
    }
}

// Payload words of the first kPrefetch blocks of a full chunk, plus its first
// two scale groups.
struct Prefetch {
    u32x4 buf[kPrefetch];
    u32x4 sc0, sc1;
};

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
// LDS offset.  The table reads run one payload word ahead: those of the next
// word (the next block's first, after a block's last) are issued before the
// arithmetic of the current one -- for Q1_0 a sub-block's eight entries, for
// Q2_0 the two nibble entries of each of four lane groups (0.6% off the Q2_0
// token sweep against reading each block's entries at its start).  (Q1_0's
// reads a whole block ahead measured no faster and hold 48 more registers,
// which the second tile's sums of run_item need.)
template <int FMT, int QA>
__device__ __forceinline__ void run_full_chunk(const float *__restrict__ T, const float *__restrict__ D1,
                                               const ChunkScales<FMT, QA> &cs, rsrc_t wp, rsrc_t sp, rsrc_t wn,
                                               rsrc_t sn, bool has_next, uint32_t lo, Prefetch &pf, float acc[8])
{
    u32x4 sc = pf.sc0, sc_next = pf.sc1;
    float tc[8], tn[8];
    if (FMT == BQ_Q1_0)
        lookups_q1(T, 0, 0, pf.buf[0][0], tc);
    else
        lookups_q2(T, 0, 0, pf.buf[0][0], tc);
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
        if (FMT == BQ_Q1_0) {
            float ab[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < 3)
                    lookups_q1(T, b, j + 1, v[j + 1], tn);
                else if (b + 1 < kChunkBlocks)
                    lookups_q1(T, b + 1, 0, pf.buf[(b + 1) % kPrefetch][0], tn);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int L = 0; L < 8; ++L)
                    ab[L] = j == 0 ? tc[L] : __builtin_fmaf(d1[j], tc[L], ab[L]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int L = 0; L < 8; ++L)
                    tc[L] = tn[L];
            }
#pragma unroll
            for (int L = 0; L < 8; ++L) {
                acc[L] = __builtin_fmaf(d0, ab[L], acc[L]);
                asm volatile("" : "+v"(acc[L]));
            }
        } else {
            float ab[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m < 3)
                    lookups_q2(T, b, m + 1, v[m + 1], tn);
                else if (b + 1 < kChunkBlocks)
                    lookups_q2(T, b + 1, 0, pf.buf[(b + 1) % kPrefetch][0], tn);
                __builtin_amdgcn_sched_barrier(0);
                const int j = m >> 1;
#pragma unroll
                for (int beta = 0; beta < 4; ++beta) {
                    const int L = 4 * (m & 1) + beta;
                    const float s = tc[2 * beta] + tc[2 * beta + 1];
                    ab[L] = j == 0 ? d1[0] * s : __builtin_fmaf(d1[1], s, ab[L]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int L = 0; L < 8; ++L)
                    tc[L] = tn[L];
            }
#pragma unroll
            for (int L = 0; L < 8; ++L) {
                acc[L] = __builtin_fmaf(d0, ab[L], acc[L]);
                asm volatile("" : "+v"(acc[L]));
            }
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

// The table (and D1) of the chunk of nbc blocks at value k0.  With X the
// f32 activation g.x is first quantized into LDS (Qs, Ds: the quantizer's
// bits, as bq_quantize_act_q8 would write them) and the table is built from
// there; otherwise from the quants g.q, g.d in memory.
template <int FMT, int QA, bool X>
__device__ __forceinline__ void chunk_table(const GemvDesc &g, int k0, int nbc, float *T, float *D1, int8_t *Qs,
                                            float *Ds)
{
    const int8_t *q = g.q;
    const float *d = g.d;
    int kq = k0;
    if (X) {
        quantize_chunk<QA>(Qs, Ds, g.x + k0, nbc * (FMT == BQ_Q1_0 ? 128 : 64));
        __syncthreads();
        q = Qs;
        d = Ds;
        kq = 0;
    }
    if (FMT == BQ_Q1_0)
        build_table_q1<QA>(T, D1, q, d, kq, nbc);
    else
        build_table_q2<QA>(T, D1, q, d, kq, nbc);
}

// Rows [64*tile0, 64*(tile0+ntiles)) of one product; wavefront w takes tiles
// tile0 + w, tile0 + w + kWaves, ...  Rows of at most one chunk share one
// table for every tile of the item; longer rows walk the chunks with a table
// rebuild between barriers, one tile per wavefront (ntiles <= kWaves) or,
// with PAIR, two (ntiles <= 2 * kWaves): each chunk's table then serves both
// of a wavefront's tiles, which halves the rebuilds per tile, for a second
// set of accumulators.  X: the activation is f32 and quantized chunk by chunk
// into Qs, Ds (chunk_table).
template <int FMT, int QA, bool X, bool PAIR>
__device__ __forceinline__ void run_item(const GemvDesc &g, int tile0, int ntiles, float *T, float *D1, int8_t *Qs,
                                         float *Ds)
{
    // the wavefront index is wave-uniform: say so, so that tile addresses live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int per_chunk = FMT == BQ_Q1_0 ? 128 * kChunkBlocks : 64 * kChunkBlocks;
    const int tend = tile0 + ntiles;
    const uint32_t lo = (uint32_t)lane * 16;
    auto wtile = [&](int tile, int cb) { return rsrc_of(g.bits + (tile_block0(FMT, tile, g.nb) + cb) * kTileRows); };
    auto stile = [&](int tile, int cb) { return rsrc_of(g.scales + ((int64_t)tile * g.ng + cb / 8) * kTileRows); };
    float acc[8];
    Prefetch pf;

    if (g.nb <= kChunkBlocks) {
        const int nbc = g.nb;
        int tile = tile0 + wave;
        if (tile < tend && nbc == kChunkBlocks)
            prefetch_chunk(pf, wtile(tile, 0), stile(tile, 0), lo);
        chunk_table<FMT, QA, X>(g, 0, nbc, T, D1, Qs, Ds);
        __syncthreads();
        ChunkScales<FMT, QA> cs;
        if (nbc == kChunkBlocks) {
            if (X)
                cs.load_lds(Ds);
            else
                cs.load(g.d);
        }
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

    static_assert(kLongRounds == 2, "the plan's items of longer rows hold two tiles per wavefront");
    const int tile = tile0 + wave, tile2 = tile + kWaves;
    const bool active = tile < tend, active2 = PAIR && tile2 < tend;
    float acc2[8];
#pragma unroll
    for (int L = 0; L < 8; ++L) {
        acc[L] = 0.0f;
        acc2[L] = 0.0f;
    }
    if (active)
        prefetch_chunk(pf, wtile(tile, 0), stile(tile, 0), lo);
    for (int cb = 0; cb < g.nb; cb += kChunkBlocks) {
        const int nbc = min(kChunkBlocks, g.nb - cb);
        const int k0 = (cb / kChunkBlocks) * per_chunk;
        if (cb > 0)
            __syncthreads();  // every wavefront is done with the previous table
        chunk_table<FMT, QA, X>(g, k0, nbc, T, D1, Qs, Ds);
        __syncthreads();
        if (active) {
            if (nbc == kChunkBlocks) {
                ChunkScales<FMT, QA> cs;
                if (X)
                    cs.load_lds(Ds);
                else
                    cs.load(g.d + k0 / QA);
                const bool has_next = cb + 2 * kChunkBlocks <= g.nb;
                // The wavefront's tiles in turn, through one instance of the
                // walk (two would not fit the register bound): the first
                // tile's walk prefetches the second's chunk, the last one the
                // first tile's next chunk; acc holds the walked tile's sums,
                // acc2 the other's.
#pragma unroll 1
                for (int r = 0; r < (active2 ? 2 : 1); ++r) {
                    const bool last = r == (active2 ? 1 : 0);
                    const int t = r ? tile2 : tile, tn = last ? tile : tile2;
                    const int cn = last ? cb + kChunkBlocks : cb;
                    run_full_chunk<FMT, QA>(T, D1, cs, wtile(t, cb), stile(t, cb), wtile(tn, cn), stile(tn, cn),
                                            last ? has_next : true, lo, pf, acc);
                    if (active2) {
#pragma unroll
                        for (int L = 0; L < 8; ++L) {
                            const float x = acc[L];
                            acc[L] = acc2[L];
                            acc2[L] = x;
                        }
                    }
                }
            } else {
                run_tail_chunk<FMT>(T, D1, wtile(tile, cb), stile(tile, cb), lo, nbc, acc);
                if (active2)
                    run_tail_chunk<FMT>(T, D1, wtile(tile2, cb), stile(tile2, cb), lo, nbc, acc2);
            }
        }
    }
    if (active)
        store_row(g, tile, lane, acc);
    if (active2)
        store_row(g, tile2, lane, acc2);
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
    const int tile0 = blockIdx.x * kSplitTiles;
    run_split<FMT>(g, tile0, min(kSplitTiles, tiles - tile0), T, D1, P, [&](int cb, int nbc) {
        if (FMT == BQ_Q1_0)
            build_table_q1<QA>(T, D1, g.q, g.d, cb * 128, nbc);
        else
            build_table_q2<QA>(T, D1, g.q, g.d, cb * 64, nbc);
    });
}

// Tiles tpw * blockIdx.x .. + tpw - 1 (tpw <= kWaves) of activation column
// blockIdx.y, one per wavefront.  (The second bound: see sweep_kernel.)
template <int FMT, int QA>
__global__ __launch_bounds__(kThreads, 4) void matvec_kernel(GemvDesc g, int64_t ld_q, int64_t ld_d, int tiles,
                                                             int tpw)
{
    __shared__ float T[kTableFloats];
    __shared__ float D1[kScaleFloats];
    const int c = blockIdx.y;  // activation column
    g.q += c * ld_q;
    g.d += c * ld_d;
    g.y += (int64_t)c * g.rows;
    const int tile0 = blockIdx.x * tpw;
    run_item<FMT, QA, false, false>(g, tile0, min(tpw, tiles - tile0), T, D1, nullptr, nullptr);
}

// The second bound holds every instantiation to 128 registers, four
// wavefronts per SIMD (two workgroups per CU): with activation blocks
// shorter than 128 values the chunk's activation scales come from LDS and
// the compiler would keep more of them in flight; elsewhere the table
// build's batched requests and the second tile's sums would take more than
// 128.  Under the bound some instantiations keep up to four values of the
// chunk loop in scratch (none in the block walk, and none at all in the
// qa-128 sweeps of quantized activations).
// X: the products' activations are f32 and every workgroup quantizes the
// chunks it needs (the quantizer's bits) into LDS before building its table.
template <int FMT, int QA, bool X>
__global__ __launch_bounds__(kThreads, 4) void sweep_kernel(const GemvDesc *__restrict__ descs,
                                                            const WorkItem *__restrict__ items)
{
    constexpr int kChunkValues = kChunkBlocks * (FMT == BQ_Q1_0 ? 128 : 64);
    __shared__ float T[kTableFloats];
    __shared__ float D1[kScaleFloats];
    __shared__ __attribute__((aligned(16))) int8_t Qs[X ? kChunkValues : 16];
    __shared__ float Ds[X ? kChunkValues / QA : 1];
    const WorkItem it = items[blockIdx.x];
    const GemvDesc g = descs[it.gemv];
    run_item<FMT, QA, X, true>(g, it.tile0, it.ntiles, T, D1, Qs, Ds);
}

template <int FMT>
static hipError_t rows_fmt(int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols, hipStream_t st)
{
    const int tpw = rows_tiles_per_workgroup((int64_t)tiles * ncols, kWaves);
    const dim3 grid((tiles + tpw - 1) / tpw, ncols);
    switch (qa) {
    case 32: hipLaunchKernelGGL((matvec_kernel<FMT, 32>), grid, dim3(kThreads), 0, st, g, ld_q, ld_d, tiles, tpw); break;
    case 64: hipLaunchKernelGGL((matvec_kernel<FMT, 64>), grid, dim3(kThreads), 0, st, g, ld_q, ld_d, tiles, tpw); break;
    default: hipLaunchKernelGGL((matvec_kernel<FMT, 128>), grid, dim3(kThreads), 0, st, g, ld_q, ld_d, tiles, tpw); break;
    }
    return hipGetLastError();
}

hipError_t launch_rows(int fmt, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                       hipStream_t st)
{
    return fmt == BQ_Q1_0 ? rows_fmt<BQ_Q1_0>(qa, g, ld_q, ld_d, tiles, ncols, st)
                          : rows_fmt<BQ_Q2_0>(qa, g, ld_q, ld_d, tiles, ncols, st);
}

template <int FMT, bool X>
static hipError_t sweep_fmt(int qa, unsigned nitems, const GemvDesc *descs, const WorkItem *items, hipStream_t st)
{
    const dim3 grid(nitems);
    switch (qa) {
    case 32: hipLaunchKernelGGL((sweep_kernel<FMT, 32, X>), grid, dim3(kThreads), 0, st, descs, items); break;
    case 64: hipLaunchKernelGGL((sweep_kernel<FMT, 64, X>), grid, dim3(kThreads), 0, st, descs, items); break;
    default: hipLaunchKernelGGL((sweep_kernel<FMT, 128, X>), grid, dim3(kThreads), 0, st, descs, items); break;
    }
    return hipGetLastError();
}

hipError_t launch_sweep(int fmt, int qa, bool quantize, unsigned nitems, const GemvDesc *descs, const WorkItem *items,
                        hipStream_t st)
{
    if (quantize)
        return fmt == BQ_Q1_0 ? sweep_fmt<BQ_Q1_0, true>(qa, nitems, descs, items, st)
                              : sweep_fmt<BQ_Q2_0, true>(qa, nitems, descs, items, st);
    return fmt == BQ_Q1_0 ? sweep_fmt<BQ_Q1_0, false>(qa, nitems, descs, items, st)
                          : sweep_fmt<BQ_Q2_0, false>(qa, nitems, descs, items, st);
}

// ------------------------------------------------------------ fixed scratch
// The descriptor table of bq_token_sweep_noalloc lives in this array rather
// than in an allocation.  In host code `scratch` only names the symbol; the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept per device (each GPU has its own copy).
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void **out)
{
    static std::mutex mu;
    static void *ptrs[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

template <int FMT>
static hipError_t split_fmt(int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols, hipStream_t st)
{
    const dim3 grid((tiles + kSplitTiles - 1) / kSplitTiles, ncols);
    switch (qa) {
    case 32: hipLaunchKernelGGL((split_kernel<FMT, 32>), grid, dim3(kThreads), 0, st, g, ld_q, ld_d, tiles); break;
    case 64: hipLaunchKernelGGL((split_kernel<FMT, 64>), grid, dim3(kThreads), 0, st, g, ld_q, ld_d, tiles); break;
    default: hipLaunchKernelGGL((split_kernel<FMT, 128>), grid, dim3(kThreads), 0, st, g, ld_q, ld_d, tiles); break;
    }
    return hipGetLastError();
}

hipError_t launch_split(int fmt, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                        hipStream_t st)
{
    return fmt == BQ_Q1_0 ? split_fmt<BQ_Q1_0>(qa, g, ld_q, ld_d, tiles, ncols, st)
                          : split_fmt<BQ_Q2_0>(qa, g, ld_q, ld_d, tiles, ncols, st);
}

}  // namespace bq
