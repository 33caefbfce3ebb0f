// bq_split.h -- internal to libbq: the four-wavefronts-per-tile walk of
// split_kernel (bq_sweep.hip).  The caller passes the function that fills the
// LDS table of a chunk.
#pragma once

#include "bq_device.h"

namespace bq {

// For matrices with few row tiles the one-row-per-lane kernel leaves most of
// the GPU idle.  Here four wavefronts share a 64-row tile: wavefront k carries
// the chains of lane groups L = k and L = k + 4 of every row, which is the
// first pairing of the final tree, so p_k = a_k + a_(k+4) is formed in
// registers and y = (p0 + p2) + (p1 + p3) is added through LDS.  Same tables,
// same chain, same bits; each wavefront reads the whole tile payload (the four
// reads of a block hit the CU's cache) and does a quarter of the table work.
constexpr int kGroup = 8;  // blocks per scale group (one 16-byte scale load)

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

// Tiles tile0 .. tile0 + ntiles - 1 of one product, kSplit wavefronts per
// tile (the workgroup has kSplit wavefronts per tile it may hold).  P holds the per-wavefront pair sums for the tree.
template <int FMT, typename Build>
__device__ __forceinline__ void run_split(const GemvDesc &g, int tile0, int ntiles, float *T, float *D1,
                                          float (*P)[kSplit][64], Build build)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int tl = wave / kSplit, k = wave % kSplit;
    const int tile = tile0 + tl;
    const bool live = tl < ntiles;
    // a wavefront past the last tile reads the first tile and stores nothing
    const rsrc_t wp = rsrc_of(g.bits + tile_block0(FMT, live ? tile : tile0, g.nb) * kTileRows);
    const rsrc_t sp = rsrc_of(g.scales + (int64_t)(live ? tile : tile0) * g.ng * kTileRows);
    const uint32_t lo = (uint32_t)lane * 16;
    const uint32_t sh = FMT == BQ_Q1_0 ? 8u * (k >> 1) + 4u * (k & 1) : 8u * k;
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
        build(cb, nbc);  // the table of blocks cb .. cb + nbc - 1
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

}  // namespace bq
