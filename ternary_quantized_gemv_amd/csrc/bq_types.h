// bq_types.h -- internal to libbq: types and sizes shared by the kernel
// sources (bq_sweep.hip, bq_cols.hip, bq_group.hip, bq_quantize.hip) and the C ABI entry
// points (bq_api.cpp).  The launchers, and the argument block of the decode
// group kernels, are declared in bq_launch.h.
//
// Every output row is computed in the dot-product order of bankML's GPU page
// ("gpu/ -- the video-card component", section "kernels.rs -- the Q1_0
// kernels"): per block, eight lanes of exact integer sums over four
// consecutive weights of each 32-weight sub-block; ab = d1*s on the first
// sub-block, ab = fma(d1, s, ab) on the others; acc = fma(d0, ab, acc); then
// the tree ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)).  All kernels are built with
// -ffp-contract=off and every fused step is an explicit fma, so the compiler
// neither fuses nor splits what that order prescribes.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "bq_layout.h"

namespace bq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkBlocks = 32;                                     // blocks per LDS table
constexpr int kSlotsPerBlock = 32;                                   // nibbles per block
constexpr int kSlotFloats = 16;                                      // entries per nibble table
constexpr int kTableFloats = kChunkBlocks * kSlotsPerBlock * kSlotFloats;  // 64 KiB
constexpr int kScaleFloats = kChunkBlocks * 4;                       // d1 per sub-block
constexpr int kWaves = 8;                                            // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kPrefetch = 4;                                         // blocks loaded ahead
// Sweep work items of single-chunk products hold up to kMaxRounds tiles per
// wavefront, all served by one table; those of longer rows kLongRounds, each
// chunk's table serving both; the last kTailItems items of the dispatch order
// are cut back to one tile per wavefront so the end of the launch drains in
// small pieces.
constexpr int kMaxRounds = 3;
constexpr int kLongRounds = 2;
constexpr int kTailItems = 1024;

constexpr uint32_t kStep = kTileRows * 16;  // bytes of one block (or scale group) of a tile

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
    const float *x;  // f32 activation, for sweeps that quantize it in the launch (q and d unused)
};

static_assert(sizeof(GemvDesc) == 64, "descriptor layout");

// A work item of a sweep: tiles tile0 .. tile0 + ntiles - 1 of product gemv;
// wavefront w takes tiles tile0 + w, tile0 + w + kWaves, ...
struct WorkItem {
    int32_t gemv;
    int32_t tile0;
    int32_t ntiles;
    int32_t pad;
};
constexpr int kSplit = 4;                     // wavefronts per tile of split_kernel
constexpr int kSplitTiles = kWaves / kSplit;  // tiles per split_kernel workgroup

}  // namespace bq
