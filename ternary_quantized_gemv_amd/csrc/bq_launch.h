// bq_launch.h -- internal to libbq: the host-side kernel launchers that the
// kernel sources define and the C ABI entry points (bq_api.cpp) call.
#pragma once

#include "bq_types.h"

namespace bq {

// The products of one decode-group launch (bq_group.hip): they share the f32
// activation x, which every workgroup quantizes for itself.  Product i owns
// workgroups wg_end[i-1] .. wg_end[i] - 1 (wg_end[-1] = 0); q and d of p[i]
// are unused.
constexpr int kGroupMax = 4;
struct GroupArgs {
    GemvDesc p[kGroupMax];
    int32_t wg_end[kGroupMax];
    const float *x;
    int32_t nprod;
    int32_t rows_tpw;    // kShapeRows: row tiles per workgroup, one per wavefront (rows_tiles_per_workgroup)
    int64_t ld_q, ld_d;  // launch_wide_q8: activation columns (grid row c reads q + c ld_q, d + c ld_d)
};

// Row tiles per workgroup of the one-row-per-lane kernels (matvec_kernel,
// rows_kernel: one tile per wavefront, at most `waves`), for `total` tiles
// over all columns or products of one launch.  Up to 2048 tiles a full
// workgroup each leaves at most one workgroup per compute unit.  Beyond
// that, full workgroups would put two on some units and one on others, and
// the doubly loaded units set the time; spreading the tiles over up to 512
// workgroups (two per unit) of fewer busy wavefronts evens the load
// (151936x4096 single product, 2374 tiles: five per workgroup, Q1_0 30.0 ->
// 24.7 us, Q2_0 52-55 -> 43-45 us).  Past 4096 tiles every workgroup is full
// again.
inline int rows_tiles_per_workgroup(int64_t total, int waves)
{
    if (total <= 2048)
        return waves;
    const int64_t tpw = (total + 511) / 512;
    return tpw > waves ? waves : (int)tpw;
}

// Kernel launchers (host side).  Each validates nothing: the entry points in
// bq_api.cpp check every argument first.  They return hipGetLastError().
//
// launch_rows: one row per lane, one grid row per activation column (bq_sweep.hip).
hipError_t launch_rows(int fmt, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                       hipStream_t st);
// launch_sweep: the work items of a sweep plan (bq_sweep.hip); quantize:
// the descriptors carry f32 activations (GemvDesc::x), quantized in the launch.
hipError_t launch_sweep(int fmt, int qa, bool quantize, unsigned nitems, const GemvDesc *descs, const WorkItem *items,
                        hipStream_t st);
// launch_split: four wavefronts per 64-row tile (bq_sweep.hip).
hipError_t launch_split(int fmt, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                        hipStream_t st);
// launch_cols: ncols columns, four per workgroup, one row per lane (bq_cols.hip).
hipError_t launch_cols(int fmt, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles, int ncols,
                       hipStream_t st);
// launch_splitcols: ncols columns, four per workgroup from interleaved
// tables, several wavefronts per tile (bq_cols.hip); shape 0: eight
// wavefronts per tile, one tile per workgroup; 1, 2, 3: four wavefronts per
// tile, two, three or four tiles per workgroup.
constexpr int kSplitColsShapes = 4;
constexpr int kSplitColsTpw[kSplitColsShapes] = {1, 2, 3, 4};
hipError_t launch_splitcols(int fmt, int shape, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int tiles,
                            int ncols, hipStream_t st);
// launch_mfma: 2 to 16 columns, the lane-group sums on the matrix cores
// (bq_mfma.hip); a wavefront takes 32 rows and eight columns, all slices of
// each sub-block (shape 0) or one of the two slice halves (shape 1, twice
// the wavefronts for matrices of few rows), or 32 rows and four columns,
// whole sub-blocks (shape 2).
hipError_t launch_mfma(int fmt, int shape, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int ncols,
                       hipStream_t st);
// launch_group: a group of products sharing one f32 activation, quantized
// inside the kernel (bq_group.hip), in one of these workgroup shapes:
enum GroupShape {
    kShapeQuarter = 0,  // a quarter tile (16 rows) per sixteen-wavefront workgroup
    kShapeHalf = 1,     // half a tile (32 rows) per sixteen-wavefront workgroup
    kShapeWide = 2,     // one tile per sixteen-wavefront workgroup
    kShapeWide2 = 3,    // two tiles per sixteen-wavefront workgroup, one after the other
    kShapeRows = 4,     // up to eight tiles per workgroup (GroupArgs::rows_tpw), one per wavefront, one row per lane
    kShapeHalf3 = 5,    // three half tiles per sixteen-wavefront workgroup, one after the other
};
// The finest shape whose workgroups fit one round of the GPU's 256 compute
// units (one sixteen-wavefront workgroup each), and its workgroup count.
inline GroupShape group_shape(int64_t tiles)
{
    return tiles <= 64 ? kShapeQuarter : tiles <= 128 ? kShapeHalf : tiles <= 256 ? kShapeWide
           : tiles <= 384 ? kShapeHalf3 : tiles <= 512 ? kShapeWide2 : kShapeRows;
}
inline int64_t group_workgroups(GroupShape shape, int64_t tiles, int rows_tpw)
{
    switch (shape) {
    case kShapeQuarter: return 4 * tiles;
    case kShapeHalf: return 2 * tiles;
    case kShapeWide: return tiles;
    case kShapeWide2: return (tiles + 1) / 2;
    case kShapeHalf3: return (2 * tiles + 2) / 3;
    default: return (tiles + rows_tpw - 1) / rows_tpw;
    }
}
constexpr int kRowsWaves = 8;  // wavefronts of a kShapeRows workgroup
hipError_t launch_group(int fmt, int qa, GroupShape shape, const GroupArgs &a, hipStream_t st);
// launch_wide_q8: the wide shapes (kShapeQuarter .. kShapeWide2) for one product
// whose activation is already quantized (p[0].q, p[0].d), ncols columns.
hipError_t launch_wide_q8(int fmt, int qa, GroupShape shape, const GroupArgs &a, int ncols, hipStream_t st);
// launch_floor: the streaming read of bytes (a multiple of 16) at p, one
// sink word per wavefront of a fixed grid (bq_floor.hip).
constexpr int kFloorGrid = 1024;
constexpr int kFloorSinkWords = 8192;
hipError_t launch_floor(const void *p, int64_t bytes, uint32_t *sink, hipStream_t st);
// The fixed device scratch of bq_token_sweep_noalloc (bq_sweep.hip): the
// descriptors of up to kScratchProducts products from offset 0, the work
// items (up to kScratchItems) from kScratchItemsOffset.  One copy per GPU,
// held until the process ends.
constexpr int kScratchProducts = 1024;
constexpr int kScratchItems = 16384;
constexpr int kScratchItemsOffset = kScratchProducts * (int)sizeof(GemvDesc);
constexpr int kScratchBytes = kScratchItemsOffset + kScratchItems * (int)sizeof(WorkItem);
static_assert(kScratchItemsOffset % 256 == 0, "work items start aligned");
// The scratch's address on the current device (looked up once per device
// with hipGetSymbolAddress, then cached).
hipError_t scratch_address(void **out);
// launch_quantize: n values in blocks of qa, f32 or f16-valued scales (bq_quantize.hip).
hipError_t launch_quantize(const float *x, int64_t n, int qa, bool f16_scale, int8_t *q, float *d, hipStream_t st);

}  // namespace bq
