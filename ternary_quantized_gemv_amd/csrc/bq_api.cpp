// bq_api.cpp -- the GPU entry points of the C ABI (include/bq.h): argument
// checks (before any launch; errors are return codes plus a thread-local
// message naming the call), the choice of kernel, and sweep plans.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/bq.h"
#include "bq_layout.h"
#include "bq_launch.h"
#include "bq_types.h"

namespace bq {

// Kernel choice (measured on MI355X).  bq_group_matvec, and
// bq_q1_0_matvec / bq_q2_0_matvec counting the tiles of all activation
// columns together: group_shape() picks the finest workgroup shape whose
// workgroups fit one round of the 256 compute units -- a quarter, half a
// tile, one tile or two tiles per sixteen-wavefront workgroup (wide_kernel,
// a tile's blocks spread over the whole CU; one grid row per column) up to
// 512 tiles, beyond that one row per lane with up to eight tiles per
// workgroup (rows_kernel for groups; matvec_kernel, the sweep's walk, for
// single products).  Several columns past 512 tiles in all: on matrices of
// up to kSplitMaxTiles tiles, the split-columns kernel (several wavefronts
// per tile, four columns per workgroup from interleaved tables; shape by
// splitcols_shape), one stream of the weights per group of four columns; on
// taller matrices four columns per workgroup one row per lane
// (launch_cols) for at least kColsMinCols columns, else one row per lane
// per column.
constexpr int kSplitMaxTiles = 1024;
constexpr int kColsMinCols = 4;

// Shape of the split-columns kernel for ncols >= 2 columns on `tiles` row
// tiles (at most kSplitMaxTiles): the first of eight wavefronts per tile
// with one tile per workgroup, then four per tile with two, three or four
// tiles, whose workgroups (row blocks times groups of four columns) fit one
// round of the 256 compute units; failing that four wavefronts per tile and
// two tiles per workgroup.  Measured on MI355X (us, event-timed replays of
// ~1 GB of weight copies; shapes 0 / 1 / 2 / 3, the rule's choice first):
//   Q1_0 12288x4096  N = 4    10.9: 10.9 / 13.6 / 16.4 / 19.3
//                    N = 8    13.6: 15.8 / 13.6 / 16.6 / 19.3
//                    N = 16   16.7: 23.1 / 20.6 / 16.7 / 19.5
//   Q2_0 12288x4096  N = 4 / 8 / 16     20.0 / 22.0 / 27.0 (shapes 0 / 1 / 2, each the fastest)
//   Q1_0 44800x1024  N = 2 / 4 / 16     6.8 / 7.1 / 18.2 (2 / 2 / 1, each the fastest)
//   Q1_0 20000x4096  N = 16   29.6: 35.7 / 29.6 / 31.6 / 36.7
//   Q1_0 65536x1024  N = 4 / 8          8.2 / 13.7 (3 / 1, each the fastest)
// Against one grid row per column the tables' single stream of the weights
// per four columns gained 1.7-9x (Q1_0 65536x1024 N = 8: 57.2 -> 13.7).
// (Measured with 8-block table chunks; launches whose workgroups fit one
// round, on rows of more than 8 blocks, now take 16-block chunks: Q1_0 12288x4096 N = 4 / 8 / 16 10.9 /
// 13.7 / 17.1 -> 10.6 / 13.5 / 16.7, Q2_0 20.1 / 21.9 / 27.2 -> 19.2 /
// 22.0 / 26.8.)
static int splitcols_shape(int tiles, int ncols)
{
    const int64_t cgroups = (ncols + 3) / 4;
    auto wgs = [&](int s) { return (int64_t)((tiles + kSplitColsTpw[s] - 1) / kSplitColsTpw[s]) * cgroups; };
    for (int s = 0; s < kSplitColsShapes; ++s)
        if (wgs(s) <= 256)
            return s;
    return 1;
}

// The small batch on the matrix cores (launch_mfma) or on the table kernels
// above.  Shapes of the matrix-core kernel: 0, eight columns per workgroup,
// both slice halves of 32 rows in one wavefront (measured faster on tall
// matrices); 1, eight columns, the two halves in two wavefronts (twice the
// wavefronts, for matrices of up to kSplitMaxTiles tiles); 2, four columns,
// whole sub-blocks (two accumulating MFMAs each; no padded outputs below
// five columns).  BQ_BATCH_AUTO takes the matrix cores where they measured
// faster (MI355X, us, event-timed replays of ~1 GB of weight copies;
// tables / matrix cores):
//   Q1_0 151936x4096  N = 2 / 4 / 8 / 16   45.3 / 48.9 / 76.6 / 136.2, 69.3 / 65.4 / 92.3 / 167.4
//   Q1_0 12288x4096   N = 2 / 4 / 8 / 16   9.1 / 10.9 / 14.2 / 17.4, 23.7 / 23.7 / 19.8 / 25.3
//   Q1_0 44800x1024   N = 4 / 8 / 16       7.1 / 11.8 / 19.7, 10.5 / 10.4 / 18.5
//   Q2_0 151936x4096  N = 2 / 4 / 8 / 16   87.4 / 87.5 / 145.0 / 267.9, 74.4 / 74.4 / 92.2 / 164.9
//   Q2_0 65536x1024   N = 2 / 8 / 16       12.2 / 21.2 / 38.3, 11.9 / 15.1 / 26.6
//   Q2_0 12288x4096   N = 2 / 4 / 8 / 16   15.1 / 20.1 / 22.3 / 28.6, 28.6 / 28.7 / 26.5 / 30.9
//   Q2_0 20000x4096   N = 4 / 12 / 16      22.5 / 34.5 / 52.6, 29.0 / 39.1 / 37.9
// so: Q1_0 always on the tables (the shapes with 4096 columns are faster
// there at every N, the others within 13%); Q2_0 on the matrix cores from
// kSplitMaxTiles tiles on, or where the tables' work items (tiles times
// groups of four columns) exceed kSplitMaxTiles.  Returns the shape, or -1
// for the tables.  BQ_BATCH_MFMA takes the matrix cores from 2 columns on,
// BQ_BATCH_TABLES never.
static std::atomic<int> g_batch_path{BQ_BATCH_AUTO};

static int mfma_choice(int fmt, int tiles, int ncols)
{
    const bool tall = tiles > kSplitMaxTiles;
    const int shape = ncols <= 4 ? 2 : tall ? 0 : 1;
    if (ncols < 2)
        return -1;
    const int path = g_batch_path.load(std::memory_order_relaxed);
    if (path != BQ_BATCH_AUTO)
        return path == BQ_BATCH_MFMA ? shape : -1;
    if (fmt == BQ_Q1_0)
        return -1;
    const int64_t items = (int64_t)tiles * ((ncols + 3) / 4);
    return tiles >= kSplitMaxTiles || items > kSplitMaxTiles ? shape : -1;
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
    if (w->rows < 1 || w->rows >= kMaxDim || w->cols < 1 || w->cols >= kMaxDim)
        return set_error(BQ_EARG, "%s: rows %lld / cols %lld out of range", fn, (long long)w->rows,
                         (long long)w->cols);
    if (w->cols % block_len(fmt))
        return set_error(BQ_EARG, "%s: cols %lld not a multiple of %d", fn, (long long)w->cols, block_len(fmt));
    if (!tile_fits(w->cols / block_len(fmt)))
        return set_error(BQ_EARG, "%s: cols %lld: a 64-row tile's payload would exceed %lld bytes", fn,
                         (long long)w->cols, (long long)kMaxTileBytes);
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
    hipError_t e;
    const int mshape = mfma_choice(FMT, tiles, a->ncols);
    if (mshape >= 0) {
        e = launch_mfma(FMT, mshape, a->qa, g, a->ld_q, a->ld_d, a->ncols, st);
    } else if (group_shape((int64_t)tiles * a->ncols) != kShapeRows) {
        // the shape is chosen for all columns together (grid row c = column c)
        GroupArgs args;
        memset(&args, 0, sizeof args);
        const GroupShape shape = group_shape((int64_t)tiles * a->ncols);
        args.p[0] = g;
        args.wg_end[0] = (int32_t)group_workgroups(shape, tiles, kRowsWaves);  // a wide shape: rows_tpw unused
        args.nprod = 1;
        args.ld_q = a->ld_q;
        args.ld_d = a->ld_d;
        e = launch_wide_q8(FMT, a->qa, shape, args, a->ncols, st);
    } else if (a->ncols >= kColsMinCols && tiles > kSplitMaxTiles)
        e = launch_cols(FMT, a->qa, g, a->ld_q, a->ld_d, tiles, a->ncols, st);
    else if (a->ncols >= 2 && tiles <= kSplitMaxTiles)
        e = launch_splitcols(FMT, splitcols_shape(tiles, a->ncols), a->qa, g, a->ld_q, a->ld_d, tiles, a->ncols, st);
    else if (tiles <= kSplitMaxTiles)
        e = launch_split(FMT, a->qa, g, a->ld_q, a->ld_d, tiles, a->ncols, st);
    else
        e = launch_rows(FMT, a->qa, g, a->ld_q, a->ld_d, tiles, a->ncols, st);
    return hip_check(fn, e);
}

}  // namespace bq

using namespace bq;

struct bq_sweep {
    int fmt;
    int qa;
    bool quantize;  // f32 activations, quantized in the launch (bq_sweep_create_x)
    int nitems;
    int count;
    void *dev;  // descriptors, then work items
    const GemvDesc *descs;
    const WorkItem *items;
};

static int quantize_entry(const char *fn, const float *x, int64_t n, int32_t qa, bool f16_scale, int8_t *q,
                          float *d, bq_stream s)
{
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
    return hip_check(fn, launch_quantize(x, n, qa, f16_scale, q, d, static_cast<hipStream_t>(s)));
}

BQ_EXPORT int bq_quantize_act_q8(const float *x, int64_t n, int32_t qa, int8_t *q, float *d, bq_stream s)
{
    return quantize_entry("bq_quantize_act_q8", x, n, qa, false, q, d, s);
}

BQ_EXPORT int bq_quantize_act_q8_f16(const float *x, int64_t n, int32_t qa, int8_t *q, float *d, bq_stream s)
{
    return quantize_entry("bq_quantize_act_q8_f16", x, n, qa, true, q, d, s);
}

BQ_EXPORT int bq_read_floor(const void *p, int64_t bytes, uint32_t *sink, bq_stream s)
{
    const char *fn = "bq_read_floor";
    static_assert(kFloorSinkWords == BQ_FLOOR_SINK_WORDS, "sink size of the header");
    if (!p || !sink)
        return set_error(BQ_EARG, "%s: null pointer", fn);
    if (bytes <= 0 || bytes % 16)
        return set_error(BQ_EARG, "%s: bytes %lld is not a positive multiple of 16", fn, (long long)bytes);
    if (!aligned(p, 16) || !aligned(sink, 4))
        return set_error(BQ_EALIGN, "%s: p must be 16-byte aligned, sink 4-byte aligned", fn);
    return hip_check(fn, launch_floor(p, bytes, sink, static_cast<hipStream_t>(s)));
}

BQ_EXPORT int bq_q1_0_matvec(const bq_weights *w, const bq_act *a, float *y, bq_stream s)
{
    return launch_matvec<BQ_Q1_0>("bq_q1_0_matvec", w, a, y, s);
}

BQ_EXPORT int bq_set_batch_path(int path)
{
    if (path != BQ_BATCH_AUTO && path != BQ_BATCH_TABLES && path != BQ_BATCH_MFMA)
        return set_error(BQ_EARG, "bq_set_batch_path: path %d unknown", path), -1;
    return g_batch_path.exchange(path);
}

BQ_EXPORT int bq_q2_0_matvec(const bq_weights *w, const bq_act *a, float *y, bq_stream s)
{
    return launch_matvec<BQ_Q2_0>("bq_q2_0_matvec", w, a, y, s);
}

BQ_EXPORT int bq_group_matvec(const bq_weights *w, int32_t count, const float *x, int32_t qa, float *const *y,
                              bq_stream s)
{
    const char *fn = "bq_group_matvec";
    if (!w || !y)
        return set_error(BQ_EARG, "%s: null weights or outputs", fn);
    if (count < 1 || count > kGroupMax)
        return set_error(BQ_EARG, "%s: count %d not in [1, %d]", fn, (int)count, kGroupMax);
    if (qa != 32 && qa != 64 && qa != 128)
        return set_error(BQ_EARG, "%s: qa %d not in {32, 64, 128}", fn, (int)qa);
    if (!x)
        return set_error(BQ_EARG, "%s: null x", fn);
    if (!aligned(x, 16))
        return set_error(BQ_EALIGN, "%s: x must be 16-byte aligned", fn);
    const int fmt = w[0].fmt;
    if (fmt != BQ_Q1_0 && fmt != BQ_Q2_0)
        return set_error(BQ_EARG, "%s: weights format %d unknown", fn, fmt);
    GroupArgs args;
    memset(&args, 0, sizeof args);
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
        char where[96];
        snprintf(where, sizeof where, "%s: product %d", fn, i);
        const int rc = check_weights(where, &w[i], fmt);
        if (rc)
            return rc;
        if (w[i].cols != w[0].cols)
            return set_error(BQ_EARG, "%s: cols %lld differ from product 0's %lld", where, (long long)w[i].cols,
                             (long long)w[0].cols);
        if (!y[i])
            return set_error(BQ_EARG, "%s: null y", where);
        if (!aligned(y[i], 4))
            return set_error(BQ_EALIGN, "%s: y must be 4-byte aligned", where);
        tiles += tiles_of(w[i].rows);
    }
    if (w[0].cols % qa)
        return set_error(BQ_EARG, "%s: cols %lld not a multiple of qa %d", fn, (long long)w[0].cols, (int)qa);
    const GroupShape shape = group_shape(tiles);
    args.rows_tpw = rows_tiles_per_workgroup(tiles, kRowsWaves);
    int64_t wgs = 0;
    for (int i = 0; i < count; ++i) {
        bq_act none;
        memset(&none, 0, sizeof none);
        args.p[i] = make_desc(&w[i], &none, y[i]);
        wgs += group_workgroups(shape, tiles_of(w[i].rows), args.rows_tpw);
        if (wgs >= (int64_t(1) << 31))
            return set_error(BQ_EARG, "%s: too many rows", fn);
        args.wg_end[i] = (int32_t)wgs;
    }
    args.x = x;
    args.nprod = count;
    return hip_check(fn, launch_group(fmt, qa, shape, args, static_cast<hipStream_t>(s)));
}

// The work items of a sweep over the products descs[0..n) (validated),
// balanced over the GPU, written to out (room for cap items; tmp has room
// for cap more).  Returns the number of items, or -1 if cap is too small.
// Allocates nothing, so the no-allocation entry point can use it on fixed
// storage.  Order: most work first -- the hardware dispatches workgroups in
// order, so the short items fill the tail; the last kTailItems are cut to
// one tile per wavefront.  Ties keep the order items were made in (the
// sequence number rides in WorkItem::pad while sorting).
static int plan_items(const GemvDesc *descs, int n, WorkItem *out, WorkItem *tmp, int cap)
{
    int m = 0;
    for (int i = 0; i < n; ++i) {
        const int tiles = (int)tiles_of(descs[i].rows);
        const int per_item = kWaves * (descs[i].nb <= kChunkBlocks ? kMaxRounds : kLongRounds);
        for (int t = 0; t < tiles; t += per_item) {
            if (m >= cap)
                return -1;
            out[m] = WorkItem{(int32_t)i, t, std::min(per_item, tiles - t), m};
            ++m;
        }
    }
    auto cost = [&](const WorkItem &w) { return (int64_t)w.ntiles * descs[w.gemv].nb; };
    auto before = [&](const WorkItem &a, const WorkItem &b) {
        const int64_t ca = cost(a), cb = cost(b);
        return ca != cb ? ca > cb : a.pad < b.pad;
    };
    std::sort(out, out + m, before);
    int head = m, nt = 0;
    while (head > 0 && nt < kTailItems) {
        const WorkItem w = out[--head];
        if (w.ntiles <= kWaves) {
            if (nt >= cap)
                return -1;
            tmp[nt] = w;
            tmp[nt].pad = nt;
            ++nt;
            continue;
        }
        for (int t = 0; t < w.ntiles; t += kWaves) {
            if (nt >= cap)
                return -1;
            tmp[nt] = WorkItem{w.gemv, w.tile0 + t, std::min(kWaves, w.ntiles - t), nt};
            ++nt;
        }
    }
    std::sort(tmp, tmp + nt, before);
    if (head + nt > cap)
        return -1;
    for (int k = 0; k < nt; ++k)
        out[head + k] = tmp[k];
    for (int k = 0; k < head + nt; ++k)
        out[k].pad = 0;
    return head + nt;
}

// A plan over the products descs (validated) that owns the device copy of
// its descriptors and work items.
static int make_plan(const char *fn, const std::vector<GemvDesc> &descs, int fmt, int qa, bool quantize, bq_sweep **plan)
{
    // the tail cut leaves at most one item per kWaves tiles of a product
    size_t cap = 0;
    for (const GemvDesc &g : descs)
        cap += (size_t)((tiles_of(g.rows) + kWaves - 1) / kWaves);
    std::vector<WorkItem> items(cap + 1), tmp(cap + 1);
    const int nitems = plan_items(descs.data(), (int)descs.size(), items.data(), tmp.data(), (int)cap + 1);
    if (nitems < 0)
        return set_error(BQ_EARG, "%s: too many work items", fn);
    const size_t dbytes = descs.size() * sizeof(GemvDesc);
    const size_t ibytes = (size_t)nitems * sizeof(WorkItem);
    void *dev = nullptr;
    if (hipMalloc(&dev, dbytes + ibytes) != hipSuccess)
        return set_error(BQ_ENOMEM, "%s: hipMalloc of %zu bytes failed", fn, dbytes + ibytes);
    hipError_t e = hipMemcpy(dev, descs.data(), dbytes, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(static_cast<char *>(dev) + dbytes, items.data(), ibytes, hipMemcpyHostToDevice);
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
    p->quantize = quantize;
    p->count = (int)descs.size();
    p->nitems = nitems;
    p->dev = dev;
    p->descs = static_cast<const GemvDesc *>(dev);
    p->items = reinterpret_cast<const WorkItem *>(static_cast<char *>(dev) + dbytes);
    *plan = p;
    return BQ_OK;
}

// One entry of a bq_gemv list, checked against the list's format and qa,
// as its descriptor.
static int gemv_entry(const char *fn, int i, const bq_gemv &e, int fmt, int qa, GemvDesc *out)
{
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
    *out = make_desc(&e.w, &e.a, e.y);
    return BQ_OK;
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
    for (int i = 0; i < count; ++i) {
        const int rc = gemv_entry(fn, i, list[i], fmt, qa, &descs[(size_t)i]);
        if (rc)
            return rc;
    }
    return make_plan(fn, descs, fmt, qa, false, plan);
}

BQ_EXPORT int bq_sweep_create_x(const bq_gemv_x *list, int32_t count, int32_t qa, bq_sweep **plan)
{
    const char *fn = "bq_sweep_create_x";
    if (!plan)
        return set_error(BQ_EARG, "%s: null plan pointer", fn);
    *plan = nullptr;
    if (!list || count < 1)
        return set_error(BQ_EARG, "%s: empty list", fn);
    if (qa != 32 && qa != 64 && qa != 128)
        return set_error(BQ_EARG, "%s: qa %d not in {32, 64, 128}", fn, (int)qa);
    const int fmt = list[0].w.fmt;
    std::vector<GemvDesc> descs((size_t)count);
    for (int i = 0; i < count; ++i) {
        const bq_gemv_x &e = list[i];
        char where[96];
        snprintf(where, sizeof where, "%s: entry %d", fn, i);
        if (e.w.fmt != fmt)
            return set_error(BQ_EARG, "%s: every entry must share the format of entry 0", where);
        const int rc = check_weights(where, &e.w, fmt);
        if (rc)
            return rc;
        if (e.w.cols % qa)
            return set_error(BQ_EARG, "%s: cols %lld not a multiple of qa %d", where, (long long)e.w.cols, (int)qa);
        if (!e.x || !e.y)
            return set_error(BQ_EARG, "%s: null x or y", where);
        if (!aligned(e.x, 16) || !aligned(e.y, 4))
            return set_error(BQ_EALIGN, "%s: x must be 16-byte aligned, y 4-byte aligned", where);
        bq_act none;
        memset(&none, 0, sizeof none);
        descs[(size_t)i] = make_desc(&e.w, &none, e.y);
        descs[(size_t)i].x = e.x;
    }
    return make_plan(fn, descs, fmt, qa, true, plan);
}

BQ_EXPORT int bq_token_sweep(const bq_sweep *plan, bq_stream s)
{
    const char *fn = "bq_token_sweep";
    if (!plan)
        return set_error(BQ_EARG, "%s: null plan", fn);
    return hip_check(fn, launch_sweep(plan->fmt, plan->qa, plan->quantize, (unsigned)plan->nitems, plan->descs, plan->items,
                                      static_cast<hipStream_t>(s)));
}

// bq_token_sweep_noalloc: the plan is built on fixed host storage (one call
// at a time, under g_stage_mu) and copied into the library's fixed device
// scratch (bq_sweep.hip), so nothing is allocated on the host or the device.
static std::mutex g_stage_mu;
alignas(256) static unsigned char g_stage[kScratchBytes];
static WorkItem g_tmp[kScratchItems];

BQ_EXPORT int bq_token_sweep_noalloc(const bq_gemv *list, int32_t count, bq_stream s)
{
    const char *fn = "bq_token_sweep_noalloc";
    if (!list || count < 1)
        return set_error(BQ_EARG, "%s: empty list", fn);
    if (count > kScratchProducts)
        return set_error(BQ_EARG, "%s: %d products exceed the fixed scratch's %d", fn, (int)count, kScratchProducts);
    std::lock_guard<std::mutex> lock(g_stage_mu);
    GemvDesc *descs = reinterpret_cast<GemvDesc *>(g_stage);
    WorkItem *items = reinterpret_cast<WorkItem *>(g_stage + kScratchItemsOffset);
    const int fmt = list[0].w.fmt, qa = list[0].a.qa;
    for (int i = 0; i < count; ++i) {
        const int rc = gemv_entry(fn, i, list[i], fmt, qa, &descs[i]);
        if (rc)
            return rc;
    }
    const int nitems = plan_items(descs, count, items, g_tmp, kScratchItems);
    if (nitems < 0)
        return set_error(BQ_EARG, "%s: the products need more than the fixed scratch's %d work items", fn,
                         kScratchItems);
    unsigned char *ptr = nullptr;
    int rc = hip_check(fn, scratch_address(reinterpret_cast<void **>(&ptr)));
    if (rc)
        return rc;
    hipStream_t st = static_cast<hipStream_t>(s);
    // one copy of the used part: descriptors from offset 0, work items from
    // kScratchItemsOffset (pageable source: the call returns once it is staged)
    const size_t used = (size_t)kScratchItemsOffset + (size_t)nitems * sizeof(WorkItem);
    rc = hip_check(fn, hipMemcpyAsync(ptr, g_stage, used, hipMemcpyHostToDevice, st));
    if (rc)
        return rc;
    return hip_check(fn, launch_sweep(fmt, qa, false, (unsigned)nitems, reinterpret_cast<const GemvDesc *>(ptr),
                                      reinterpret_cast<const WorkItem *>(ptr + kScratchItemsOffset), st));
}

BQ_EXPORT void bq_sweep_destroy(bq_sweep *plan)
{
    if (!plan)
        return;
    (void)hipDeviceSynchronize();
    (void)hipFree(plan->dev);
    delete plan;
}
