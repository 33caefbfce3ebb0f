// bq_api.cpp -- the GPU entry points of the C ABI (include/bq.h): argument
// checks (before any launch; errors are return codes plus a thread-local
// message naming the call), the choice of kernel, and sweep plans.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
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
// single products).  Several columns past 512 tiles in all: four wavefronts
// per tile, one grid row per column (launch_split), up to kSplitMaxTiles
// tiles per column, above that four columns per workgroup from interleaved
// tables (launch_cols) for at least kColsMinCols columns, else one row per
// lane per column: there the per-column kernels re-stream the weights once
// per column, while on smaller matrices their extra parallelism wins.
constexpr int kSplitMaxTiles = 1024;
constexpr int kColsMinCols = 4;

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
    if (group_shape((int64_t)tiles * a->ncols) != kShapeRows) {
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

// The work items of a plan over the products descs (validated), balanced
// over the GPU, and the plan that owns their device copy.
static int make_plan(const char *fn, const std::vector<GemvDesc> &descs, int fmt, int qa, bool quantize, bq_sweep **plan)
{
    std::vector<WorkItem> items;
    for (size_t i = 0; i < descs.size(); ++i) {
        const int tiles = (int)tiles_of(descs[i].rows);
        const int per_item = descs[i].nb <= kChunkBlocks ? kWaves * kMaxRounds : kWaves;
        for (int t = 0; t < tiles; t += per_item) {
            WorkItem it;
            it.gemv = (int32_t)i;
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
    p->quantize = quantize;
    p->count = (int)descs.size();
    p->nitems = (int)sorted.size();
    p->dev = dev;
    p->descs = static_cast<const GemvDesc *>(dev);
    p->items = reinterpret_cast<const WorkItem *>(static_cast<char *>(dev) + dbytes);
    *plan = p;
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

BQ_EXPORT void bq_sweep_destroy(bq_sweep *plan)
{
    if (!plan)
        return;
    (void)hipDeviceSynchronize();
    (void)hipFree(plan->dev);
    delete plan;
}
