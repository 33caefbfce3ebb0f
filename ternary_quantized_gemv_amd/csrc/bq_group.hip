// bq_group.hip -- one group of a dependency-ordered decode step in one
// launch: the products that read the same activation (bankML "gpu/" page,
// section "Limitations": Q/K/V, and gate/up, submitted together with one wait
// per group) run from an f32 vector that each workgroup quantizes itself
// while it fills its LDS table, so a group needs no separate quantizer launch
// and the int8 vector never goes to memory.  Bits are those of
// bq_quantize_act_q8 followed by bq_q1_0_matvec / bq_q2_0_matvec.
//
// Two kernels: wide_kernel spreads the tiles of a small group over whole
// compute units (sixteen wavefronts on a quarter, a half, one or two tiles;
// the single-product entry points use it too, reading their quantized
// activation), rows_kernel walks large groups one row per lane as the token
// sweep does.
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

// Maximum over aligned groups of N lanes (exact in any order).  Within a
// 16-lane row the partners come through DPP (quad permutations, then the
// half-row and row mirrors, each of which maps a group onto its neighbour),
// across rows through ds_bpermute.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float m)
{
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, m), CTRL, 0xF, 0xF, false);
    return fmaxf(m, __builtin_bit_cast(float, o));
}

template <int N>
__device__ __forceinline__ float group_max(float m)
{
    if constexpr (N >= 2)
        m = dpp_max<0xB1>(m);  // quad_perm [1,0,3,2]
    if constexpr (N >= 4)
        m = dpp_max<0x4E>(m);  // quad_perm [2,3,0,1]
    if constexpr (N >= 8)
        m = dpp_max<0x141>(m);  // row_half_mirror
    if constexpr (N >= 16)
        m = dpp_max<0x140>(m);  // row_mirror
    if constexpr (N >= 32)
        m = fmaxf(m, __shfl_xor(m, 16, 64));
    if constexpr (N >= 64)
        m = fmaxf(m, __shfl_xor(m, 32, 64));
    return m;
}

constexpr int kScaleSlots = 4;  // scale groups held in a ring (the current one, the next, spares)

// ------------------------------------------------------------- wide tiles
// One or two 64-row tiles (RW = 64), or a half or quarter of one (RW = 32,
// 16), per workgroup of kWideWaves wavefronts, for groups with few tiles:
// the GPU has more compute units than such a group has tiles, so a tile's
// work is spread over all sixteen wavefronts of a CU, and with RW < 64 over
// several CUs.  A chunk runs in
// three phases separated by barriers:
//   A  every thread quantizes its share of the chunk's activation into the
//      LDS table (build_slot);
//   B  wavefront w computes ab, the sub-block chain of all eight lane groups,
//      of its blocks for the workgroup's rows (RW = 64: blocks 2w and 2w+1,
//      one row per lane, in turn; RW = 32: lanes 0-31 take block 2w and
//      lanes 32-63 block 2w+1 of the same 32 rows; RW = 16: wavefronts 0-7
//      take blocks 4w .. 4w+3, sixteen lanes each) and puts them in LDS;
//   C  8 * RW / 64 wavefronts, one lane per (lane group, row), extend the
//      block chain acc = fma(d0, ab, acc) over the chunk's blocks in order.
// ab values are exact functions of one block, so computing them in parallel
// changes nothing; the only sequential step, C, runs in block order as the
// dot-product order prescribes.  The next chunk's activation, payload and
// scales are requested as soon as the registers they replace are consumed.
constexpr int kWideWaves = 16;
constexpr int kWideThreads = kWideWaves * 64;
static_assert(kChunkBlocks == 2 * kWideWaves, "two blocks per wavefront and chunk (four for RW = 16)");

// Phase A of the wide kernel: thread t owns nibble slot t of the chunk
// (Q1_0: values 4t .. 4t+3; Q2_0: values 2t, 2t+1), so all sixteen
// wavefronts share the work.  XSlot holds its values until the build.
template <int FMT>
struct XSlot {
    static constexpr int V = FMT == BQ_Q1_0 ? 4 : 2;
    float v[V];
};

template <int FMT>
__device__ __forceinline__ void load_slot(XSlot<FMT> &xs, const float *__restrict__ x, int cb, int nbc, int t)
{
    constexpr int BL = FMT == BQ_Q1_0 ? 128 : 64, V = XSlot<FMT>::V;
    // past the chunk's end a thread re-reads the chunk's last slot (and drops it)
    const int v0 = min(t * V, nbc * BL - V);
    const float *xp = x + (int64_t)cb * BL + v0;
    if constexpr (FMT == BQ_Q1_0) {
        const f32x4 t = *reinterpret_cast<const f32x4 *>(xp);
#pragma unroll
        for (int i = 0; i < V; ++i)
            xs.v[i] = t[i];
    } else {
        const float2 t = *reinterpret_cast<const float2 *>(xp);
        xs.v[0] = t.x;
        xs.v[1] = t.y;
    }
}

// The wide kernel's table layout (WIDE), against the plain one of the row
// kernel, which keeps it for its registers (a second workgroup per CU):
// - Thread t stores slot t's 16 entries as four 16-byte quarters, slots 64
//   bytes apart.  Stored in the same order by every lane, the quarters of
//   eight neighbouring lanes meet four to an LDS bank; lane t stores quarter
//   (k + t/2) % 4 at step k instead, which spreads them over all banks.
//   (Padding the slots instead would push the far slots' table offsets past
//   the 16-bit immediate of the lookups.)
// - The odd blocks' slots are stored pairwise swapped (slot s of block b at
//   b*32 + (s ^ (b & 1))), so that the same slot of two neighbouring blocks
//   falls in opposite halves of the LDS banks: in the half- and quarter-tile
//   shapes a half-wavefront reads two blocks' tables at once (block_ab).
template <bool WIDE>
__device__ __forceinline__ int slot_quarter(int k, int t) { return WIDE ? (k + (t >> 1)) & 3 : k; }

template <bool WIDE>
__device__ __forceinline__ int slot_pos(int t) { return WIDE ? t ^ ((t / kSlotsPerBlock) & 1) : t; }

// The quantizer's per-block maximum (over the QA / V threads of an
// activation block, group_max), its quants, and the slot's
// 16-entry table.  Entries are sums of quants, exact in f32, formed from
// converted quants; on a Q1_0 block's first sub-block they are multiplied by
// d1 (one rounding, as the order prescribes).
template <int FMT, int QA, bool WIDE>
__device__ __forceinline__ void build_slot(float *T, float *D1, const XSlot<FMT> &xs, int nbc, int t)
{
    constexpr int V = XSlot<FMT>::V, kLanes = QA / V;
    float m = fabsf(xs.v[0]);
#pragma unroll
    for (int i = 1; i < V; ++i)
        m = fmaxf(m, fabsf(xs.v[i]));
    m = group_max<kLanes>(m);
    if (t >= nbc * kSlotsPerBlock)
        return;
    const float db = m / 127.0f;
    float f[V];
    quant_block<V>(xs.v, db, f);
    f32x4 *dst = reinterpret_cast<f32x4 *>(T + slot_pos<WIDE>(t) * kSlotFloats);
    if constexpr (FMT == BQ_Q1_0) {
        // entry 4h + e: +-q0 +-q1 by bits 0, 1 of e, +-q2 +-q3 by bits 0, 1 of h
        float lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            lo[e] = ((e & 1) ? f[0] : -f[0]) + ((e & 2) ? f[1] : -f[1]);
        // times d1 on a block's first sub-block, times 1 (exact) elsewhere
        const float s1 = ((t >> 3) & 3) == 0 ? db : 1.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int h = slot_quarter<WIDE>(k, t);
            const float hi = ((h & 1) ? f[2] : -f[2]) + ((h & 2) ? f[3] : -f[3]);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = s1 * (lo[e] + hi);
            dst[h] = v;
        }
        if ((t & 7) == 0)
            D1[t / 8] = db;
    } else {
        // entry 4h + e: (e-1) q0 + (h-1) q1
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int h = slot_quarter<WIDE>(k, t);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (float)(e - 1) * f[0] + (float)(h - 1) * f[1];
            dst[h] = v;
        }
        if ((t & 15) == 0) {
            // d1 of sub-block j of block b at D1[4b + j], j = 0, 1; 2 and 3 unused
            const int sb = t / 16;
            D1[4 * (sb >> 1) + (sb & 1)] = db;
            if ((sb & 1) == 0)
                D1[4 * (sb >> 1) + 2] = D1[4 * (sb >> 1) + 3] = 0.0f;
        }
    }
}

// Phase A from an activation that is already quantized (the single-product
// entry points on small matrices): thread t reads its slot's quants (Q1_0:
// 4, Q2_0: 2) and the scale of their activation block, and writes the same
// table build_table_q1 / build_table_q2 would (Q1_0 negation keeps -128).
struct QSlot {
    uint32_t w;
    float d;
};

template <int FMT, int QA>
__device__ __forceinline__ void load_qslot(QSlot &qs, const int8_t *__restrict__ q, const float *__restrict__ d,
                                           int cb, int nbc, int t)
{
    constexpr int BL = FMT == BQ_Q1_0 ? 128 : 64, V = FMT == BQ_Q1_0 ? 4 : 2;
    // past the chunk's end a thread re-reads the chunk's last slot (and drops it)
    const int64_t e = (int64_t)cb * BL + min(t * V, nbc * BL - V);
    if constexpr (FMT == BQ_Q1_0)
        qs.w = *reinterpret_cast<const uint32_t *>(q + e);
    else
        qs.w = *reinterpret_cast<const uint16_t *>(q + e);
    qs.d = d[e / QA];
}

template <int FMT, bool WIDE>
__device__ __forceinline__ void build_qslot(float *T, float *D1, const QSlot &qs, int nbc, int t)
{
    if (t >= nbc * kSlotsPerBlock)
        return;
    f32x4 *dst = reinterpret_cast<f32x4 *>(T + slot_pos<WIDE>(t) * kSlotFloats);
    if constexpr (FMT == BQ_Q1_0) {
        int p1[4], p0[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = (int8_t)(qs.w >> (8 * i));
            p1[i] = v;
            p0[i] = v == -128 ? -128 : -v;
        }
        const float s1 = ((t >> 3) & 3) == 0 ? qs.d : 1.0f;  // d1 on a block's first sub-block
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int h = slot_quarter<WIDE>(k, t);
            const int hi = ((h & 1) ? p1[2] : p0[2]) + ((h & 2) ? p1[3] : p0[3]);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = s1 * (float)(((e & 1) ? p1[0] : p0[0]) + ((e & 2) ? p1[1] : p0[1]) + hi);
            dst[h] = v;
        }
        if ((t & 7) == 0)
            D1[t / 8] = qs.d;
    } else {
        const int q0 = (int8_t)(qs.w & 0xFF), q1 = (int8_t)(qs.w >> 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int h = slot_quarter<WIDE>(k, t);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (float)((e - 1) * q0 + (h - 1) * q1);
            dst[h] = v;
        }
        if ((t & 15) == 0) {
            const int sb = t / 16;
            D1[4 * (sb >> 1) + (sb & 1)] = qs.d;
            if ((sb & 1) == 0)
                D1[4 * (sb >> 1) + 2] = D1[4 * (sb >> 1) + 3] = 0.0f;
        }
    }
}

// ab of the eight lane groups of chunk block B (payload v, activation scales
// d1) for the calling lane's row.  B is a constant at every call (a template
// argument or an unrolled loop index), so each table offset is an immediate.
// WIDE: the wide kernel's layout (slot_pos).  hoff_e / hoff_o are per-lane
// byte offsets into the table for even and odd slots: a further block for
// lanes that read one (half and quarter tiles), with the pairwise swap of an
// odd block's slots folded in; B itself is even there, or the lanes share it.
// LH >= 0 restricts the lane groups to half LH (0: lane groups 0-3, 1: 4-7);
// only those entries of ab are written.
template <int FMT, bool WIDE, int LH = -1>
__device__ __forceinline__ void block_ab(const float *__restrict__ T, f32x4 d1, u32x4 v, int B, uint32_t hoff_e,
                                         uint32_t hoff_o, float ab[8])
{
    // position of local slot s of block B, and the lane's offset for it
    auto pos = [&](int s) { return B * kSlotsPerBlock + (WIDE ? s ^ (B & 1) : s); };
    auto hoff = [&](int s) { return (s & 1) ? hoff_o : hoff_e; };
    if (FMT == BQ_Q1_0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t wa = v[j];
            const uint32_t wb = __builtin_amdgcn_alignbit(wa, wa, 4);
#pragma unroll
            for (int L = 0; L < 8; ++L) {
                if (LH >= 0 && (L >> 2) != LH)
                    continue;
                const float t = tab(T, pos(j * 8 + L), nib4((L & 1) ? wb : wa, L >> 1) + hoff(j * 8 + L));
                ab[L] = j == 0 ? t : __builtin_fmaf(d1[j], t, ab[L]);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (LH >= 0 && (m & 1) != LH)
                continue;  // words 0, 2 hold lane groups 0-3, words 1, 3 lane groups 4-7
            const uint32_t wa = v[m];
            const uint32_t wb = __builtin_amdgcn_alignbit(wa, wa, 4);
            const int j = m >> 1;
#pragma unroll
            for (int beta = 0; beta < 4; ++beta) {
                const int L = 4 * (m & 1) + beta;
                const int s0 = m * 8 + 2 * beta;
                const float sv = tab(T, pos(s0), nib4(wa, beta) + hoff(s0)) + tab(T, pos(s0 + 1), nib4(wb, beta) + hoff(s0 + 1));
                ab[L] = j == 0 ? d1[0] * sv : __builtin_fmaf(d1[1], sv, ab[L]);
            }
        }
    }
}

// Rows of 8 lane groups per block in the wide kernel's AB array, padded to 9
// for quarter tiles: there a wavefront's phase-B stores go to four blocks
// (16 lanes each), and 128-float blocks would put the two blocks of each
// half-wavefront in the same LDS banks; 144 floats put them 16 banks apart.
constexpr int ab_rows(int rw) { return rw == 16 ? 9 : 8; }

// Phase B for the wavefront whose first block is WB: with RW = 64 its lanes
// (rows) take blocks WB and WB + 1 in turn; with RW = 32 or 16 the lanes
// split into 64 / RW groups of RW rows, group h taking block WB + h; with
// RW = 16 two wavefronts share those four blocks, LH = 0 taking lane groups
// 0-3 and LH = 1 lane groups 4-7 (each ab depends on its own lane group
// only), so that all sixteen wavefronts work.
template <int FMT, int WB, int RW, int LH = -1>
__device__ __forceinline__ void phase_b(const float *__restrict__ T, const float *__restrict__ D1,
                                        float (*AB)[ab_rows(RW)][RW], const u32x4 (&v)[2], int nbc, int lane)
{
    static_assert(WB < kChunkBlocks, "a block for every wavefront");
    float ab[8];
    if (RW == 64) {
        if (WB < nbc) {
            block_ab<FMT, true>(T, *reinterpret_cast<const f32x4 *>(D1 + 4 * WB), v[0], WB, 0u, 0u, ab);
#pragma unroll
            for (int L = 0; L < 8; ++L)
                AB[WB][L][lane] = ab[L];
        }
        if (WB + 1 < nbc) {
            block_ab<FMT, true>(T, *reinterpret_cast<const f32x4 *>(D1 + 4 * WB + 4), v[1], WB + 1, 0u, 0u, ab);
#pragma unroll
            for (int L = 0; L < 8; ++L)
                AB[WB + 1][L][lane] = ab[L];
        }
    } else {
        const int h = lane / RW, r = lane % RW;
        if (WB + h < nbc) {
            // block WB + h; WB is even, so the block is odd (its slots swapped) when h is
            static_assert(WB % 2 == 0, "the wavefront's first block is even");
            const uint32_t hoff = (uint32_t)h * (kSlotsPerBlock * kSlotFloats * 4);
            const uint32_t swap = (h & 1) ? kSlotFloats * 4 : 0u;
            block_ab<FMT, true, LH>(T, *reinterpret_cast<const f32x4 *>(D1 + 4 * (WB + h)), v[0], WB, hoff + swap,
                                    hoff - swap, ab);
#pragma unroll
            for (int L = 0; L < 8; ++L)
                if (LH < 0 || (L >> 2) == LH)
                    AB[WB + h][L][r] = ab[L];
        }
    }
}

template <int FMT, int QA, int RW, int TPW, bool Q8>
__global__ __launch_bounds__(kWideThreads) void wide_kernel(GroupArgs a)
{
    static_assert(RW == 64 || RW == 32 || TPW == 1, "several units per workgroup: whole or half tiles");
    constexpr int kParts = kTileRows / RW;           // workgroups per tile
    constexpr int kChainWaves = 8 * RW / 64;
    constexpr int kBPW = RW == 64 ? 2 : 64 / RW;     // first block of wavefront w: kBPW * (w % kBWaves)
    constexpr int kBWaves = kChunkBlocks / kBPW;     // wavefronts per set of the chunk's blocks (8 for RW = 16)
    __shared__ float T[kTableFloats];
    // half tiles in turn (RW = 32, TPW > 1): two ab buffers, so that unit
    // t + 1's phase B (buffer (t + 1) & 1) needs no barrier after unit t's
    // phase C (buffer t & 1); 128.5 KiB of LDS with the table
    constexpr int kABBufs = RW == 32 && TPW > 1 ? 2 : 1;
    __shared__ float AB[kABBufs * kChunkBlocks][ab_rows(RW)][RW];
    __shared__ float D1[kScaleFloats];
    const int wg = blockIdx.x;
    GemvDesc g = a.p[0];
    int wg0 = 0;
#pragma unroll
    for (int i = 1; i < kGroupMax; ++i)
        if (i < a.nprod && wg >= a.wg_end[i - 1]) {
            g = a.p[i];
            wg0 = a.wg_end[i - 1];
        }
    if (Q8) {  // grid row c: activation column c
        const int c = blockIdx.y;
        g.q += c * a.ld_q;
        g.d += c * a.ld_d;
        g.y += (int64_t)c * g.rows;
    }
    const int tiles = (g.rows + kTileRows - 1) / kTileRows;
    // the workgroup's units (RW rows each) in turn: unit t is part upart(t) of tile utile(t)
    const int unit0 = (wg - wg0) * TPW;
    auto utile = [&](int t) { return (unit0 + t) / kParts; };
    auto upart = [&](int t) { return (unit0 + t) % kParts; };
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int h = lane / RW, r = lane % RW;  // half-wave and row of this lane (h = 0 when RW = 64)
    auto ulo = [&](int t) { return (uint32_t)(upart(t) * RW + r) * 16; };
    const int nb = g.nb, ng = g.ng;
    // a tile past the product's last one re-reads the last tile and stores nothing
    auto wtile = [&](int t) { return rsrc_of(g.bits + tile_block0(FMT, min(utile(t), tiles - 1), g.nb) * kTileRows); };
    auto stile = [&](int t) { return rsrc_of(g.scales + (int64_t)min(utile(t), tiles - 1) * g.ng * kTileRows); };

    // Requests in the order of use (vector memory counts complete in order);
    // all unconditional, clamped to the row's last block / scale group.
    XSlot<FMT> xs;
    QSlot qs;
    auto load_a = [&](int cb, int nbc, int t) {
        if constexpr (Q8)
            load_qslot<FMT, QA>(qs, g.q, g.d, cb, nbc, t);
        else
            load_slot<FMT>(xs, a.x, cb, nbc, t);
    };
    auto build_a = [&](int nbc, int t) {
        if constexpr (Q8)
            build_qslot<FMT, true>(T, D1, qs, nbc, t);
        else
            build_slot<FMT, QA, true>(T, D1, xs, nbc, t);
    };
    u32x4 v[2], sc[kChunkBlocks / kScalesPerGroup];
    auto request = [&](int t, int cb) {
        const rsrc_t wp = wtile(t);
        if (RW == 64) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                v[i] = bload(wp, ulo(t), (uint32_t)min(cb + 2 * wave + i, nb - 1) * kStep);
        } else {
            v[0] = bload(wp, ulo(t) + (uint32_t)min(cb + kBPW * (wave % kBWaves) + h, nb - 1) * kStep, 0);
        }
    };
    auto request_scales = [&](int t, int cb) {
        const rsrc_t sp = stile(t);
#pragma unroll
        for (int j = 0; j < kChunkBlocks / kScalesPerGroup; ++j)
            sc[j] = bload(sp, ulo(t), (uint32_t)min(cb / kScalesPerGroup + j, ng - 1) * kStep);
    };
    const int slot = threadIdx.x;
    load_a(0, min(kChunkBlocks, nb), slot);
    __builtin_amdgcn_sched_barrier(0);
    request(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    request_scales(0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // chain wavefronts: one lane per (lane group L, row r), one accumulator per tile
    const int L = (wave * 64 + lane) / RW;
    float acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        acc[t] = 0.0f;
    for (int cb = 0; cb < nb; cb += kChunkBlocks) {
        const int nbc = min(kChunkBlocks, nb - cb);
        const int nx = cb + kChunkBlocks < nb ? cb + kChunkBlocks : cb;  // the last chunk re-reads itself
        // A
        build_a(nbc, slot);
        __syncthreads();
        load_a(nx, min(kChunkBlocks, nb - nx), slot);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            // the unit after (tile t, this chunk): the next tile, or the first tile of the next chunk
            const int tn = t + 1 < TPW ? t + 1 : 0, cn = t + 1 < TPW ? cb : nx;
            float(*ABt)[ab_rows(RW)][RW] = AB + (kABBufs == 2 ? (t & 1) * kChunkBlocks : 0);
            // B (wavefront-uniform dispatch, so that every table offset is a constant)
            switch (wave) {
#define BQ_PHASE_B(w) \
    case w: phase_b<FMT, kBPW * ((w) % kBWaves), RW, (RW == 16 ? (w) / kBWaves : -1)>(T, D1, ABt, v, nbc, lane); break;
                BQ_PHASE_B(0) BQ_PHASE_B(1) BQ_PHASE_B(2) BQ_PHASE_B(3) BQ_PHASE_B(4) BQ_PHASE_B(5)
                BQ_PHASE_B(6) BQ_PHASE_B(7) BQ_PHASE_B(8) BQ_PHASE_B(9) BQ_PHASE_B(10) BQ_PHASE_B(11)
                BQ_PHASE_B(12) BQ_PHASE_B(13) BQ_PHASE_B(14) BQ_PHASE_B(15)
#undef BQ_PHASE_B
            default: break;
            }
            request(tn, cn);
            __syncthreads();
            // C
            if (wave < kChainWaves) {
                // all reads first, then the chain; blocks past a short last chunk
                // leave acc unchanged (a select, so the reads need no branches)
                float abv[kChunkBlocks];
#pragma unroll
                for (int b = 0; b < kChunkBlocks; ++b)
                    abv[b] = ABt[b][L][r];
#pragma unroll
                for (int b = 0; b < kChunkBlocks; ++b) {
                    const float next = __builtin_fmaf(scale_of(sc[b / kScalesPerGroup], b), abv[b], acc[t]);
                    acc[t] = b < nbc ? next : acc[t];
                }
            }
            request_scales(tn, cn);
            if (t + 1 < TPW && kABBufs == 1)
                __syncthreads();  // this phase C reads AB before the next tile's phase B writes it
            // after the last tile: the next chunk's phase A writes only T and D1,
            // and its barrier orders this phase C before the next phase B
        }
    }
    // the units' eight lane accumulators through AB (slot t for unit t),
    // then wavefront t forms unit t's tree
    static_assert(TPW <= kChunkBlocks && TPW <= kWideWaves, "one AB slot and one wavefront per unit");
    __syncthreads();  // every phase C has read AB
    if (wave < kChainWaves) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            AB[t][L][r] = acc[t];
    }
    __syncthreads();
    if (wave < TPW && lane < RW && utile(wave) < tiles) {
        const int t = wave;
        const int row = utile(t) * kTileRows + upart(t) * RW + lane;
        const float y = ((AB[t][0][lane] + AB[t][4][lane]) + (AB[t][2][lane] + AB[t][6][lane])) +
                        ((AB[t][1][lane] + AB[t][5][lane]) + (AB[t][3][lane] + AB[t][7][lane]));
        if (row < g.rows)
            g.y[row] = y;
    }
}

// -------------------------------------------------------------- row tiles
// Large groups (the LM head): one row per lane and one tile per wavefront,
// a.rows_tpw (at most eight) tiles per workgroup, walked as the token sweep
// walks them -- every lane carries the eight lane accumulators of its row
// through all blocks in order.  The workgroup builds each chunk's table from
// x (two slots per thread, every wavefront taking part) once for its tiles;
// payload requests run kRowsDepth blocks ahead across chunk ends.
constexpr int kRowsThreads = kRowsWaves * 64;
constexpr int kRowsDepth = 4;
static_assert(kChunkBlocks * kSlotsPerBlock == 2 * kRowsThreads, "two table slots per thread");

template <int FMT, int QA>
__global__ __launch_bounds__(kRowsThreads) void rows_kernel(GroupArgs a)
{
    __shared__ float T[kTableFloats];
    __shared__ float D1[kScaleFloats];
    const int wg = blockIdx.x;
    GemvDesc g = a.p[0];
    int wg0 = 0;
#pragma unroll
    for (int i = 1; i < kGroupMax; ++i)
        if (i < a.nprod && wg >= a.wg_end[i - 1]) {
            g = a.p[i];
            wg0 = a.wg_end[i - 1];
        }
    const int tiles = (g.rows + kTileRows - 1) / kTileRows;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // wavefronts past rows_tpw only help build the tables; a wavefront past
    // the product's last tile re-reads it and stores nothing
    const bool busy = wave < a.rows_tpw;
    const int tile = (wg - wg0) * a.rows_tpw + wave;
    const int tl = min(tile, tiles - 1);
    const rsrc_t wp = rsrc_of(g.bits + tile_block0(FMT, tl, g.nb) * kTileRows);
    const rsrc_t sp = rsrc_of(g.scales + (int64_t)tl * g.ng * kTileRows);
    const uint32_t lo = (uint32_t)lane * 16;
    const int nb = g.nb, ng = g.ng;
    const int s0 = threadIdx.x, s1 = threadIdx.x + kRowsThreads;

    // Requests in the order of use, all unconditional and clamped to the row.
    XSlot<FMT> x0, x1;
    u32x4 p[kRowsDepth], sc[kScaleSlots];
    load_slot<FMT>(x0, a.x, 0, min(kChunkBlocks, nb), s0);
    load_slot<FMT>(x1, a.x, 0, min(kChunkBlocks, nb), s1);
    __builtin_amdgcn_sched_barrier(0);
    if (busy) {
#pragma unroll
        for (int b = 0; b < kRowsDepth; ++b) {
            if (b % kScalesPerGroup == 0)
                sc[(b / kScalesPerGroup) % kScaleSlots] =
                    bload(sp, lo, (uint32_t)min(b / kScalesPerGroup, ng - 1) * kStep);
            p[b] = bload(wp, lo, (uint32_t)min(b, nb - 1) * kStep);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    float acc[8];
#pragma unroll
    for (int L = 0; L < 8; ++L)
        acc[L] = 0.0f;
    // block i of the chunk at cb: the chain step, then the request kRowsDepth ahead
    auto step = [&](int cb, int i) {
        float ab[8];
        block_ab<FMT, false>(T, *reinterpret_cast<const f32x4 *>(D1 + 4 * i), p[i % kRowsDepth], i, 0u, 0u, ab);
        float d0 = scale_of(sc[(i / kScalesPerGroup) % kScaleSlots], i);
        asm volatile("" : "+v"(d0));  // widen once, then full-rate fmas
#pragma unroll
        for (int L = 0; L < 8; ++L)
            acc[L] = __builtin_fmaf(d0, ab[L], acc[L]);
    };
    auto ahead = [&](int cb, int i) {
        const int b = cb + i + kRowsDepth;
        if ((i + kRowsDepth) % kScalesPerGroup == 0)
            sc[((i + kRowsDepth) / kScalesPerGroup) % kScaleSlots] = bload(sp, lo, (uint32_t)min(b / kScalesPerGroup, ng - 1) * kStep);
        p[i % kRowsDepth] = bload(wp, lo, (uint32_t)min(b, nb - 1) * kStep);
    };
    for (int cb = 0; cb < nb; cb += kChunkBlocks) {
        const int nbc = min(kChunkBlocks, nb - cb);
        const int nx = cb + kChunkBlocks < nb ? cb + kChunkBlocks : cb;  // the last chunk re-reads itself
        if (cb > 0)
            __syncthreads();  // every wavefront is done with the previous table
        // (without the rotation: its registers would cost the second workgroup per CU)
        build_slot<FMT, QA, false>(T, D1, x0, nbc, s0);
        build_slot<FMT, QA, false>(T, D1, x1, nbc, s1);
        __syncthreads();
        load_slot<FMT>(x0, a.x, nx, min(kChunkBlocks, nb - nx), s0);
        load_slot<FMT>(x1, a.x, nx, min(kChunkBlocks, nb - nx), s1);
        if (!busy)
            continue;
        if (nbc == kChunkBlocks) {
#pragma unroll
            for (int i = 0; i < kChunkBlocks; ++i) {
                step(cb, i);
                ahead(cb, i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kChunkBlocks; ++i) {
                if (i < nbc)
                    step(cb, i);
                ahead(cb, i);
            }
        }
    }
    const int row = tile * kTileRows + lane;
    if (busy && tile < tiles && row < g.rows)
        g.y[row] = ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));
}

template <int FMT>
static void rows_qa(int qa, const GroupArgs &a, hipStream_t st)
{
    const dim3 grid(a.wg_end[a.nprod - 1]), block(kRowsThreads);
    switch (qa) {
    case 32: hipLaunchKernelGGL((rows_kernel<FMT, 32>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((rows_kernel<FMT, 64>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((rows_kernel<FMT, 128>), grid, block, 0, st, a); break;
    }
}

template <int FMT, int RW, int TPW, bool Q8>
static void wide_qa(int qa, const GroupArgs &a, int ncols, hipStream_t st)
{
    const dim3 grid(a.wg_end[a.nprod - 1], ncols), block(kWideThreads);
    switch (qa) {
    case 32: hipLaunchKernelGGL((wide_kernel<FMT, 32, RW, TPW, Q8>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((wide_kernel<FMT, 64, RW, TPW, Q8>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((wide_kernel<FMT, 128, RW, TPW, Q8>), grid, block, 0, st, a); break;
    }
}

hipError_t launch_group(int fmt, int qa, GroupShape shape, const GroupArgs &a, hipStream_t st)
{
    const bool q1 = fmt == BQ_Q1_0;
    switch (shape) {
    case kShapeQuarter: q1 ? wide_qa<BQ_Q1_0, 16, 1, false>(qa, a, 1, st) : wide_qa<BQ_Q2_0, 16, 1, false>(qa, a, 1, st); break;
    case kShapeHalf: q1 ? wide_qa<BQ_Q1_0, 32, 1, false>(qa, a, 1, st) : wide_qa<BQ_Q2_0, 32, 1, false>(qa, a, 1, st); break;
    case kShapeWide: q1 ? wide_qa<BQ_Q1_0, 64, 1, false>(qa, a, 1, st) : wide_qa<BQ_Q2_0, 64, 1, false>(qa, a, 1, st); break;
    case kShapeHalf3: q1 ? wide_qa<BQ_Q1_0, 32, 3, false>(qa, a, 1, st) : wide_qa<BQ_Q2_0, 32, 3, false>(qa, a, 1, st); break;
    case kShapeWide2: q1 ? wide_qa<BQ_Q1_0, 64, 2, false>(qa, a, 1, st) : wide_qa<BQ_Q2_0, 64, 2, false>(qa, a, 1, st); break;
    default: q1 ? rows_qa<BQ_Q1_0>(qa, a, st) : rows_qa<BQ_Q2_0>(qa, a, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_wide_q8(int fmt, int qa, GroupShape shape, const GroupArgs &a, int ncols, hipStream_t st)
{
    const bool q1 = fmt == BQ_Q1_0;
    if (shape == kShapeQuarter)
        q1 ? wide_qa<BQ_Q1_0, 16, 1, true>(qa, a, ncols, st) : wide_qa<BQ_Q2_0, 16, 1, true>(qa, a, ncols, st);
    else if (shape == kShapeHalf)
        q1 ? wide_qa<BQ_Q1_0, 32, 1, true>(qa, a, ncols, st) : wide_qa<BQ_Q2_0, 32, 1, true>(qa, a, ncols, st);
    else if (shape == kShapeWide)
        q1 ? wide_qa<BQ_Q1_0, 64, 1, true>(qa, a, ncols, st) : wide_qa<BQ_Q2_0, 64, 1, true>(qa, a, ncols, st);
    else if (shape == kShapeHalf3)
        q1 ? wide_qa<BQ_Q1_0, 32, 3, true>(qa, a, ncols, st) : wide_qa<BQ_Q2_0, 32, 3, true>(qa, a, ncols, st);
    else
        q1 ? wide_qa<BQ_Q1_0, 64, 2, true>(qa, a, ncols, st) : wide_qa<BQ_Q2_0, 64, 2, true>(qa, a, ncols, st);
    return hipGetLastError();
}

}  // namespace bq
