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
// Tables cover a chunk of 4 blocks: 4 x 32 slots x 16 entries x 16 bytes =
// 32 KiB, rebuilt between barriers.  A workgroup is four wavefronts, one
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
constexpr int kColsSlotBytes = 16 * kColsNC * 4;
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

// Tables of one chunk for columns c0 .. c0+3 (zeros for columns >= ncols).
// Q1_0 slot t covers chunk values 4t..4t+3 (block t/32, sub-block (t/8)%4,
// lane group t%8); entry n: sum_i (bit i of n ? q_i : wrap8(-q_i)), times d1
// on sub-block 0.  Q2_0 slot t covers values 2t, 2t+1; entry n = 4h + e:
// (e-1)*q_2t + (h-1)*q_2t+1.
template <int FMT, int QA>
__device__ void build_cols(f32x4 *T, float *D1, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int c0, int ncols,
                           int k0, int nbc)
{
    constexpr int S = FMT == BQ_Q1_0 ? 4 : 2;
    constexpr int kThreadsHere = kColsWaves * 64;
    constexpr int kIters = kColsChunk * kSlotsPerBlock * 4 * kColsNC / kThreadsHere;
    // unit u = (slot t, quarter h, column c): entries 4h..4h+3 of column c.
    // All of a thread's loads are issued before any is used.
    const int nunits = nbc * kSlotsPerBlock * 4 * kColsNC;
    float *Tf = reinterpret_cast<float *>(T);
    uint32_t wq[kIters];
    float d1[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int u = threadIdx.x + it * kThreadsHere;
        const int c = u % kColsNC, t = u / (4 * kColsNC);
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
        const int c = u % kColsNC, h = (u / kColsNC) & 3, t = u / (4 * kColsNC);
        float v[4];
        if (FMT == BQ_Q1_0) {
            int p1[4], p0[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int x = (int8_t)(wq[it] >> (8 * i));
                p1[i] = x;
                p0[i] = x == -128 ? -128 : -x;
            }
            const int hi = ((h & 1) ? p1[2] : p0[2]) + ((h & 2) ? p1[3] : p0[3]);
            const bool first = ((t >> 3) & 3) == 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int lo = ((e & 1) ? p1[0] : p0[0]) + ((e & 2) ? p1[1] : p0[1]);
                const float sf = (float)(lo + hi);
                v[e] = first ? d1[it] * sf : sf;
            }
        } else {
            const int qa0 = (int8_t)(wq[it] & 0xFF), qa1 = (int8_t)(wq[it] >> 8);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (float)((e - 1) * qa0 + (h - 1) * qa1);
        }
        // a column past ncols loaded zeros: its entries are 0 (Q1_0 d1 = 0 on sub-block 0, and
        // the integer sums of zero quants are 0)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Tf[(t * 16 + 4 * h + e) * kColsNC + c] = v[e];
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
    __shared__ f32x4 T[kColsChunk * kSlotsPerBlock * 16];
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
    const rsrc_t wp = rsrc_of(g.bits + (int64_t)(live ? tile : rb * kColsWaves) * g.nb * kTileRows);
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

}  // namespace bq
