// bq_batch.hip -- several activation columns against one matrix, on the
// matrix cores.
#include "bq_device.h"

namespace bq {

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
__global__ __launch_bounds__(kMfThreads) __attribute__((amdgpu_waves_per_eu(4))) void batch_kernel(GemvDesc g, int64_t ld_q, int64_t ld_d, int ncols,
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

template <int FMT>
static hipError_t batch_fmt(int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int ncols, hipStream_t st)
{
    const int cgroups = (ncols + kMfCols - 1) / kMfCols;
    const int64_t rblocks = (g.rows + kMfRows - 1) / kMfRows;
    const dim3 grid((unsigned)(((rblocks + 7) / 8) * 8 * cgroups));
    switch (qa) {
    case 32: hipLaunchKernelGGL((batch_kernel<FMT, 32>), grid, dim3(kMfThreads), 0, st, g, ld_q, ld_d, ncols, cgroups); break;
    case 64: hipLaunchKernelGGL((batch_kernel<FMT, 64>), grid, dim3(kMfThreads), 0, st, g, ld_q, ld_d, ncols, cgroups); break;
    default: hipLaunchKernelGGL((batch_kernel<FMT, 128>), grid, dim3(kMfThreads), 0, st, g, ld_q, ld_d, ncols, cgroups); break;
    }
    return hipGetLastError();
}

hipError_t launch_batch(int fmt, int qa, const GemvDesc &g, int64_t ld_q, int64_t ld_d, int ncols, hipStream_t st)
{
    return fmt == BQ_Q1_0 ? batch_fmt<BQ_Q1_0>(qa, g, ld_q, ld_d, ncols, st)
                          : batch_fmt<BQ_Q2_0>(qa, g, ld_q, ld_d, ncols, st);
}

}  // namespace bq
