// bq_device.h -- internal to libbq: device helpers shared by the kernel
// sources: buffer loads of the packed planes, f16 widening, and the LDS
// nibble tables that turn an activation chunk into per-nibble partial sums.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/bq.h"
#include "bq_types.h"

namespace bq {

typedef const float __attribute__((address_space(4))) *cfptr;

// Weight planes are read through buffer resources: the wave-uniform base of
// a tile sits in scalar registers, each lane adds its 16-byte offset, and the
// block offset is a scalar constant, so a load costs no vector address math.
// A resource spans kMaxTileBytes (the entry points refuse larger tiles).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t rsrc_of(const u32x4 *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(base), (short)0, (int)kMaxTileBytes, 0x00020000);
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

__device__ __forceinline__ float scale_of(u32x4 sc, int b)
{
    const uint32_t sw = sc[(b & 7) >> 1];
    return f16_bits_to_f32((b & 1) ? (sw >> 16) : (sw & 0xFFFFu));
}

// The activation quantizer's rule for one value x of a block whose scale is
// db = amax / 127: x / db (correctly rounded) rounded half away from zero,
// clamped to [-127, 127]; a zero block gives 0.
__device__ __forceinline__ int quant_of(float x, float db)
{
    if (db == 0.0f)
        return 0;
    const float r = fminf(fmaxf(__builtin_roundf(x / db), -127.0f), 127.0f);
    return (int)r;
}

// The quantizer's rule (quant_of) for the values of one activation block
// with scale db, through a reciprocal.  p = x * rcp(db) is within 2^-15 of
// x / db (|x| <= 127.0001 db, v_rcp_f32 is accurate to 1 ulp), and the
// correctly rounded x / db within 2^-18 of it, so both round to the same
// integer unless p lies within 2^-14 of a half-integer.  Those values, and
// scales too small for a safe reciprocal (or zero), take the correctly
// rounded division.  Zero comes out as +0, as quant_of's integer does.
template <int V>
__device__ __forceinline__ void quant_block(const float (&x)[V], float db, float (&q)[V])
{
    const float rdb = __builtin_amdgcn_rcpf(db);
    bool slow = !(db >= 0x1p-120f);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const float p = x[i] * rdb;
        const float a = fabsf(p);
        const float fl = floorf(a);
        const float dist = a - fl - 0.5f;  // exact wherever it decides
        slow |= fabsf(dist) <= 0x1p-14f;
        q[i] = __builtin_copysignf(dist >= 0.0f ? fl + 1.0f : fl, p) + 0.0f;
    }
    if (slow) {
#pragma unroll
        for (int i = 0; i < V; ++i)
            q[i] = (float)quant_of(x[i], db);
    }
}

// The activation quantizer's rule (quant_block: the bits of quant_of) applied to nvals values at x
// (a whole number of activation blocks, 16-byte aligned), eight per thread,
// into LDS: Qs[i] = the quant of x[i], Ds[i / QA] = the block's scale
// amax / 127.  A block's QA / 8 threads are consecutive lanes of one
// wavefront and combine their |x| maxima by butterfly shuffles (max is exact
// in any order); threads past the values take part with zeros.
template <int QA>
__device__ __forceinline__ void quantize_chunk(int8_t *Qs, float *Ds, const float *x, int nvals)
{
    constexpr int TPB = QA / 8;
    for (int t0 = 0; t0 < nvals / 8; t0 += (int)blockDim.x) {
        const int t = t0 + (int)threadIdx.x;
        const bool live = t < nvals / 8;
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, b = {0.0f, 0.0f, 0.0f, 0.0f};
        if (live) {
            a = reinterpret_cast<const f32x4 *>(x)[2 * t];
            b = reinterpret_cast<const f32x4 *>(x)[2 * t + 1];
        }
        float m = fmaxf(fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3]))),
                        fmaxf(fmaxf(fabsf(b[0]), fabsf(b[1])), fmaxf(fabsf(b[2]), fabsf(b[3]))));
#pragma unroll
        for (int off = 1; off < TPB; off <<= 1)
            m = fmaxf(m, __shfl_xor(m, off, 64));
        const float db = m / 127.0f;
        if (live) {
            const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            float qv[8];
            quant_block<8>(v, db, qv);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo |= (uint32_t)((int)qv[e] & 0xFF) << (8 * e);
                hi |= (uint32_t)((int)qv[4 + e] & 0xFF) << (8 * e);
            }
            reinterpret_cast<uint32_t *>(Qs)[2 * t] = lo;
            reinterpret_cast<uint32_t *>(Qs)[2 * t + 1] = hi;
            if (t % TPB == 0)
                Ds[t / TPB] = db;
        }
    }
}

// --------------------------------------------------------------- tables
// Each thread writes one quarter (4 entries, 16 bytes) of a slot's table per
// step, so a wavefront's stores cover 1 KiB of consecutive LDS addresses.
//
// Q1_0: slot t of a chunk covers chunk values 4t..4t+3 (block t/32, sub-block
// (t/8)%4, lane t%8).  Entry n = 4h + e: s = sum_i (bit i of n ? q_i : -q_i),
// where the negation of -128 stays -128; on sub-block 0 the entry is d1*s.
// One quarter (entries 4h .. 4h+3) of Q1_0 slot t from its four quants w4
// and, on sub-block 0, the activation scale d1.
__device__ __forceinline__ void quarter_q1(float *T, int t, int h, uint32_t w4, float d1)
{
    int p1[4], p0[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int v = (int8_t)(w4 >> (8 * i));
        p1[i] = v;
        p0[i] = v == -128 ? -128 : -v;
    }
    const int hi = ((h & 1) ? p1[2] : p0[2]) + ((h & 2) ? p1[3] : p0[3]);
    const bool first = ((t >> 3) & 3) == 0;
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int lo = ((e & 1) ? p1[0] : p0[0]) + ((e & 2) ? p1[1] : p0[1]);
        const float sf = (float)(lo + hi);
        v[e] = first ? d1 * sf : sf;
    }
    reinterpret_cast<f32x4 *>(T + t * kSlotFloats)[h] = v;
}

// A full chunk built by a workgroup of kThreads takes kIt steps per thread,
// in batches of kBatch: a batch's quants (and scales) are all requested
// before the first is used, so the build waits for memory once per batch
// rather than once per step.  (Larger batches hold more registers than two
// workgroups per CU leave.)
constexpr int kTableBatch = 4;

template <int QA>
__device__ void build_table_q1(float *T, float *D1, const int8_t *q, const float *d, int k0, int nbc)
{
    const int nquarters = nbc * kSlotsPerBlock * 4;
    constexpr int kIt = kChunkBlocks * kSlotsPerBlock * 4 / kThreads;
    if (nbc == kChunkBlocks && blockDim.x == kThreads) {
#pragma unroll
        for (int i0 = 0; i0 < kIt; i0 += kTableBatch) {
            uint32_t w4[kTableBatch];
            float d1[kTableBatch];
#pragma unroll
            for (int i = 0; i < kTableBatch; ++i) {
                const int t = (threadIdx.x + (i0 + i) * kThreads) >> 2;
                w4[i] = *reinterpret_cast<const uint32_t *>(q + k0 + 4 * t);
                d1[i] = ((t >> 3) & 3) == 0 ? d[(k0 + 4 * t) / QA] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < kTableBatch; ++i) {
                const int u = threadIdx.x + (i0 + i) * kThreads;
                quarter_q1(T, u >> 2, u & 3, w4[i], d1[i]);
            }
        }
    } else {
        for (int u = threadIdx.x; u < nquarters; u += blockDim.x) {
            const int t = u >> 2;
            const float d1 = ((t >> 3) & 3) == 0 ? d[(k0 + 4 * t) / QA] : 0.0f;
            quarter_q1(T, t, u & 3, *reinterpret_cast<const uint32_t *>(q + k0 + 4 * t), d1);
        }
    }
    for (int i = threadIdx.x; i < nbc * 4; i += blockDim.x)
        D1[i] = d[(k0 + 32 * i) / QA];
}

// Q2_0: slot t of a chunk covers chunk values 2t and 2t+1 (the low or high
// nibble of payload byte t/2 of its block).  Entry n = 4h + e holds the codes
// (e, h): (e-1)*q_2t + (h-1)*q_2t+1.
__device__ __forceinline__ void quarter_q2(float *T, int t, int h, uint32_t w2)
{
    const int qa0 = (int8_t)(w2 & 0xFF), qa1 = (int8_t)(w2 >> 8);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        v[e] = (float)((e - 1) * qa0 + (h - 1) * qa1);
    reinterpret_cast<f32x4 *>(T + t * kSlotFloats)[h] = v;
}

template <int QA>
__device__ void build_table_q2(float *T, float *D1, const int8_t *q, const float *d, int k0, int nbc)
{
    const int nquarters = nbc * kSlotsPerBlock * 4;
    constexpr int kIt = kChunkBlocks * kSlotsPerBlock * 4 / kThreads;
    if (nbc == kChunkBlocks && blockDim.x == kThreads) {
#pragma unroll
        for (int i0 = 0; i0 < kIt; i0 += kTableBatch) {
            uint32_t w2[kTableBatch];
#pragma unroll
            for (int i = 0; i < kTableBatch; ++i)
                w2[i] = *reinterpret_cast<const uint16_t *>(q + k0 + 2 * ((threadIdx.x + (i0 + i) * kThreads) >> 2));
#pragma unroll
            for (int i = 0; i < kTableBatch; ++i) {
                const int u = threadIdx.x + (i0 + i) * kThreads;
                quarter_q2(T, u >> 2, u & 3, w2[i]);
            }
        }
    } else {
        for (int u = threadIdx.x; u < nquarters; u += blockDim.x)
            quarter_q2(T, u >> 2, u & 3, *reinterpret_cast<const uint16_t *>(q + k0 + 2 * (u >> 2)));
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
    if (m == 1) {
        uint32_t r;
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
            : "=v"(r)
            : "v"(w), "v"(0x3Cu));
        return r;
    }
    return (w >> (8 * m)) & 0x3Cu;
}

}  // namespace bq
