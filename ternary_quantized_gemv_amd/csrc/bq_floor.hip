// bq_floor.hip -- the streaming-read floor: the read bandwidth HBM gives a
// plain kernel that touches every byte of a buffer once, the yardstick the
// products are compared against (bankML "par.rs -- the persistent thread
// pool and row scheduler", sections "How it is verified" and "Advantages and
// efficiency": a streaming read of a buffer far larger than the caches sets
// the memory floor of a token).
//
// 1024 workgroups of 512 threads (two per compute unit, the occupancy of the
// sweep) walk the buffer grid-stride with one 16-byte non-temporal load per
// thread per step, so at any moment the GPU streams one contiguous window of
// about 8 MiB.  Measured on MI355X this simplest form reads fastest (about
// 7.1 TB/s over 1 GiB and 4 GiB): four or eight loads in flight per thread,
// or each wavefront walking a contiguous range of its own, keep more
// requests and more DRAM rows open at once and read 4-15% slower.  The
// loaded words are folded by XOR, reduced across the wavefront and written
// once per wavefront, which keeps every load live and lets the caller check
// that every byte was read exactly once (the XOR of all sink words equals
// the XOR of all 32-bit words of the buffer).
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

constexpr int kFloorThreads = 512;

__global__ __launch_bounds__(kFloorThreads) void floor_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                              uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * kFloorThreads;
    uint32_t acc = 0;
    for (int64_t u = (int64_t)blockIdx.x * kFloorThreads + threadIdx.x; u < n16; u += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + u);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0)
        sink[(int64_t)blockIdx.x * (kFloorThreads / 64) + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_floor(const void *p, int64_t bytes, uint32_t *sink, hipStream_t st)
{
    static_assert(kFloorGrid * (kFloorThreads / 64) == kFloorSinkWords, "one sink word per wavefront");
    hipLaunchKernelGGL(floor_kernel, dim3(kFloorGrid), dim3(kFloorThreads), 0, st, static_cast<const u32x4 *>(p),
                       bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace bq
