// bq_quantize.hip -- the activation quantizer: per block of qa values,
// d = amax / 127 and q = round-half-away(x / d).
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

// Each thread quantizes 4 consecutive values; QA/4 threads share a block and
// combine their |x| maxima with butterfly shuffles (max is exact in any order).
template <int QA>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ x, int64_t n4, int8_t *__restrict__ q,
                                                       float *__restrict__ d)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (i < n4)
        v = reinterpret_cast<const f32x4 *>(x)[i];
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int off = 1; off < QA / 4; off <<= 1)
        m = fmaxf(m, __shfl_xor(m, off, 64));
    if (i >= n4)
        return;
    const float db = m / 127.0f;
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        packed |= (uint32_t)(quant_of(v[e], db) & 0xFF) << (8 * e);
    reinterpret_cast<uint32_t *>(q)[i] = packed;
    if ((i & (QA / 4 - 1)) == 0)
        d[i / (QA / 4)] = db;
}

hipError_t launch_quantize(const float *x, int64_t n, int qa, int8_t *q, float *d, hipStream_t st)
{
    const int64_t n4 = n / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    switch (qa) {
    case 32: hipLaunchKernelGGL((quantize_kernel<32>), grid, dim3(256), 0, st, x, n4, q, d); break;
    case 64: hipLaunchKernelGGL((quantize_kernel<64>), grid, dim3(256), 0, st, x, n4, q, d); break;
    default: hipLaunchKernelGGL((quantize_kernel<128>), grid, dim3(256), 0, st, x, n4, q, d); break;
    }
    return hipGetLastError();
}

}  // namespace bq
