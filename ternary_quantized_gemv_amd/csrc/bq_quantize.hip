// bq_quantize.hip -- the activation quantizer: per block of qa values,
// d = amax / 127 (optionally narrowed to an f16 value, nearest with ties to
// even) and q = round-half-away(x / d).
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

// Each thread quantizes 4 consecutive values; QA/4 threads share a block and
// combine their |x| maxima with butterfly shuffles (max is exact in any order).
template <int QA, bool F16>
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
    float db = m / 127.0f;
    if (F16)
        db = (float)(_Float16)db;  // v_cvt_f16_f32 rounds to nearest even; the widening is exact
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        packed |= (uint32_t)(quant_of(v[e], db) & 0xFF) << (8 * e);
    reinterpret_cast<uint32_t *>(q)[i] = packed;
    if ((i & (QA / 4 - 1)) == 0)
        d[i / (QA / 4)] = db;
}

template <bool F16>
static void quantize_qa(const float *x, int64_t n4, int qa, int8_t *q, float *d, hipStream_t st)
{
    const dim3 grid((unsigned)((n4 + 255) / 256));
    switch (qa) {
    case 32: hipLaunchKernelGGL((quantize_kernel<32, F16>), grid, dim3(256), 0, st, x, n4, q, d); break;
    case 64: hipLaunchKernelGGL((quantize_kernel<64, F16>), grid, dim3(256), 0, st, x, n4, q, d); break;
    default: hipLaunchKernelGGL((quantize_kernel<128, F16>), grid, dim3(256), 0, st, x, n4, q, d); break;
    }
}

hipError_t launch_quantize(const float *x, int64_t n, int qa, bool f16_scale, int8_t *q, float *d, hipStream_t st)
{
    f16_scale ? quantize_qa<true>(x, n / 4, qa, q, d, st) : quantize_qa<false>(x, n / 4, qa, q, d, st);
    return hipGetLastError();
}

}  // namespace bq
