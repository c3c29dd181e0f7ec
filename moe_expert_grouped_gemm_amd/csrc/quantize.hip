// quantize.hip -- OCP-MX quantisation of a bf16 matrix along its rows:
// bf16 [rows, cols] -> E4M3 [rows, cols] or E2M1 x2 [rows, cols/2], plus one
// E8M0 scale byte per 32 consecutive values.
//
// Streaming kernel: four lanes share one 32-value block (8 values = 16 bytes
// each, so a wave reads 1 KiB of consecutive input per load), the block's
// largest magnitude is combined with two lane shuffles, and every step of
// the conversion is integer arithmetic on the bf16 bits (common.hpp), so
// the result is exact and identical for every launch shape.
#include "common.hpp"
#include "launch.hpp"

namespace ptgg {

namespace {

template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(const uint16_t *__restrict__ x,
                                                               uint8_t *__restrict__ q,
                                                               uint8_t *__restrict__ scales,
                                                               int64_t nquads)
{
    constexpr int EMAX = FMT == 0 ? 8 : 2;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < nquads; t += stride) {
        // t indexes 8-value groups; the group's block is t / 4
        const uintx4 v = *(const uintx4 *)(x + t * 8);
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[2 * i] = v[i] & 0xFFFFu;
            h[2 * i + 1] = v[i] >> 16;
        }
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = max(amax, h[i] & 0x7FFFu);
        // the four lanes of a block are consecutive lanes 4j..4j+3
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 64));
        const uint32_t E = mx_scale_byte<EMAX>(amax);
        if (FMT == 0) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w0 |= mx_encode<0>(h[i], E) << (8 * i);
                w1 |= mx_encode<0>(h[4 + i], E) << (8 * i);
            }
            *(uintx2 *)(q + t * 8) = uintx2{w0, w1};
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) w |= mx_encode<1>(h[i], E) << (4 * i);
            *(uint32_t *)(q + t * 4) = w;
        }
        if ((t & 3) == 0) scales[t >> 2] = (uint8_t)E;
    }
}

}  // namespace

hipError_t launch_quantize(const uint16_t *x, uint8_t *q, uint8_t *scales, int64_t rows, int64_t cols,
                           int fmt, hipStream_t s)
{
    const int64_t nquads = rows * cols / 8;
    if (nquads == 0) return hipSuccess;
    // whole blocks per workgroup (256 lanes = 64 blocks), a few waves per SIMD
    int64_t grid = (nquads + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cus() * 16;
    if (grid > cap) grid = cap;
    if (fmt == 0)
        hipLaunchKernelGGL(mx_quantize_kernel<0>, dim3((unsigned)grid), dim3(kThreads), 0, s, x, q, scales, nquads);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, s, x, q, scales, nquads);
    return hipGetLastError();
}

}  // namespace ptgg
