// Standalone MXFP8 quantisation of a bf16 matrix (the encoding of the decode
// output's MXFP8 variant, applied to any [rows, cols] bf16 data with cols a
// multiple of 32).  One thread per 8 consecutive values; the 4 threads of a
// 32-value block share its scale through two lane exchanges.
#include "msa_internal.hpp"
#include "mxfp8.hpp"

namespace msa {

__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t *__restrict__ in, int64_t n8,
                                                             uint8_t *__restrict__ q,
                                                             uint8_t *__restrict__ scale) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // elements 8i..8i+7
    const bool ok = i < n8;  // n8 is a multiple of 4: a block's 4 threads agree
    uint16_t x[8];
    const u32x4 v = ok ? *(const u32x4 *)(in + 8 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = uint16_t(v[j] & 0xFFFFu);
        x[2 * j + 1] = uint16_t(v[j] >> 16);
    }
    uint32_t sc;
    const uint64_t codes = mxfp8_encode8(x, sc);
    if (ok) {
        *(uint64_t *)(q + 8 * i) = codes;
        if ((i & 3) == 0) scale[i >> 2] = uint8_t(sc);
    }
}

hipError_t launch_mxfp8_quantize(const uint16_t *in, int64_t n, uint8_t *q, uint8_t *scale,
                                 hipStream_t stream) {
    const int64_t n8 = n / 8;
    const int64_t grid = (n8 + 255) / 256;
    hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, in, n8, q, scale);
    return hipGetLastError();
}

}  // namespace msa
