// MXFP8 encoding of bf16 values: E4M3FN elements with one E8M0 scale per 32
// consecutive values (the decode-output format of the vLLM MiniMax-M3 page,
// MiniMaxM3SparseRocmNvfp4Impl.forward_decode_mxfp8; quantisation as in the
// OCP Microscaling format):
//   scale 2^s, s = floor(log2 amax) - 8 clamped to [-127, 127], stored as
//   s + 127 (an all-zero block takes code 0);
//   element = nearest E4M3FN value of x / 2^s, ties to the even code,
//   magnitudes past 448 saturating to 448, sign of x kept.
// Inputs are finite.
#pragma once

#include "msa_common.hpp"

namespace msa {

// E4M3FN magnitude code nearest to a (0 <= a < 512), ties to even, saturating.
__device__ __forceinline__ uint32_t e4m3_mag_code(float a) {
    if (a < 0.015625f)  // below the smallest normal 2^-6: subnormal steps of 2^-9 (code 8 = 2^-6)
        return uint32_t(__builtin_rintf(a * 512.f));
    const int e = int((__float_as_uint(a) >> 23) & 0xff) - 127;  // floor(log2 a), -6..8
    const float m = __builtin_rintf(a * __uint_as_float(uint32_t(127 + 3 - e) << 23));  // 8..16
    // m == 16 carries into the next exponent; code 0x7F would be NaN, so clamp
    return min(uint32_t(8 * (e + 7)) + uint32_t(m) - 8u, 0x7Eu);
}

// floor(log2) of a non-zero bf16 magnitude (bits without the sign)
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
    const int e = int(mag >> 7);
    return e ? e - 127 : -133 + (31 - __builtin_clz(mag));  // subnormal: m * 2^-133
}

// |x| * 2^-s for a bf16 magnitude, built from the bits (exact; results below
// 2^-126 become 0, far under E4M3's resolution at any scale)
__device__ __forceinline__ float mx_scaled(uint32_t mag, int s) {
    const int E = int(mag >> 7), M = int(mag & 0x7F);
    if (E) {
        const int e2 = E - s;  // biased exponent after the shift
        return e2 >= 1 ? __uint_as_float((uint32_t(e2) << 23) | (uint32_t(M) << 16)) : 0.f;
    }
    const int p = 127 - 133 - s;  // biased exponent of 2^(-133 - s)
    return p >= 1 ? float(M) * __uint_as_float(uint32_t(p) << 23) : 0.f;
}

// MXFP8 of 32 consecutive bf16 values held 8 per lane by 4 consecutive lanes
// (lanes 4k..4k+3, all active): returns this lane's 8 codes (byte i =
// element i) and the block's E8M0 code (the same in the 4 lanes).
__device__ __forceinline__ uint64_t mxfp8_encode8(const uint16_t (&x)[8], uint32_t &scale) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, uint32_t(x[i]) & 0x7FFFu);
    amax = max(amax, uint32_t(__shfl_xor(int(amax), 1)));
    amax = max(amax, uint32_t(__shfl_xor(int(amax), 2)));
    const int s = amax ? max(min(bf16_floor_log2(amax) - 8, 127), -127) : -127;
    scale = uint32_t(s + 127);
    uint64_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t code = e4m3_mag_code(mx_scaled(uint32_t(x[i]) & 0x7FFFu, s)) | ((uint32_t(x[i]) >> 8) & 0x80u);
        out |= uint64_t(code) << (8 * i);
    }
    return out;
}

}  // namespace msa
