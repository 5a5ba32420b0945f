// Device-side building blocks shared by the libmsa kernels (gfx950 only).
//
// MFMA register layouts used throughout (wave64, lane l):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: lane m + 32*(k-group), 8 bf16 per lane
//                             B[k][n]: lane n + 32*(k-group), 8 bf16 per lane
//                             D[m][n]: lane n + 32*((m/4)%2), reg 4*(m/8) + m%4
//   v_mfma_f32_16x16x32_bf16  A[m][k]: lane m + 16*(k-group), 8 per lane
//                             B[k][n]: lane n + 16*(k-group), 8 per lane
//                             D[m][n]: lane n + 16*(m/4), reg m%4
// The contraction index only has to be assigned to (k-group, element) the
// same way in A and B, so each kernel picks the k order that makes its
// loads contiguous; the m/n lane mapping and the D layout are fixed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kHeads = 64;     // query heads
constexpr int kKvHeads = 4;    // key/value heads
constexpr int kGroup = 16;     // query heads per KV head (contiguous groups)
constexpr int kDim = 128;      // head dim = index dim
constexpr int kIdxHeads = 4;   // index heads (index head g selects for KV head g)
constexpr int kBlock = 128;    // key block = page size
constexpr int kMaxTopk = 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Sanitised document bounds: start and length, clamped into [0, T] and to
// max_seqlen so that no kernel can index past the token buffers.
struct DocSpan {
    int start;
    int len;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(uint32_t(b) << 16);
}

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp8 E4M3 x E4M3 with unit block scales (E8M0 127 = 2^0): an unscaled
// E4M3 product accumulated in FP32.  Format code 0 selects E4M3 for A and B.
__device__ __forceinline__ f32x16 mfma_32x32x64_e4m3(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ f32x4 mfma_16x16x128_e4m3(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Order-preserving map of an fp32 score to uint32 (larger float -> larger).
__device__ __forceinline__ uint32_t float_order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Document containing compact token t (binary search over sanitised spans);
// -1 when t lies in no span.
__device__ __forceinline__ int find_doc(const DocSpan *docs, int ndocs, int t) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (docs[mid].start <= t) lo = mid; else hi = mid - 1;
    }
    const DocSpan d = docs[lo];
    return (t >= d.start && t < d.start + d.len) ? lo : -1;
}

// Number of forced blocks among 0..c: {b < init} U {c-local+1 <= b <= c}.
__device__ __forceinline__ int forced_count(int c, int init, int local) {
    int n_init = min(init, c + 1);
    if (local <= 0) return n_init;
    int lo = max(c - local + 1, 0);
    int n_local = c - lo + 1;
    int overlap = max(0, n_init - lo);
    return n_init + n_local - overlap;
}

__device__ __forceinline__ bool is_forced(int b, int c, int init, int local) {
    return b < init || b >= c - local + 1;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

}  // namespace msa
