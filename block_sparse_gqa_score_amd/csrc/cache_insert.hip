// Cache insertion (the write that precedes decode; TensorRT-LLM
// "MiniMaxM3SparseAttentionConfig", fuse_qkv_index_projection: a producer
// writes the normed, RoPE'd rows into the paged caches; the side index-K
// cache is parallel to the main K/V cache, same slot).  Token n's K and V
// rows (4 heads x 128) and its index-K row go to slot slot_mapping[n]; a
// negative slot, or one past num_slots, is skipped.  With the E4M3 indexer
// the index-K row is stored as unscaled E4M3FN (nearest, ties to even,
// saturating at 448).
#include "msa_internal.hpp"
#include "mxfp8.hpp"

namespace msa {

// One 256-thread workgroup per token: threads 0..63 copy the K row (1 KiB),
// 64..127 the V row, 128..143 the index-K row (16 bytes of bf16 each).
__global__ __launch_bounds__(256) void cache_insert_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const uint16_t *__restrict__ ik,
    const int32_t *__restrict__ slots, int num_slots, bool fp8, uint16_t *__restrict__ kc,
    uint16_t *__restrict__ vc, uint8_t *__restrict__ ikc) {
    const int n = blockIdx.x, tid = threadIdx.x;
    const int slot = slots[n];
    if (slot < 0 || slot >= num_slots) return;
    constexpr int kRow = kKvHeads * kDim;  // 512 elements
    if (tid < 64) {
        *(u32x4 *)(kc + size_t(slot) * kRow + 8 * tid) = *(const u32x4 *)(k + size_t(n) * kRow + 8 * tid);
    } else if (tid < 128) {
        const int t = tid - 64;
        *(u32x4 *)(vc + size_t(slot) * kRow + 8 * t) = *(const u32x4 *)(v + size_t(n) * kRow + 8 * t);
    } else if (tid < 144) {
        const int t = tid - 128;
        const u32x4 x = *(const u32x4 *)(ik + size_t(n) * kDim + 8 * t);
        if (!fp8) {
            *(u32x4 *)((uint16_t *)ikc + size_t(slot) * kDim + 8 * t) = x;
        } else {
            uint64_t out = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t b = (j & 1) ? (x[j >> 1] >> 16) : (x[j >> 1] & 0xFFFFu);
                const float a = mx_scaled(b & 0x7FFFu, 0);  // |x|, exact
                const uint32_t code = (a >= 448.f ? 0x7Eu : e4m3_mag_code(a)) | ((b >> 8) & 0x80u);
                out |= uint64_t(code) << (8 * j);
            }
            *(uint64_t *)(ikc + size_t(slot) * kDim + 8 * t) = out;
        }
    }
}

hipError_t launch_cache_insert(const uint16_t *k, const uint16_t *v, const uint16_t *ik, const int32_t *slots,
                               int n, int num_slots, bool fp8, uint16_t *kc, uint16_t *vc, void *ikc,
                               hipStream_t stream) {
    hipLaunchKernelGGL(cache_insert_kernel, dim3(n), dim3(256), 0, stream, k, v, ik, slots, num_slots, fp8, kc,
                       vc, (uint8_t *)ikc);
    return hipGetLastError();
}

}  // namespace msa
