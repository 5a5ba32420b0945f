// Optional debug validators of the device-side data contract, never on the
// timed path: the document map of a packed prefill batch (NeMo AutoModel
// minimax_m3_vl.msa, the document-map classmethod: a non-empty map, no
// interrupted or empty document, coordinates within int32) and the page
// table of a decode batch (TensorRT-LLM "MiniMaxM3SparseAttentionConfig",
// class description: the paged main K/V cache and the side index-K cache
// share their slots, so every page id a request uses must lie in the cache).
//
// One workgroup scans the whole input (these are small: num_docs + 1
// offsets, or the used page-table entries) and writes a status pair
// status[0] = OR of the violation bits, status[1] = the lowest offending
// document or request (-1 when valid).  The kernel overwrites both words,
// so the caller need not clear them (no memset node inside a captured graph).
#include "msa.h"
#include "msa_internal.hpp"

namespace msa {

namespace {
constexpr int kValThreads = 256;
}

__global__ __launch_bounds__(kValThreads) void validate_prefill_kernel(const int32_t *__restrict__ cu, int ndocs,
                                                                       int T, int max_seqlen,
                                                                       int32_t *__restrict__ status) {
    __shared__ int s_bits, s_first;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_bits = 0;
        s_first = 0x7fffffff;
    }
    __syncthreads();
    int bits = 0, first = 0x7fffffff;
    if (tid == 0) {
        if (cu[0] != 0) { bits |= MSA_INVALID_CU_START; first = 0; }
        if (cu[ndocs] != T) { bits |= MSA_INVALID_CU_END; first = min(first, ndocs - 1); }
    }
    for (int d = tid; d < ndocs; d += kValThreads) {
        const int64_t len = int64_t(cu[d + 1]) - int64_t(cu[d]);
        int b = 0;
        if (len <= 0) b |= MSA_INVALID_DOC_EMPTY;          // not strictly increasing
        if (len > max_seqlen) b |= MSA_INVALID_DOC_LONG;    // longer than max_seqlen
        if (cu[d + 1] < 0 || cu[d + 1] > T) b |= MSA_INVALID_CU_RANGE;
        if (b) {
            bits |= b;
            first = min(first, d);
        }
    }
    if (bits) {
        atomicOr(&s_bits, bits);
        atomicMin(&s_first, first);
    }
    __syncthreads();
    if (tid == 0) {
        status[0] = s_bits;
        status[1] = s_bits ? s_first : -1;
    }
}

__global__ __launch_bounds__(kValThreads) void validate_decode_kernel(const int32_t *__restrict__ pt, int max_pages,
                                                                      const int32_t *__restrict__ ctx, int B,
                                                                      int max_ctx, int num_pages,
                                                                      int32_t *__restrict__ status) {
    __shared__ int s_bits, s_first;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_bits = 0;
        s_first = 0x7fffffff;
    }
    __syncthreads();
    int bits = 0, first = 0x7fffffff;
    for (int r = 0; r < B; ++r) {
        const int L = ctx[r];
        int b = 0;
        if (L < 0 || L > max_ctx) b |= MSA_INVALID_CONTEXT_LEN;
        const int np = min(max(L, 0), max_ctx);
        const int nb = (np + kBlock - 1) / kBlock;
        for (int j = tid; j < nb; j += kValThreads) {
            const int page = pt[size_t(r) * max_pages + j];
            if (page < 0 || page >= num_pages) b |= MSA_INVALID_PAGE_ID;
        }
        if (b) {
            bits |= b;
            first = min(first, r);
        }
    }
    if (bits) {
        atomicOr(&s_bits, bits);
        atomicMin(&s_first, first);
    }
    __syncthreads();
    if (tid == 0) {
        status[0] = s_bits;
        status[1] = s_bits ? s_first : -1;
    }
}

hipError_t launch_validate_prefill(const int32_t *cu, int ndocs, int T, int max_seqlen, int32_t *status,
                                   hipStream_t stream) {
    hipLaunchKernelGGL(validate_prefill_kernel, dim3(1), dim3(kValThreads), 0, stream, cu, ndocs, T, max_seqlen,
                       status);
    return hipGetLastError();
}

hipError_t launch_validate_decode(const int32_t *pt, int max_pages, const int32_t *ctx, int B, int max_ctx,
                                  int num_pages, int32_t *status, hipStream_t stream) {
    hipLaunchKernelGGL(validate_decode_kernel, dim3(1), dim3(kValThreads), 0, stream, pt, max_pages, ctx, B,
                       max_ctx, num_pages, status);
    return hipGetLastError();
}

}  // namespace msa
