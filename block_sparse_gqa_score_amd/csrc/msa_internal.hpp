// Internal launch interface between the C ABI (msa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "msa_common.hpp"

namespace msa {

constexpr int kScoreTile = 64;   // query tokens per block-scorer workgroup
constexpr int kAttnTile = 16;    // query tokens per backward dQ workgroup
constexpr int kFwdTile = 24;     // most query tokens per prefill-attention (forward) workgroup:
                                 // a 128-token query block is cut into 6 tiles of 21-22
constexpr int kFwdWaves = 8;     // waves per prefill-attention workgroup (two per SIMD)
constexpr int kAttnUnit = 32;    // keys per prefill-attention pipeline unit

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// LDS of one workgroup on gfx950.  A kernel's static LDS plus the dynamic
// size it is launched with must fit: the queue rejects a larger dispatch
// (and aborts) instead of failing the launch call.
constexpr size_t kCuLdsBytes = 160 * 1024;
inline bool lds_fits(const void *kernel, size_t dynamic_bytes) {
    hipFuncAttributes a{};
    return hipFuncGetAttributes(&a, kernel) == hipSuccess && a.sharedSizeBytes + dynamic_bytes <= kCuLdsBytes;
}

// Geometry: sanitised document spans plus, for two tile sizes, the prefix
// count of document-aligned tiles (off[d] = tiles in documents < d).
hipError_t launch_doc_setup(const int32_t *cu, int ndocs, int T, int max_seqlen, int tile_a,
                            int tile_b, DocSpan *docs, int32_t *off_a, int32_t *off_b,
                            hipStream_t stream);

// Block scores S[h][b][t] (fp32, [4][nb_max][T]) for b <= c(t).
hipError_t launch_block_scores(const void *iq, const void *ik, bool fp8, const DocSpan *docs,
                               const int32_t *tile_off, const int32_t *work_off, int ndocs, int T,
                               int max_seqlen, float *S, hipStream_t stream);

// Forced blocks + top-k from S into q2k [4][T][topk].
hipError_t launch_topk_prefill(const float *S, const DocSpan *docs, int ndocs, int T, int nb_max,
                               int topk, int init, int local, int32_t *q2k, hipStream_t stream);

// Sparse GQA prefill attention: V re-laid as per-unit V^T (unit_off = prefix
// count of kAttnUnit-key units per document; vt holds prefill_units_bytes),
// then the attention kernel over K and V^T.
size_t prefill_units_bytes(int T, int ndocs);
hipError_t launch_kv_units(const uint16_t *k, const uint16_t *v, const DocSpan *docs,
                               const int32_t *unit_off, int ndocs, int T, uint16_t *vt, hipStream_t stream);
// lse (optional, NULL to skip): natural-log log-sum-exp of every row [T,64].
hipError_t launch_attend_prefill(const uint16_t *q, const uint16_t *vt,
                                 const int32_t *q2k, int topk, const DocSpan *docs,
                                 const int32_t *tile_off, const int32_t *unit_off, int ndocs, int T,
                                 float scale, uint16_t *out, float *lse, hipStream_t stream);

// Backward of the prefill attention.  Block lists: for list li = g*nb_max +
// Bg (KV head g, document block Bg numbered over all documents by blk_off)
// the tokens selecting the block, ascending; chunks of kBwdChunk tokens.
constexpr int kBwdChunk = 512;
constexpr int kBwdMaxTokens = 1 << 22;  // keeps 4 * T * topk list entries within int32
struct BwdLayout {
    int nb_max;           // upper bound on the number of document blocks
    int nlists;           // 4 * nb_max
    int max_chunks;       // upper bound on the number of list chunks
    size_t list_entries;  // upper bound on the list entries: 4 * T * topk
    int ntiles;           // 256-token tiles of the list build
};
BwdLayout bwd_layout(int T, int ndocs, int topk);
hipError_t launch_bwd_lists(const int32_t *q2k, int topk, int T, const DocSpan *docs,
                            const int32_t *blk_off, int ndocs, const BwdLayout &L, int32_t *hist, int32_t *cnt,
                            int32_t *list_off, int32_t *chunk_off, int32_t *lists, hipStream_t stream);
hipError_t launch_bwd_dq(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                         const uint16_t *o, const float *lse, float *Dsum, const int32_t *q2k, int topk,
                         const DocSpan *docs, const int32_t *tile_off, int ndocs, int T, float scale,
                         uint16_t *dq, hipStream_t stream);
hipError_t launch_bwd_dkdv(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                           const float *lse, const float *Dsum, const DocSpan *docs,
                           const int32_t *blk_off, int ndocs, const BwdLayout &L, const int32_t *lists,
                           const int32_t *list_off, const int32_t *chunk_off, float scale, float *part,
                           uint16_t *dk, uint16_t *dv, hipStream_t stream);
hipError_t launch_bwd_reduce(const float *part, const int32_t *chunk_off, const DocSpan *docs,
                             const int32_t *blk_off, int ndocs, const BwdLayout &L, uint16_t *dk,
                             uint16_t *dv, hipStream_t stream);

// Paged decode.
hipError_t launch_decode_scores(const void *iq, const void *ikc, bool fp8, const int32_t *pt,
                                int max_pages, const int32_t *ctx, int B, int max_ctx, int nb_max,
                                float *S, hipStream_t stream);
// Selection of each (request, KV head) row from S, then the attention over
// the selected blocks into ceil(topk/8) partials per row; q2k_out [4, B, topk]
// is optional.  kc/vc: bf16 caches, or (fp8kv) E4M3FN caches dequantised as
// byte * k_scale / v_scale.
hipError_t launch_decode_attend(const uint16_t *q, const void *kc, const void *vc, bool fp8kv, float k_scale,
                                float v_scale, const int32_t *pt, int max_pages, const int32_t *ctx,
                                int max_ctx, int B, const float *S, int nb_max, int topk, int init, int local,
                                float scale, float *partial, int32_t *q2k_out, hipStream_t stream);
// bf16 output, or (out_q != NULL) its MXFP8 encoding: E4M3 [B, 64*128] and
// E8M0 scales [B, 64*128/32].
hipError_t launch_decode_combine(const float *partial, int B, int topk, bool fp8kv, uint16_t *out,
                                 uint8_t *out_q, uint8_t *out_scale, hipStream_t stream);
int decode_parts(int topk, int B);  // attention partials per (request, KV head)

// Paged-cache insertion of n tokens' K, V and index-K rows (index-K stored
// as bf16, or as unscaled E4M3 when fp8).
hipError_t launch_cache_insert(const uint16_t *k, const uint16_t *v, const uint16_t *ik, const int32_t *slots,
                               int n, int num_slots, bool fp8, uint16_t *kc, uint16_t *vc, void *ikc,
                               hipStream_t stream);

// Debug validators of the device-side contract: status[0] = violation bits
// (msa_invalid_bits), status[1] = lowest offending document / request.
hipError_t launch_validate_prefill(const int32_t *cu, int ndocs, int T, int max_seqlen, int32_t *status,
                                   hipStream_t stream);
hipError_t launch_validate_decode(const int32_t *pt, int max_pages, const int32_t *ctx, int B, int max_ctx,
                                  int num_pages, int32_t *status, hipStream_t stream);

// MXFP8 encoding of n bf16 values (n a multiple of 32): q [n] E4M3, scale [n/32] E8M0.
hipError_t launch_mxfp8_quantize(const uint16_t *in, int64_t n, uint8_t *q, uint8_t *scale,
                                 hipStream_t stream);

}  // namespace msa
