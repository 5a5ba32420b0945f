// C ABI of libmsa: argument validation, workspace layout and kernel launch
// order.  Declarations and the contract of every entry point are in
// include/msa.h.  No entry point allocates device memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "msa.h"
#include "msa_internal.hpp"

using namespace msa;

namespace {

thread_local char g_err[512] = "";

msa_status fail(msa_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

msa_status hip_fail(hipError_t e, const char *where) {
    return fail(MSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Benchmark instrumentation armed by msa_set_timing_events (one call).
struct Timing {
    void *const *events = nullptr;
    int capacity = 0;
    int recorded = 0;
    const char *names[16] = {};
    int kernels = 0;
};
thread_local Timing g_timing;

// Start of an entry point: take the arming for this call.
struct TimingScope {
    void *const *events;
    int capacity;
    int n = 0;
    explicit TimingScope() : events(g_timing.events), capacity(g_timing.capacity) {
        g_timing.events = nullptr;
        g_timing.capacity = 0;
        if (events) g_timing.kernels = 0;
    }
    // before launching kernel `name` (or after the last one with name == nullptr)
    void mark(hipStream_t s, const char *name) {
        if (!events || n >= capacity) return;
        hipEventRecord((hipEvent_t)events[n], s);
        if (name && n < 16) g_timing.names[n] = name;
        g_timing.kernels = name ? n + 1 : n;
        ++n;
    }
};

// Decode top-k holds up to 128 candidates per lane: 8192 blocks.
constexpr int kDecodeMaxBlocks = 64 * 128;

struct SelectWs {
    size_t docs, off, work_off, scores, total;
};

// document spans; per document, prefix counts of the scorer's tiles and of
// its (tile, key block) work items; block scores
SelectWs select_layout(int T, int ndocs, int max_seqlen) {
    SelectWs w;
    const int nb_max = ceil_div(max_seqlen, kBlock);
    w.docs = 0;
    w.off = align256(w.docs + sizeof(DocSpan) * size_t(ndocs));
    w.work_off = align256(w.off + sizeof(int32_t) * (size_t(ndocs) + 1));
    w.scores = align256(w.work_off + sizeof(int32_t) * (size_t(ndocs) + 1));
    w.total = align256(w.scores + sizeof(float) * size_t(kIdxHeads) * nb_max * size_t(T));
    return w;
}

struct PrefillWs {
    size_t docs, off, uoff, vt, total;
};

PrefillWs prefill_layout(int T, int ndocs) {
    PrefillWs w;
    w.docs = 0;
    w.off = align256(sizeof(DocSpan) * size_t(ndocs));
    w.uoff = align256(w.off + sizeof(int32_t) * (size_t(ndocs) + 1));
    w.vt = align256(w.uoff + sizeof(int32_t) * (size_t(ndocs) + 1));
    w.total = align256(w.vt + prefill_units_bytes(T, ndocs));
    return w;
}

struct BwdWs {
    size_t docs, tile_off, blk_off, dsum, hist, cnt, list_off, chunk_off, lists, part, total;
    BwdLayout L;
};

BwdWs backward_layout(int T, int ndocs, int topk) {
    BwdWs w;
    w.L = bwd_layout(T, ndocs, topk);
    size_t o = 0;
    w.docs = o;
    o = align256(o + sizeof(DocSpan) * size_t(ndocs));
    w.tile_off = o;
    o = align256(o + sizeof(int32_t) * (size_t(ndocs) + 1));
    w.blk_off = o;
    o = align256(o + sizeof(int32_t) * (size_t(ndocs) + 1));
    w.dsum = o;
    o = align256(o + sizeof(float) * size_t(T) * kHeads);
    w.hist = o;
    o = align256(o + sizeof(int32_t) * size_t(w.L.ntiles) * size_t(w.L.nlists));
    w.cnt = o;
    o = align256(o + sizeof(int32_t) * size_t(w.L.nlists));
    w.list_off = o;
    o = align256(o + sizeof(int32_t) * (size_t(w.L.nlists) + 1));
    w.chunk_off = o;
    o = align256(o + sizeof(int32_t) * (size_t(w.L.nlists) + 1));
    w.lists = o;
    o = align256(o + sizeof(int32_t) * w.L.list_entries);
    w.part = o;
    o = align256(o + sizeof(float) * size_t(w.L.max_chunks) * 2 * kBlock * kDim);
    w.total = o;
    return w;
}

struct DecodeWs {
    size_t scores, part, total;
};

// scores fp32 [B][4][nb_max]; partials: O fp32 [B][4][parts][16][128], then
// (m, l) fp32 [B][4][parts][16][2]
DecodeWs decode_layout(int B, int max_ctx, int topk) {
    DecodeWs w;
    const int nb_max = ceil_div(max_ctx, kBlock);
    w.scores = 0;
    w.part = align256(sizeof(float) * size_t(B) * kIdxHeads * nb_max);
    const size_t part_floats = size_t(B) * kKvHeads * decode_parts(topk, B) * kGroup * (kDim + 2);
    w.total = align256(w.part + sizeof(float) * part_floats);
    return w;
}

msa_status check_geometry(const int32_t *cu, int ndocs, int T, int max_seqlen) {
    if (!cu) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (T < 1) return fail(MSA_ERR_INVALID_ARG, "total_tokens must be >= 1 (got %d)", T);
    if (ndocs < 1 || ndocs > T)
        return fail(MSA_ERR_INVALID_ARG, "num_docs must be in [1, total_tokens] (got %d)", ndocs);
    if (max_seqlen < 1 || max_seqlen > T)
        return fail(MSA_ERR_INVALID_ARG, "max_seqlen must be in [1, total_tokens] (got %d)", max_seqlen);
    return MSA_OK;
}

msa_status check_selection(int topk, int init, int local) {
    if (topk < 1 || topk > kMaxTopk)
        return fail(MSA_ERR_UNSUPPORTED, "topk must be in [1, %d] (got %d)", kMaxTopk, topk);
    if (init < 0 || local < 0)
        return fail(MSA_ERR_INVALID_ARG, "init_blocks and local_blocks must be >= 0");
    if (init + local > topk)
        return fail(MSA_ERR_INVALID_ARG, "init_blocks + local_blocks (%d) exceeds topk (%d)",
                    init + local, topk);
    return MSA_OK;
}

}  // namespace

extern "C" {

const char *msa_last_error(void) { return g_err; }

void msa_set_timing_events(void *const *events, int count) {
    g_timing.events = count > 0 ? events : nullptr;
    g_timing.capacity = count > 0 ? count : 0;
}

int msa_timing_kernel_count(void) { return g_timing.kernels; }

const char *msa_timing_kernel_name(int i) {
    return (i >= 0 && i < g_timing.kernels && i < 16) ? g_timing.names[i] : "";
}

int msa_version(void) { return 100; }

const char *msa_unsupported_reason(int num_heads, int num_kv_heads, int head_dim,
                                   int num_index_heads, int index_dim, int topk,
                                   int block_size) {
    if (num_heads != MSA_NUM_HEADS) return "num_heads must be 64";
    if (num_kv_heads != MSA_NUM_KV_HEADS) return "num_kv_heads must be 4";
    if (head_dim != MSA_HEAD_DIM) return "head_dim must be 128";
    if (num_index_heads != MSA_NUM_INDEX_HEADS) return "num_index_heads must be 4";
    if (index_dim != MSA_INDEX_DIM) return "index_dim must be 128";
    if (block_size != MSA_BLOCK_SIZE) return "block_size must be 128";
    if (topk < 1 || topk > MSA_MAX_TOPK) return "topk must be in [1, 16]";
    return NULL;
}

size_t msa_select_blocks_workspace_bytes(int total_tokens, int num_docs, int max_seqlen) {
    if (total_tokens < 1 || num_docs < 1 || num_docs > total_tokens || max_seqlen < 1 ||
        max_seqlen > total_tokens)
        return 0;
    return select_layout(total_tokens, num_docs, max_seqlen).total;
}

size_t msa_prefill_workspace_bytes(int total_tokens, int num_docs, int max_seqlen) {
    if (total_tokens < 1 || num_docs < 1 || num_docs > total_tokens || max_seqlen < 1 ||
        max_seqlen > total_tokens)
        return 0;
    return prefill_layout(total_tokens, num_docs).total;
}

size_t msa_prefill_backward_workspace_bytes(int total_tokens, int num_docs, int max_seqlen, int topk) {
    if (total_tokens < 1 || num_docs < 1 || num_docs > total_tokens || max_seqlen < 1 ||
        max_seqlen > total_tokens || topk < 1 || topk > kMaxTopk || total_tokens > kBwdMaxTokens)
        return 0;
    return backward_layout(total_tokens, num_docs, topk).total;
}

size_t msa_decode_workspace_bytes(int batch, int max_context_len, int topk) {
    if (batch < 1 || max_context_len < 1 || topk < 1 || topk > kMaxTopk ||
        ceil_div(max_context_len, kBlock) > kDecodeMaxBlocks)
        return 0;
    return decode_layout(batch, max_context_len, topk).total;
}

msa_status msa_select_blocks(const void *index_q, const void *index_k, int index_dtype,
                             const int32_t *cu_seqlens, int num_docs, int total_tokens,
                             int max_seqlen, int topk, int init_blocks, int local_blocks,
                             int32_t *q2k, float *scores_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
    if (!index_q || !index_k || !q2k) return fail(MSA_ERR_INVALID_ARG, "index_q, index_k and q2k must be non-NULL");
    if (index_dtype != MSA_INDEX_BF16 && index_dtype != MSA_INDEX_FP8_E4M3)
        return fail(MSA_ERR_UNSUPPORTED, "index_dtype must be MSA_INDEX_BF16 or MSA_INDEX_FP8_E4M3");
    msa_status st = check_geometry(cu_seqlens, num_docs, total_tokens, max_seqlen);
    if (st != MSA_OK) return st;
    if ((st = check_selection(topk, init_blocks, local_blocks)) != MSA_OK) return st;
    const SelectWs ws = select_layout(total_tokens, num_docs, max_seqlen);
    if (!workspace || workspace_bytes < ws.total)
        return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                    workspace ? workspace_bytes : size_t(0));
    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = (uint8_t *)workspace;
    DocSpan *docs = (DocSpan *)(base + ws.docs);
    int32_t *off = (int32_t *)(base + ws.off);
    int32_t *work_off = (int32_t *)(base + ws.work_off);
    float *S = scores_out ? scores_out : (float *)(base + ws.scores);
    const int nb_max = ceil_div(max_seqlen, kBlock);
    TimingScope tm;
    tm.mark(s, "doc_setup");
    hipError_t e = launch_doc_setup(cu_seqlens, num_docs, total_tokens, max_seqlen, kScoreTile, -1,
                                    docs, off, work_off, s);
    if (e != hipSuccess) return hip_fail(e, "doc_setup");
    tm.mark(s, "block_scores");
    e = launch_block_scores(index_q, index_k, index_dtype == MSA_INDEX_FP8_E4M3, docs, off, work_off,
                            num_docs, total_tokens, max_seqlen, S, s);
    if (e != hipSuccess) return hip_fail(e, "block_scores");
    tm.mark(s, "topk_prefill");
    e = launch_topk_prefill(S, docs, num_docs, total_tokens, nb_max, topk, init_blocks, local_blocks,
                            q2k, s);
    if (e != hipSuccess) return hip_fail(e, "topk");
    tm.mark(s, nullptr);
    return MSA_OK;
}

static msa_status prefill_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *q2k, int topk, const int32_t *cu_seqlens, int num_docs,
                               int total_tokens, int max_seqlen, float softmax_scale, uint16_t *out,
                               float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !q2k || !out) return fail(MSA_ERR_INVALID_ARG, "q, k, v, q2k and out must be non-NULL");
    if (topk < 1 || topk > kMaxTopk)
        return fail(MSA_ERR_UNSUPPORTED, "topk must be in [1, %d] (got %d)", kMaxTopk, topk);
    msa_status st = check_geometry(cu_seqlens, num_docs, total_tokens, max_seqlen);
    if (st != MSA_OK) return st;
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
        return fail(MSA_ERR_INVALID_ARG, "softmax_scale must be a positive finite number");
    const PrefillWs ws = prefill_layout(total_tokens, num_docs);
    if (!workspace || workspace_bytes < ws.total)
        return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                    workspace ? workspace_bytes : size_t(0));
    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = (uint8_t *)workspace;
    DocSpan *docs = (DocSpan *)(base + ws.docs);
    int32_t *off = (int32_t *)(base + ws.off);
    int32_t *uoff = (int32_t *)(base + ws.uoff);
    uint16_t *vt = (uint16_t *)(base + ws.vt);
    TimingScope tm;
    tm.mark(s, "doc_setup");
    hipError_t e = launch_doc_setup(cu_seqlens, num_docs, total_tokens, max_seqlen, kFwdTile,
                                    kAttnUnit, docs, off, uoff, s);
    if (e != hipSuccess) return hip_fail(e, "doc_setup");
    tm.mark(s, "kv_units");
    e = launch_kv_units(k, v, docs, uoff, num_docs, total_tokens, vt, s);
    if (e != hipSuccess) return hip_fail(e, "kv_units");
    tm.mark(s, "attend_prefill");
    e = launch_attend_prefill(q, vt, q2k, topk, docs, off, uoff, num_docs, total_tokens,
                              softmax_scale, out, lse, s);
    if (e != hipSuccess) return hip_fail(e, "attend_prefill");
    tm.mark(s, nullptr);
    return MSA_OK;
}

msa_status msa_sparse_attend_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     const int32_t *q2k, int topk, const int32_t *cu_seqlens,
                                     int num_docs, int total_tokens, int max_seqlen,
                                     float softmax_scale, uint16_t *out, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    return prefill_impl(q, k, v, q2k, topk, cu_seqlens, num_docs, total_tokens, max_seqlen, softmax_scale,
                        out, nullptr, workspace, workspace_bytes, stream);
}

msa_status msa_sparse_attend_prefill_lse(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                         const int32_t *q2k, int topk, const int32_t *cu_seqlens,
                                         int num_docs, int total_tokens, int max_seqlen,
                                         float softmax_scale, uint16_t *out, float *lse, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    if (!lse) return fail(MSA_ERR_INVALID_ARG, "lse must be non-NULL");
    return prefill_impl(q, k, v, q2k, topk, cu_seqlens, num_docs, total_tokens, max_seqlen, softmax_scale,
                        out, lse, workspace, workspace_bytes, stream);
}

msa_status msa_sparse_attend_prefill_backward(
    const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *out, const float *lse,
    const uint16_t *dout, const int32_t *q2k, int topk, const int32_t *cu_seqlens, int num_docs,
    int total_tokens, int max_seqlen, float softmax_scale, uint16_t *dq, uint16_t *dk, uint16_t *dv,
    void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !out || !lse || !dout || !q2k || !dq || !dk || !dv)
        return fail(MSA_ERR_INVALID_ARG, "q, k, v, out, lse, dout, q2k, dq, dk and dv must be non-NULL");
    if (topk < 1 || topk > kMaxTopk)
        return fail(MSA_ERR_UNSUPPORTED, "topk must be in [1, %d] (got %d)", kMaxTopk, topk);
    msa_status st = check_geometry(cu_seqlens, num_docs, total_tokens, max_seqlen);
    if (st != MSA_OK) return st;
    if (total_tokens > kBwdMaxTokens)
        return fail(MSA_ERR_UNSUPPORTED, "total_tokens above %d is not supported by the backward (got %d)",
                    kBwdMaxTokens, total_tokens);
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
        return fail(MSA_ERR_INVALID_ARG, "softmax_scale must be a positive finite number");
    const BwdWs ws = backward_layout(total_tokens, num_docs, topk);
    if (!workspace || workspace_bytes < ws.total)
        return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                    workspace ? workspace_bytes : size_t(0));
    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = (uint8_t *)workspace;
    DocSpan *docs = (DocSpan *)(base + ws.docs);
    int32_t *tile_off = (int32_t *)(base + ws.tile_off);
    int32_t *blk_off = (int32_t *)(base + ws.blk_off);
    float *dsum = (float *)(base + ws.dsum);
    int32_t *hist = (int32_t *)(base + ws.hist);
    int32_t *cnt = (int32_t *)(base + ws.cnt);
    int32_t *list_off = (int32_t *)(base + ws.list_off);
    int32_t *chunk_off = (int32_t *)(base + ws.chunk_off);
    int32_t *lists = (int32_t *)(base + ws.lists);
    float *part = (float *)(base + ws.part);
    TimingScope tm;
    tm.mark(s, "doc_setup");
    hipError_t e = launch_doc_setup(cu_seqlens, num_docs, total_tokens, max_seqlen, kAttnTile, kBlock, docs,
                                    tile_off, blk_off, s);
    if (e != hipSuccess) return hip_fail(e, "doc_setup");
    tm.mark(s, "bwd_lists");
    e = launch_bwd_lists(q2k, topk, total_tokens, docs, blk_off, num_docs, ws.L, hist, cnt, list_off, chunk_off,
                         lists, s);
    if (e != hipSuccess) return hip_fail(e, "bwd_lists");
    tm.mark(s, "bwd_dq");
    e = launch_bwd_dq(q, k, v, dout, out, lse, dsum, q2k, topk, docs, tile_off, num_docs, total_tokens,
                      softmax_scale, dq, s);
    if (e != hipSuccess) return hip_fail(e, "bwd_dq");
    tm.mark(s, "bwd_dkdv");
    e = launch_bwd_dkdv(q, k, v, dout, lse, dsum, docs, blk_off, num_docs, ws.L, lists, list_off, chunk_off,
                        softmax_scale, part, dk, dv, s);
    if (e != hipSuccess) return hip_fail(e, "bwd_dkdv");
    tm.mark(s, "bwd_reduce");
    e = launch_bwd_reduce(part, chunk_off, docs, blk_off, num_docs, ws.L, dk, dv, s);
    if (e != hipSuccess) return hip_fail(e, "bwd_reduce");
    tm.mark(s, nullptr);
    return MSA_OK;
}

// One decode step; the output is bf16 `out`, or its MXFP8 encoding when
// out_q / out_scale are given instead.
static msa_status decode_paged_impl(
    const uint16_t *q, const void *index_q, const void *k_cache, const void *v_cache, bool kv_fp8,
    float k_scale, float v_scale, const void *index_k_cache, int index_dtype, const int32_t *page_table,
    int max_pages_per_seq,
    const int32_t *context_lens, int batch, int max_context_len, int topk, int init_blocks,
    int local_blocks, float softmax_scale, uint16_t *out, uint8_t *out_q, uint8_t *out_scale,
    int32_t *q2k_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !index_q || !k_cache || !v_cache || !index_k_cache || !page_table || !context_lens ||
        !(out || (out_q && out_scale)))
        return fail(MSA_ERR_INVALID_ARG, "tensor arguments must be non-NULL (q2k_out may be NULL)");
    if (index_dtype != MSA_INDEX_BF16 && index_dtype != MSA_INDEX_FP8_E4M3)
        return fail(MSA_ERR_UNSUPPORTED, "index_dtype must be MSA_INDEX_BF16 or MSA_INDEX_FP8_E4M3");
    if (batch < 1) return fail(MSA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (max_context_len < 1) return fail(MSA_ERR_INVALID_ARG, "max_context_len must be >= 1");
    const int nb_max = ceil_div(max_context_len, kBlock);
    if (nb_max > kDecodeMaxBlocks)
        return fail(MSA_ERR_UNSUPPORTED, "max_context_len above %d is not supported",
                    kDecodeMaxBlocks * kBlock);
    if (max_pages_per_seq < nb_max)
        return fail(MSA_ERR_INVALID_ARG, "max_pages_per_seq (%d) < ceil(max_context_len/128) (%d)",
                    max_pages_per_seq, nb_max);
    msa_status st = check_selection(topk, init_blocks, local_blocks);
    if (st != MSA_OK) return st;
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
        return fail(MSA_ERR_INVALID_ARG, "softmax_scale must be a positive finite number");
    const DecodeWs ws = decode_layout(batch, max_context_len, topk);
    if (!workspace || workspace_bytes < ws.total)
        return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                    workspace ? workspace_bytes : size_t(0));
    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = (uint8_t *)workspace;
    float *S = (float *)(base + ws.scores);
    float *part = (float *)(base + ws.part);
    TimingScope tm;
    tm.mark(s, "decode_scores");
    hipError_t e = launch_decode_scores(index_q, index_k_cache, index_dtype == MSA_INDEX_FP8_E4M3,
                                        page_table, max_pages_per_seq, context_lens, batch,
                                        max_context_len, nb_max, S, s);
    if (e != hipSuccess) return hip_fail(e, "decode_scores");
    tm.mark(s, "decode_attend");
    e = launch_decode_attend(q, k_cache, v_cache, kv_fp8, k_scale, v_scale, page_table, max_pages_per_seq,
                             context_lens, max_context_len, batch, S, nb_max, topk, init_blocks, local_blocks,
                             softmax_scale, part, q2k_out, s);
    if (e != hipSuccess) return hip_fail(e, "decode_attend");
    tm.mark(s, "decode_combine");
    e = launch_decode_combine(part, batch, topk, kv_fp8, out, out_q, out_scale, s);
    if (e != hipSuccess) return hip_fail(e, "decode_combine");
    tm.mark(s, nullptr);
    return MSA_OK;
}

msa_status msa_sparse_attend_decode_paged(
    const uint16_t *q, const void *index_q, const uint16_t *k_cache, const uint16_t *v_cache,
    const void *index_k_cache, int index_dtype, const int32_t *page_table, int max_pages_per_seq,
    const int32_t *context_lens, int batch, int max_context_len, int topk, int init_blocks,
    int local_blocks, float softmax_scale, uint16_t *out, int32_t *q2k_out, void *workspace,
    size_t workspace_bytes, void *stream) {
    if (!out) return fail(MSA_ERR_INVALID_ARG, "out must be non-NULL");
    return decode_paged_impl(q, index_q, k_cache, v_cache, false, 1.f, 1.f, index_k_cache, index_dtype, page_table,
                             max_pages_per_seq, context_lens, batch, max_context_len, topk, init_blocks,
                             local_blocks, softmax_scale, out, nullptr, nullptr, q2k_out, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free decode: the workspace is a file-scope device array of
// MSA_NOALLOC_SCRATCH_BYTES per GPU (held from library load to process end).
// Host code never uses the array's name as an address: on a device's first
// call, with that device current, hipGetSymbolAddress gives the device
// address, which is kept per device and passed to the kernels.
// ---------------------------------------------------------------------------
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) uint8_t scratch[MSA_NOALLOC_SCRATCH_BYTES];

static msa_status scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MSA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MSA_OK;
}

extern "C" {

msa_status msa_sparse_attend_decode_paged_noalloc(
    const uint16_t *q, const void *index_q, const uint16_t *k_cache, const uint16_t *v_cache,
    const void *index_k_cache, int index_dtype, const int32_t *page_table, int max_pages_per_seq,
    const int32_t *context_lens, int batch, int max_context_len, int topk, int init_blocks,
    int local_blocks, float softmax_scale, uint16_t *out, int32_t *q2k_out, void *stream) {
    if (!out) return fail(MSA_ERR_INVALID_ARG, "out must be non-NULL");
    const size_t need = msa_decode_workspace_bytes(batch, max_context_len, topk);
    if (need > MSA_NOALLOC_SCRATCH_BYTES)
        return fail(MSA_ERR_UNSUPPORTED,
                    "this batch needs %zu bytes of scratch; the allocation-free decode holds %zu "
                    "(use msa_sparse_attend_decode_paged with a workspace)",
                    need, size_t(MSA_NOALLOC_SCRATCH_BYTES));
    void *ws = nullptr;
    const msa_status st = scratch_of_current_device(&ws);
    if (st != MSA_OK) return st;
    // every scratch byte the kernels read is written earlier in the same
    // call (scores, then partials), so nothing needs clearing
    return decode_paged_impl(q, index_q, k_cache, v_cache, false, 1.f, 1.f, index_k_cache, index_dtype, page_table,
                             max_pages_per_seq, context_lens, batch, max_context_len, topk, init_blocks,
                             local_blocks, softmax_scale, out, nullptr, nullptr, q2k_out, ws,
                             MSA_NOALLOC_SCRATCH_BYTES, stream);
}

msa_status msa_sparse_attend_decode_paged_mxfp8(
    const uint16_t *q, const void *index_q, const uint16_t *k_cache, const uint16_t *v_cache,
    const void *index_k_cache, int index_dtype, const int32_t *page_table, int max_pages_per_seq,
    const int32_t *context_lens, int batch, int max_context_len, int topk, int init_blocks,
    int local_blocks, float softmax_scale, uint8_t *out_q, uint8_t *out_scale, int32_t *q2k_out,
    void *workspace, size_t workspace_bytes, void *stream) {
    if (!out_q || !out_scale) return fail(MSA_ERR_INVALID_ARG, "out_q and out_scale must be non-NULL");
    return decode_paged_impl(q, index_q, k_cache, v_cache, false, 1.f, 1.f, index_k_cache, index_dtype, page_table,
                             max_pages_per_seq, context_lens, batch, max_context_len, topk, init_blocks,
                             local_blocks, softmax_scale, nullptr, out_q, out_scale, q2k_out, workspace,
                             workspace_bytes, stream);
}

msa_status msa_sparse_attend_decode_paged_fp8kv(
    const uint16_t *q, const void *index_q, const uint8_t *k_cache, const uint8_t *v_cache, float k_scale,
    float v_scale, const void *index_k_cache, int index_dtype, const int32_t *page_table,
    int max_pages_per_seq, const int32_t *context_lens, int batch, int max_context_len, int topk,
    int init_blocks, int local_blocks, float softmax_scale, uint16_t *out, int32_t *q2k_out,
    void *workspace, size_t workspace_bytes, void *stream) {
    if (!out) return fail(MSA_ERR_INVALID_ARG, "out must be non-NULL");
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale > 1e30f || v_scale > 1e30f)
        return fail(MSA_ERR_INVALID_ARG, "k_scale and v_scale must be positive finite numbers");
    return decode_paged_impl(q, index_q, k_cache, v_cache, true, k_scale, v_scale, index_k_cache, index_dtype,
                             page_table, max_pages_per_seq, context_lens, batch, max_context_len, topk,
                             init_blocks, local_blocks, softmax_scale, out, nullptr, nullptr, q2k_out, workspace,
                             workspace_bytes, stream);
}

msa_status msa_cache_insert(const uint16_t *k, const uint16_t *v, const uint16_t *index_k,
                            const int32_t *slot_mapping, int num_tokens, int index_dtype, uint16_t *k_cache,
                            uint16_t *v_cache, void *index_k_cache, int num_slots, void *stream) {
    if (!k || !v || !index_k || !slot_mapping || !k_cache || !v_cache || !index_k_cache)
        return fail(MSA_ERR_INVALID_ARG, "tensor arguments must be non-NULL");
    if (index_dtype != MSA_INDEX_BF16 && index_dtype != MSA_INDEX_FP8_E4M3)
        return fail(MSA_ERR_UNSUPPORTED, "index_dtype must be MSA_INDEX_BF16 or MSA_INDEX_FP8_E4M3");
    if (num_tokens < 0) return fail(MSA_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (num_slots < 1) return fail(MSA_ERR_INVALID_ARG, "num_slots must be >= 1 (got %d)", num_slots);
    if (num_tokens == 0) return MSA_OK;
    const hipError_t e = launch_cache_insert(k, v, index_k, slot_mapping, num_tokens, num_slots,
                                             index_dtype == MSA_INDEX_FP8_E4M3, k_cache, v_cache,
                                             index_k_cache, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "cache_insert");
    return MSA_OK;
}

msa_status msa_validate_prefill_inputs(const int32_t *cu_seqlens, int num_docs, int total_tokens,
                                       int max_seqlen, int32_t *status, void *stream) {
    if (!status) return fail(MSA_ERR_INVALID_ARG, "status must be non-NULL");
    msa_status st = check_geometry(cu_seqlens, num_docs, total_tokens, max_seqlen);
    if (st != MSA_OK) return st;
    const hipError_t e = launch_validate_prefill(cu_seqlens, num_docs, total_tokens, max_seqlen, status,
                                                 (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "validate_prefill");
    return MSA_OK;
}

msa_status msa_validate_decode_inputs(const int32_t *page_table, int max_pages_per_seq,
                                      const int32_t *context_lens, int batch, int max_context_len,
                                      int num_pages, int32_t *status, void *stream) {
    if (!page_table || !context_lens || !status)
        return fail(MSA_ERR_INVALID_ARG, "page_table, context_lens and status must be non-NULL");
    if (batch < 1) return fail(MSA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (max_context_len < 1) return fail(MSA_ERR_INVALID_ARG, "max_context_len must be >= 1");
    if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages must be >= 1 (got %d)", num_pages);
    if (max_pages_per_seq < ceil_div(max_context_len, kBlock))
        return fail(MSA_ERR_INVALID_ARG, "max_pages_per_seq (%d) < ceil(max_context_len/128) (%d)",
                    max_pages_per_seq, ceil_div(max_context_len, kBlock));
    const hipError_t e = launch_validate_decode(page_table, max_pages_per_seq, context_lens, batch,
                                                max_context_len, num_pages, status, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "validate_decode");
    return MSA_OK;
}

msa_status msa_mxfp8_quantize(const uint16_t *in, int rows, int cols, uint8_t *out_q, uint8_t *out_scale,
                              void *stream) {
    if (!in || !out_q || !out_scale) return fail(MSA_ERR_INVALID_ARG, "in, out_q and out_scale must be non-NULL");
    if (rows < 1 || cols < 32 || cols % 32)
        return fail(MSA_ERR_INVALID_ARG, "rows must be >= 1 and cols a positive multiple of 32 (got %d x %d)",
                    rows, cols);
    const hipError_t e = launch_mxfp8_quantize(in, int64_t(rows) * cols, out_q, out_scale, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mxfp8_quantize");
    return MSA_OK;
}

}  // extern "C"
