/*
 * msa.h - C ABI of libmsa, MiniMax-M3 two-step block-sparse GQA attention
 * on AMD Instinct MI355X (gfx950).
 *
 * Step one (index branch): index queries [T,4,128] score a single shared
 * index key [T,1,128]; every 128-key block of the query's own document gets
 * the maximum raw dot product over its causal keys; a hard top-k per
 * (KV head, query token) with init blocks forced at the head and local
 * blocks forced at the tail yields int32 q2k [4,T,topk] padded with -1.
 * Step two: GQA softmax attention (64 query heads, 4 KV heads, head dim 128,
 * bf16) over only the selected blocks, for prefill over packed documents and
 * for decode over a paged K/V cache plus a side index-K cache.
 *
 * Sources: TensorRT-LLM "MiniMaxM3SparseAttentionConfig" (class description;
 * fields sparse_num_index_heads, sparse_index_dim, sparse_block_size,
 * sparse_topk_blocks, sparse_init_blocks, sparse_local_blocks,
 * sparse_score_type, indexer_kv_dtype); NeMo AutoModel
 * "nemo_automodel.components.models.minimax_m3_vl.msa" (MSAMicrobatch.
 * select_blocks, sparse_attention, the document-map classmethod,
 * require_msa_support); vLLM "vllm.models.minimax_m3.amd.
 * sparse_attention_nvfp4" (rocm_nvfp4_unsupported_reason).
 *
 * Conventions for every entry point:
 *  - Tensor arguments are caller-owned DEVICE pointers, contiguous,
 *    row-major, in the layouts stated.  bf16 is passed as its uint16_t bit
 *    pattern; E4M3 as uint8_t bytes (OCP E4M3FN).
 *  - Host scalars (token counts, max_seqlen, max_context_len) bound the
 *    launch grids, so no call reads device memory back to the host.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it and return; they never synchronise and never
 *    allocate: scratch memory is the caller's `workspace` (size from the
 *    matching *_workspace_bytes query; any 256-byte-aligned device buffer).
 *  - Host-side argument errors return a non-zero msa_status before any
 *    GPU work is enqueued; msa_last_error() then returns a message
 *    (thread-local).  Contract violations in device data (e.g. a
 *    cu_seqlens that is not increasing, a page id out of range) are not
 *    detected by the compute calls: kernels clamp document bounds to
 *    [0, total_tokens] so they never read outside the buffers the host
 *    scalars describe, but the output is then unspecified.  Page ids must
 *    lie in the cache; a negative page id reads nothing (see the decode
 *    call).  msa_validate_prefill_inputs / msa_validate_decode_inputs check
 *    the device data on request (a debugging aid, off the hot path).
 *  - The same inputs give bitwise identical outputs on every call (no
 *    atomics in any reduction).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARG = 1, /* malformed argument (null pointer, bad size)      */
    MSA_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle  */
    MSA_ERR_WORKSPACE = 3,   /* workspace_bytes below the *_workspace_bytes size */
    MSA_ERR_HIP = 4          /* a HIP launch failed; message has the HIP error   */
} msa_status;

/* Storage and score dtype of index q/k (TensorRT-LLM config, indexer_kv_dtype:
 * 'fp8' means unscaled E4M3 values with FP32 score accumulation). */
typedef enum { MSA_INDEX_BF16 = 0, MSA_INDEX_FP8_E4M3 = 1 } msa_index_dtype;

/* Fixed topology (NeMo msa page, require_msa_support: 64 query heads, 4 KV
 * heads, 128 channels, max block score; TensorRT-LLM config: 4 index heads
 * of dim 128, blocks of 128). */
#define MSA_NUM_HEADS 64
#define MSA_NUM_KV_HEADS 4
#define MSA_HEAD_DIM 128
#define MSA_NUM_INDEX_HEADS 4
#define MSA_INDEX_DIM 128
#define MSA_BLOCK_SIZE 128
#define MSA_MAX_TOPK 16

/* NULL when the kernels serve this layer shape, else a static string saying
 * why not (same role as rocm_nvfp4_unsupported_reason on the vLLM page and
 * the ValueError of require_msa_support on the NeMo page).  Served: the
 * fixed topology above with 1 <= topk <= 16. */
const char *msa_unsupported_reason(int num_heads, int num_kv_heads, int head_dim,
                                   int num_index_heads, int index_dim, int topk,
                                   int block_size);

/* Message of the last failed call on this thread ("" if none). */
const char *msa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int msa_version(void);

/* Workspace sizes in bytes (0 if the arguments are invalid).  The select
 * query takes num_docs besides the token count and the longest document:
 * the workspace holds the sanitised document spans and the per-document
 * tile offsets, whose size grows with the number of documents. */
size_t msa_select_blocks_workspace_bytes(int total_tokens, int num_docs, int max_seqlen);
size_t msa_prefill_workspace_bytes(int total_tokens, int num_docs, int max_seqlen);
/* also 0 above 4194304 tokens */
size_t msa_prefill_backward_workspace_bytes(int total_tokens, int num_docs, int max_seqlen, int topk);
size_t msa_decode_workspace_bytes(int batch, int max_context_len, int topk);

/*
 * Index-branch block selection over packed documents (NeMo msa page,
 * MSAMicrobatch.select_blocks; TensorRT-LLM config class description).
 *
 *  index_q     [T,4,128]  bf16 bits or E4M3 bytes, post norm and RoPE.
 *  index_k     [T,1,128]  same dtype; one key shared by the 4 index heads.
 *  index_dtype msa_index_dtype.
 *  cu_seqlens  int32 [num_docs+1]: 0 = cu[0] < cu[1] < ... < cu[num_docs] = T;
 *              document d is tokens cu[d]..cu[d+1]-1 (compact packed layout).
 *  num_docs >= 1, total_tokens = T >= 1, max_seqlen >= every document length.
 *  topk in [1,16]; init_blocks, local_blocks >= 0, init+local <= topk.
 *  q2k         out int32 [4,T,topk]: row (g,t) lists the document-local block
 *              ids chosen for KV head g and token t, ascending, then -1.
 *              Block b of a document holds its positions 128b..128b+127.  For
 *              a token at position p (c = p div 128) the candidates are blocks
 *              0..c; blocks 0..init-1 and c-local+1..c are forced; the other
 *              slots take the highest-scoring candidates (lower id on ties).
 *  scores_out  optional out fp32 [4, ceil(max_seqlen/128), T] (head, block,
 *              token): the block score max_{j in block b, j<=t} iq.ik
 *              (raw dot, FP32 accumulation) for b <= c; entries b > c are
 *              left unwritten.  NULL to skip.  Blocks before tokens (rather
 *              than [4, T, nb]): the scorer writes one block's scores for
 *              consecutive tokens and the top-k reads one block for
 *              consecutive tokens, both coalesced.
 */
msa_status msa_select_blocks(const void *index_q, const void *index_k, int index_dtype,
                             const int32_t *cu_seqlens, int num_docs, int total_tokens,
                             int max_seqlen, int topk, int init_blocks, int local_blocks,
                             int32_t *q2k, float *scores_out, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Sparse GQA attention over the selected blocks, prefill (NeMo msa page,
 * sparse_attention; TensorRT-LLM config class description, step two).
 *
 *  q [T,64,128], k [T,4,128], v [T,4,128]  bf16 bits.
 *  q2k int32 [4,T,topk] as produced by msa_select_blocks (any order; ids
 *      outside 0..c and -1 contribute no keys; repeats count once).
 *  cu_seqlens / num_docs / total_tokens / max_seqlen as above.
 *  softmax_scale: logits are softmax_scale * q.k.
 *  out [T,64,128] bf16 bits: for query head h (KV head g = h/16) and token t,
 *      softmax attention over keys j of t's document with j <= t whose block
 *      is in q2k row (g,t); fp32 accumulation, rounded to nearest even.
 */
msa_status msa_sparse_attend_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     const int32_t *q2k, int topk, const int32_t *cu_seqlens,
                                     int num_docs, int total_tokens, int max_seqlen,
                                     float softmax_scale, uint16_t *out, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * msa_sparse_attend_prefill that also returns the log-sum-exp of every
 * attention row, the state the backward needs (NeMo msa page,
 * _SparseAttention: the forward saves what the backward uses).
 *
 *  lse out fp32 [T,64]: lse[t,h] = log sum_j exp(softmax_scale * q[t,h].k_j)
 *      over the row's key set (natural log; -inf for an empty key set).
 *  Every other argument, the workspace and the errors are those of
 *  msa_sparse_attend_prefill; lse == NULL is MSA_ERR_INVALID_ARG.
 */
msa_status msa_sparse_attend_prefill_lse(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                         const int32_t *q2k, int topk, const int32_t *cu_seqlens,
                                         int num_docs, int total_tokens, int max_seqlen,
                                         float softmax_scale, uint16_t *out, float *lse, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * Backward of msa_sparse_attend_prefill for a fixed selection (NeMo msa
 * page, _SparseAttention.backward: bf16 grad_out [tokens,64,128] -> dq
 * [tokens,64,128] and dk, dv [tokens,4,128]; the block selection is a hard
 * top-k and receives no gradient).
 *
 *  q, k, v, q2k, topk, cu_seqlens, num_docs, total_tokens, max_seqlen,
 *      softmax_scale: those of the forward call.
 *  out  [T,64,128] bf16: the forward output; lse [T,64] fp32: the forward's
 *      log-sum-exp (msa_sparse_attend_prefill_lse).
 *  dout [T,64,128] bf16: gradient of the loss with respect to out.
 *  dq [T,64,128], dk [T,4,128], dv [T,4,128] out, bf16: with P the rows'
 *      softmax weights, dS = P * (dout.v - rowsum(dout*out)):
 *      dq = softmax_scale * sum_j dS_j k_j; dk_j and dv_j sum softmax_scale *
 *      dS q and P * dout over the query rows (all 16 heads of the KV group)
 *      whose key set holds j; zero for keys no row attends to.  fp32
 *      accumulation in a fixed order (results repeat bit for bit), rounded
 *      to nearest even once.
 *  workspace: msa_prefill_backward_workspace_bytes(T, num_docs, max_seqlen,
 *      topk) bytes of device memory, owned by the caller, no alignment
 *      beyond 256 bytes, contents on entry ignored.
 *  Errors: NULL pointers, bad geometry or scale (MSA_ERR_INVALID_ARG), topk
 *  outside 1..16 or T above 4194304 (MSA_ERR_UNSUPPORTED), a short
 *  workspace (MSA_ERR_WORKSPACE), all before any work is enqueued.
 */
msa_status msa_sparse_attend_prefill_backward(
    const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *out, const float *lse,
    const uint16_t *dout, const int32_t *q2k, int topk, const int32_t *cu_seqlens, int num_docs,
    int total_tokens, int max_seqlen, float softmax_scale, uint16_t *dq, uint16_t *dk, uint16_t *dv,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step over a paged cache (TensorRT-LLM config class description:
 * paged side index-K cache [num_slots,1,index_dim] parallel to the main K/V
 * cache, same slot).  Request r has context length L = context_lens[r]
 * (including the current token, whose K, V and index-K are already in the
 * caches); its query is position L-1.  Logical key j lives in slot
 * page_table[r, j div 128]*128 + j mod 128.  Selection and attention are
 * those of msa_select_blocks / msa_sparse_attend_prefill for that token.
 *
 *  q [B,64,128] bf16; index_q [B,4,128] bf16 or E4M3.
 *  k_cache, v_cache [num_pages*128,4,128] bf16; index_k_cache
 *      [num_pages*128,1,128] in index_dtype.  Slots past L are never used
 *      (they may hold anything, NaN included).
 *  page_table int32 [B,max_pages_per_seq]; entries past ceil(L/128) unread.
 *      Ids must lie in [0, num_pages); a negative id marks an absent page:
 *      nothing of it is read, its block scores -inf and, if forced or
 *      selected, adds no key.
 *  context_lens int32 [B], each in [0, max_context_len]; 0 (or less) marks an
 *      empty (padding) request: nothing of it is read, its out row is zero
 *      and its q2k_out row is all -1.
 *  out [B,64,128] bf16.  q2k_out optional int32 [4,B,topk] (NULL to skip).
 */
msa_status msa_sparse_attend_decode_paged(
    const uint16_t *q, const void *index_q, const uint16_t *k_cache, const uint16_t *v_cache,
    const void *index_k_cache, int index_dtype, const int32_t *page_table,
    int max_pages_per_seq, const int32_t *context_lens, int batch, int max_context_len,
    int topk, int init_blocks, int local_blocks, float softmax_scale, uint16_t *out,
    int32_t *q2k_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * msa_sparse_attend_decode_paged without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The same kernels run
 * with their scratch (block scores, attention partials) in a device array
 * of MSA_NOALLOC_SCRATCH_BYTES that the library holds per GPU from load to
 * process end; the call allocates nothing.
 *
 *  Arguments, outputs and errors are those of msa_sparse_attend_decode_paged;
 *  in addition MSA_ERR_UNSUPPORTED when msa_decode_workspace_bytes(batch,
 *  max_context_len, topk) exceeds MSA_NOALLOC_SCRATCH_BYTES (e.g. batch 128
 *  at 131072 tokens fits; batch 256 at 131072 does not).
 *  The scratch of a GPU is that of the device current on the calling thread
 *  (call with the stream's device current).  Every call on one GPU shares
 *  its array, so calls that overlap on one GPU (several streams, or several
 *  threads) race: serialise them.  No byte of the array needs to start at
 *  zero: each call writes what it reads.
 */
#define MSA_NOALLOC_SCRATCH_BYTES (16u << 20)
msa_status msa_sparse_attend_decode_paged_noalloc(
    const uint16_t *q, const void *index_q, const uint16_t *k_cache, const uint16_t *v_cache,
    const void *index_k_cache, int index_dtype, const int32_t *page_table,
    int max_pages_per_seq, const int32_t *context_lens, int batch, int max_context_len,
    int topk, int init_blocks, int local_blocks, float softmax_scale, uint16_t *out,
    int32_t *q2k_out, void *stream);

/*
 * The same decode step with its output emitted as MXFP8 for the projection
 * that follows (vLLM MiniMax-M3 page, MiniMaxM3SparseRocmNvfp4Impl,
 * forward_decode_mxfp8): equal to msa_mxfp8_quantize of the bf16 output
 * that msa_sparse_attend_decode_paged returns for the same inputs.
 *
 *  out_q     [B, 64*128] E4M3FN bytes, row-major (query head, then d).
 *  out_scale [B, 64*128/32] E8M0 bytes: scale of out_q[r, 32k..32k+31].
 *  Every other argument, the workspace size and the errors are those of
 *  msa_sparse_attend_decode_paged.
 */
msa_status msa_sparse_attend_decode_paged_mxfp8(
    const uint16_t *q, const void *index_q, const uint16_t *k_cache, const uint16_t *v_cache,
    const void *index_k_cache, int index_dtype, const int32_t *page_table,
    int max_pages_per_seq, const int32_t *context_lens, int batch, int max_context_len,
    int topk, int init_blocks, int local_blocks, float softmax_scale, uint8_t *out_q,
    uint8_t *out_scale, int32_t *q2k_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The decode step over an FP8 main K/V cache (TensorRT-LLM config class
 * description, fuse_qkv_index_projection: the MiniMax-M3 MSA path runs with
 * an FP8 main KV cache).  Per-tensor scales: key j's K row is
 * e4m3(k_cache byte) * k_scale and its V row e4m3(v_cache byte) * v_scale.
 *
 *  k_cache, v_cache [num_pages*128, 4, 128] E4M3FN bytes (slots past L are
 *  never used and may hold anything, NaN included).
 *  k_scale, v_scale > 0, finite.
 *  Every other argument, the workspace size and the errors are those of
 *  msa_sparse_attend_decode_paged.
 */
msa_status msa_sparse_attend_decode_paged_fp8kv(
    const uint16_t *q, const void *index_q, const uint8_t *k_cache, const uint8_t *v_cache,
    float k_scale, float v_scale, const void *index_k_cache, int index_dtype,
    const int32_t *page_table, int max_pages_per_seq, const int32_t *context_lens, int batch,
    int max_context_len, int topk, int init_blocks, int local_blocks, float softmax_scale,
    uint16_t *out, int32_t *q2k_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Paged-cache insertion: the write that precedes decode (TensorRT-LLM config
 * class description, fuse_qkv_index_projection: the norm/RoPE/cache-insertion
 * producer; the side index-K cache parallel to the main K/V cache, same
 * slot).  Only the write: the rows arrive normed and RoPE'd.
 *
 *  k, v          [num_tokens, 4, 128] bf16 bits; index_k [num_tokens, 1, 128]
 *                bf16 bits.
 *  slot_mapping  int32 [num_tokens]: token n goes to slot slot_mapping[n]
 *                (= page * 128 + offset); negative slots, and slots
 *                >= num_slots, are skipped.  Slots must be distinct.
 *  k_cache, v_cache [num_slots, 4, 128] bf16; index_k_cache
 *                [num_slots, 1, 128] in index_dtype: bf16 rows are copied,
 *                MSA_INDEX_FP8_E4M3 stores unscaled E4M3FN (nearest value,
 *                ties to the even code, magnitudes past 448 saturate).
 *  Slots not named are left untouched.  No workspace.
 */
msa_status msa_cache_insert(const uint16_t *k, const uint16_t *v, const uint16_t *index_k,
                            const int32_t *slot_mapping, int num_tokens, int index_dtype,
                            uint16_t *k_cache, uint16_t *v_cache, void *index_k_cache,
                            int num_slots, void *stream);

/*
 * MXFP8 quantisation of bf16 values (the encoding of the decode output
 * above; OCP Microscaling blocks of 32 consecutive values along a row).
 *
 *  in        [rows, cols] bf16 bits, finite; cols a positive multiple of 32.
 *  out_q     [rows, cols] E4M3FN bytes: the value nearest to x / 2^s (ties
 *            to the even code, magnitudes past 448 saturate to 448, the
 *            sign of x kept).
 *  out_scale [rows, cols/32] E8M0 bytes s + 127 per block, where
 *            s = floor(log2(max |x| over the block)) - 8, clamped to
 *            [-127, 127]; an all-zero block gets code 0.
 *  No workspace.  MSA_ERR_INVALID_ARG for NULL pointers or bad sizes.
 */
msa_status msa_mxfp8_quantize(const uint16_t *in, int rows, int cols, uint8_t *out_q,
                              uint8_t *out_scale, void *stream);

/*
 * Debug validators of the device-side data contract (a debugging aid: the
 * compute calls never run them).  Each enqueues one small kernel on
 * `stream` that reads the device data and writes a status pair:
 *   status[0] = OR of msa_invalid_bits (0 when the data is valid),
 *   status[1] = the lowest offending document (prefill) or request
 *               (decode), -1 when valid.
 * `status` is caller-owned device memory of 2 int32; both words are
 * overwritten (no clearing needed).  The host scalars are those of the
 * compute call; host-side errors return MSA_ERR_INVALID_ARG as there.
 *
 * msa_validate_prefill_inputs follows the document-map rules of the NeMo
 * msa page (the document-map classmethod's ValueErrors: no empty or
 * interrupted document, coordinates within range): cu_seqlens[0] == 0,
 * strictly increasing, cu_seqlens[num_docs] == total_tokens, every length
 * <= max_seqlen.
 *
 * msa_validate_decode_inputs checks, for every request, context_lens[r] in
 * [0, max_context_len] and every page id it uses (blocks below
 * ceil(L/128)) in [0, num_pages), num_pages being the caches' page count
 * (TensorRT-LLM config class description: main K/V and side index-K share
 * the slots).
 */
typedef enum {
    MSA_INVALID_CU_START = 1,     /* cu_seqlens[0] != 0                       */
    MSA_INVALID_CU_END = 2,       /* cu_seqlens[num_docs] != total_tokens     */
    MSA_INVALID_DOC_EMPTY = 4,    /* a document of length <= 0                */
    MSA_INVALID_DOC_LONG = 8,     /* a document longer than max_seqlen        */
    MSA_INVALID_CU_RANGE = 16,    /* an offset outside [0, total_tokens]      */
    MSA_INVALID_CONTEXT_LEN = 32, /* a context length outside [0, max_ctx]    */
    MSA_INVALID_PAGE_ID = 64      /* a used page id outside [0, num_pages)    */
} msa_invalid_bits;

msa_status msa_validate_prefill_inputs(const int32_t *cu_seqlens, int num_docs, int total_tokens,
                                       int max_seqlen, int32_t *status, void *stream);
msa_status msa_validate_decode_inputs(const int32_t *page_table, int max_pages_per_seq,
                                      const int32_t *context_lens, int batch, int max_context_len,
                                      int num_pages, int32_t *status, void *stream);

/*
 * Benchmark instrumentation (not part of the method).  Arms the NEXT
 * entry-point call on this thread to record caller-created hipEvent_t
 * handles on its stream: events[0] before its first kernel, events[i]
 * before kernel i, events[k] after its last kernel (k = kernels launched).
 * The call consumes the arming (one-shot); it records at most `count`
 * events.  msa_timing_kernel_count() then returns k and
 * msa_timing_kernel_name(i) the name of kernel i of that call.  Events stay
 * owned by the caller; pass count = 0 to disarm.
 */
void msa_set_timing_events(void *const *events, int count);
int msa_timing_kernel_count(void);
const char *msa_timing_kernel_name(int i);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
