/*
 * CPU oracle for the MiniMax-M3 two-step block-sparse GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, literal reference the
 * GPU library is checked against.  Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * (the HIP library and its Python binding) never does, and the two share no
 * source, header, table or helper.
 *
 * Everything is computed from the definitions, in fp64, with no tiling, no
 * online softmax and no reordering beyond what the definitions state.
 * Sources (titles of the public pages and the part of each that defines a
 * step):
 *   [TRT]  TensorRT-LLM, "MiniMaxM3SparseAttentionConfig": class description
 *          (two-step method: index branch scores K/V blocks and takes a top-k
 *          per (kv head, query token) with init blocks forced at the head and
 *          local blocks forced at the tail; sparse GQA attention over only the
 *          selected blocks; side index-K cache [num_slots,1,index_dim] beside
 *          the main paged K/V), fields sparse_block_size, sparse_topk_blocks,
 *          sparse_init_blocks, sparse_local_blocks, sparse_score_type ('max'),
 *          indexer_kv_dtype ('fp8' = unscaled E4M3 with FP32 accumulation).
 *   [MSA]  NeMo AutoModel, "nemo_automodel.components.models.minimax_m3_vl.msa":
 *          MSAMicrobatch.select_blocks (choices restricted to the query's own
 *          document; hard top-k over unnormalised QK maxima; int32
 *          [4, tokens, 16] document-local ids padded with -1), the document-map
 *          classmethod (0 = padding, each document one contiguous run),
 *          MSAMicrobatch.build (causal only), sparse_attention (bf16 q
 *          [tokens,64,128], k/v [tokens,4,128] -> bf16 out [tokens,64,128]),
 *          _SparseAttention.backward (grad_out -> dq, dk, dv; no gradient
 *          for the selection).
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes): raw dot products for scores (no 1/sqrt(d)); keys j <= t only, in
 * scores and attention; block 0 starts at the document's first token; the
 * local blocks are the tail of the query's causal range c-local+1..c; forced
 * blocks take top-k slots; forced sets are a union counted once; rows are
 * emitted ascending with -1 last; ties in score prefer the lower block id;
 * index head g selects for KV head g; query head h uses KV head h/16; a decode
 * query is the last token L-1 of its request, whose keys are read through
 * slot = page_table[r, j/128]*128 + j%128.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_QH 64   /* query heads                        */
#define ORC_KVH 4   /* key/value heads                    */
#define ORC_IH 4    /* index heads                        */
#define ORC_D 128   /* head dim = index dim               */
#define ORC_BS 128  /* key block size                     */
#define ORC_GROUP (ORC_QH / ORC_KVH)

enum { ORC_BF16 = 0, ORC_E4M3 = 1 };

/* ---- storage formats ---------------------------------------------------- */

/* bf16 is the upper 16 bits of an IEEE binary32. */
static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent 0
 * encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no infinity;
 * the largest finite magnitude is 1.75 * 2^8 = 448. */
static double e4m3_value(uint8_t byte) {
    int s = byte >> 7, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);          /* (m/8) * 2^-6      */
    else
        mag = ldexp(8.0 + m, e - 10);        /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

static double index_elem(const void *base, int dtype, size_t i) {
    if (dtype == ORC_E4M3) return e4m3_value(((const uint8_t *)base)[i]);
    return bf16_value(((const uint16_t *)base)[i]);
}

/* exported so the tests can pin the decoders against library conversions */
double oracle_bf16_value(uint16_t bits) { return bf16_value(bits); }
double oracle_e4m3_value(uint8_t byte) { return e4m3_value(byte); }

/* ---- geometry (document map from cu_seqlens) ---------------------------- */

/* Document d of compact token t: cu[d] <= t < cu[d+1].  -1 if out of range. */
static int doc_of(const int32_t *cu, int ndocs, int t) {
    for (int d = 0; d < ndocs; ++d)
        if (cu[d] <= t && t < cu[d + 1]) return d;
    return -1;
}

static int check_cu(const int32_t *cu, int ndocs) {
    if (ndocs < 1 || cu[0] != 0) return 1;
    for (int d = 0; d < ndocs; ++d)
        if (cu[d + 1] <= cu[d]) return 1;
    return 0;
}

/* Query block c = p div 128 of each listed token (p = position in its doc). */
int oracle_query_blocks(const int32_t *cu, int ndocs, const int32_t *tokens,
                        int ntok, int32_t *c_out) {
    if (check_cu(cu, ndocs)) return 1;
    for (int i = 0; i < ntok; ++i) {
        int d = doc_of(cu, ndocs, tokens[i]);
        if (d < 0) return 2;
        c_out[i] = (tokens[i] - cu[d]) / ORC_BS;
    }
    return 0;
}

/* ---- step 1: block scores ----------------------------------------------- */

/* Score of query token t, index head h, against key block b of its own
 * document: the largest raw dot product iq[t,h,:] . ik[j,0,:] over keys j of
 * block b with j <= t ([TRT] sparse_score_type 'max'; [MSA] select_blocks:
 * unnormalised QK maxima, own document; causal per MSAMicrobatch.build).
 * Entries for blocks past the query's own block are -inf (not candidates). */
int oracle_scores(const void *iq, const void *ik, int dtype, const int32_t *cu,
                  int ndocs, const int32_t *tokens, int ntok, int nb_max,
                  double *S /* [ntok][4][nb_max] */) {
    if (check_cu(cu, ndocs) || nb_max < 1) return 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < ntok; ++i) {
        int t = tokens[i];
        int d = doc_of(cu, ndocs, t);
        if (d < 0) { bad |= 1; continue; }
        int start = cu[d];
        int c = (t - start) / ORC_BS;
        if (c >= nb_max) { bad |= 1; continue; }
        for (int h = 0; h < ORC_IH; ++h) {
            double *row = S + ((size_t)i * ORC_IH + h) * nb_max;
            for (int b = 0; b < nb_max; ++b) row[b] = -INFINITY;
            for (int b = 0; b <= c; ++b) {
                double best = -INFINITY;
                for (int j = start + b * ORC_BS; j < start + (b + 1) * ORC_BS && j <= t; ++j) {
                    double dot = 0.0;
                    for (int x = 0; x < ORC_D; ++x)
                        dot += index_elem(iq, dtype, ((size_t)t * ORC_IH + h) * ORC_D + x) *
                               index_elem(ik, dtype, (size_t)j * ORC_D + x);
                    if (dot > best) best = dot;
                }
                row[b] = best;
            }
        }
    }
    return bad ? 2 : 0;
}

/* ---- step 2: forced blocks + hard top-k ---------------------------------- */

typedef struct { double s; int b; } cand_t;

/* Order: higher score first; equal scores: lower block id first. */
static int cand_cmp(const void *a, const void *b) {
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->b > y->b) - (x->b < y->b);
}

/* One row: candidates are blocks 0..c.  Forced F = {b < init} U
 * {c-local+1 <= b <= c} ([TRT] sparse_init_blocks / sparse_local_blocks,
 * forced regardless of score).  The remaining topk-|F| slots go to the
 * highest-scoring non-forced candidates ([TRT] sparse_topk_blocks; [MSA]
 * select_blocks: hard top-k).  Output ascending, padded with -1 ([MSA]
 * select_blocks Returns).  margin = s_R - s_{R+1} over the sorted non-forced
 * scores (R = free slots), +inf when no choice is contested. */
static void select_row(const double *S, int c, int topk, int init, int local,
                       int32_t *out, double *margin) {
    int n = c + 1;
    unsigned char *mark = (unsigned char *)calloc((size_t)n, 1);
    cand_t *cand = (cand_t *)malloc(sizeof(cand_t) * (size_t)n);
    int nforced = 0, ncand = 0;
    for (int b = 0; b < n; ++b) {
        int forced = (b < init) || (b >= c - local + 1);
        if (forced) { mark[b] = 1; ++nforced; }
        else { cand[ncand].s = S[b]; cand[ncand].b = b; ++ncand; }
    }
    int R = topk - nforced;
    if (R < 0) R = 0;
    qsort(cand, (size_t)ncand, sizeof(cand_t), cand_cmp);
    int take = ncand < R ? ncand : R;
    for (int i = 0; i < take; ++i) mark[cand[i].b] = 1;
    *margin = (R > 0 && ncand > R) ? cand[R - 1].s - cand[R].s : INFINITY;
    int k = 0;
    for (int b = 0; b < n && k < topk; ++b)
        if (mark[b]) out[k++] = b;
    while (k < topk) out[k++] = -1;
    free(cand);
    free(mark);
}

int oracle_select(const double *S /* [n][4][nb_max] */, const int32_t *c /* [n] */,
                  int n, int nb_max, int topk, int init, int local,
                  int32_t *q2k /* [n][4][topk] */, double *margin /* [n][4] */) {
    if (topk < 1 || init < 0 || local < 0 || init + local > topk) return 1;
    for (int i = 0; i < n; ++i)
        if (c[i] < 0 || c[i] >= nb_max) return 2;
#pragma omp parallel for schedule(dynamic, 16)
    for (int i = 0; i < n; ++i)
        for (int h = 0; h < ORC_IH; ++h)
            select_row(S + ((size_t)i * ORC_IH + h) * nb_max, c[i], topk, init, local,
                       q2k + ((size_t)i * ORC_IH + h) * topk, margin + (size_t)i * ORC_IH + h);
    return 0;
}

/* ---- step 3: sparse GQA attention ---------------------------------------- */

/* Softmax attention of one query row over the key set K.  z_j = scale *
 * q.k_j, out = sum_j e^(z_j - max z) v_j / sum_j e^(z_j - max z).  An empty
 * key set gives a zero row (never produced by the selection, which always
 * has at least one block containing key t). */
static void attend_keys(const uint16_t *qrow, const uint16_t *const *krows,
                        const uint16_t *const *vrows, int nkeys, double scale,
                        double *z, double *out) {
    for (int x = 0; x < ORC_D; ++x) out[x] = 0.0;
    if (nkeys == 0) return;
    double zmax = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int x = 0; x < ORC_D; ++x) dot += bf16_value(qrow[x]) * bf16_value(krows[j][x]);
        z[j] = scale * dot;
        if (z[j] > zmax) zmax = z[j];
    }
    double denom = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        double w = exp(z[j] - zmax);
        denom += w;
        for (int x = 0; x < ORC_D; ++x) out[x] += w * bf16_value(vrows[j][x]);
    }
    for (int x = 0; x < ORC_D; ++x) out[x] /= denom;
}

/* Prefill: for token t and query head h (KV head g = h/16), the key set is
 * every key j of t's document with j <= t whose document-local block
 * (j - cu[d]) div 128 appears in q2k row (g, t) ([TRT] class description:
 * sparse GQA over only the selected blocks; [MSA] sparse_attention). */
int oracle_attend(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const int32_t *q2k /* [ntok][4][topk] */, int topk,
                  const int32_t *cu, int ndocs, const int32_t *tokens, int ntok,
                  double scale, double *out /* [ntok][64][128] */) {
    if (check_cu(cu, ndocs) || topk < 1) return 1;
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
        const uint16_t **krows = NULL, **vrows = NULL;
        double *z = NULL;
        size_t cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < ntok; ++i) {
            int t = tokens[i];
            int d = doc_of(cu, ndocs, t);
            if (d < 0) { bad |= 1; continue; }
            int start = cu[d];
            size_t need = (size_t)(t - start + 1);
            if (need > cap) {
                cap = need;
                krows = (const uint16_t **)realloc((void *)krows, cap * sizeof *krows);
                vrows = (const uint16_t **)realloc((void *)vrows, cap * sizeof *vrows);
                z = (double *)realloc(z, cap * sizeof *z);
            }
            for (int g = 0; g < ORC_KVH; ++g) {
                const int32_t *row = q2k + ((size_t)i * ORC_KVH + g) * topk;
                int nkeys = 0;
                for (int j = start; j <= t; ++j) {
                    int blk = (j - start) / ORC_BS, sel = 0;
                    for (int s = 0; s < topk; ++s) sel |= (row[s] == blk);
                    if (!sel) continue;
                    krows[nkeys] = k + ((size_t)j * ORC_KVH + g) * ORC_D;
                    vrows[nkeys] = v + ((size_t)j * ORC_KVH + g) * ORC_D;
                    ++nkeys;
                }
                for (int hh = 0; hh < ORC_GROUP; ++hh) {
                    int h = g * ORC_GROUP + hh;
                    attend_keys(q + ((size_t)t * ORC_QH + h) * ORC_D, krows, vrows, nkeys,
                                scale, z, out + ((size_t)i * ORC_QH + h) * ORC_D);
                }
            }
        }
        free((void *)krows);
        free((void *)vrows);
        free(z);
    }
    return bad ? 2 : 0;
}

/* ---- step 3, backward: gradients of the sparse attention ------------------ */

/* The selection is a hard top-k and carries no gradient ([MSA] select_blocks
 * runs under no_grad); the backward differentiates step 3 alone for a fixed
 * q2k ([MSA] _SparseAttention.backward: bf16 grad_out [tokens,64,128] ->
 * dq [tokens,64,128], dk and dv [tokens,4,128]).  With K(t,g) the key set of
 * oracle_attend, z_tj = scale q_th.k_j, lse_th = log sum_{j in K} e^z_tj,
 * P_tj = e^(z_tj - lse_th) and dO = d(loss)/d(out):
 *   dP_tj = dO_th . v_j        D_th = sum_j P_tj dP_tj
 *   dS_tj = P_tj (dP_tj - D_th)
 *   dq_th = scale sum_{j in K(t,g)} dS_tj k_j
 *   dk_jg = scale sum over (t, h in group g) with j in K(t,g) of dS_tj q_th
 *   dv_jg =       sum over the same rows of P_tj dO_th
 * q2k is token-major [T][4][topk] here (row of token t, KV head g). */

/* Whether key j (document start `start`) is in K(t,g): j <= t, same
 * document, block (j - start) div 128 listed in the row. */
static int key_selected(const int32_t *row, int topk, int start, int j, int t) {
    if (j > t || j < start) return 0;
    int blk = (j - start) / ORC_BS;
    for (int s = 0; s < topk; ++s)
        if (row[s] == blk) return 1;
    return 0;
}

static double dot_bf16(const uint16_t *a, const uint16_t *b) {
    double acc = 0.0;
    for (int x = 0; x < ORC_D; ++x) acc += bf16_value(a[x]) * bf16_value(b[x]);
    return acc;
}

/* Phase 1, per query row of the listed tokens: lse, D and dq.  A row with an
 * empty key set has lse = -inf, D = 0, dq = 0. */
int oracle_attend_backward_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const uint16_t *dout, const int32_t *q2k /* [T][4][topk] */,
                                int topk, const int32_t *cu, int ndocs, const int32_t *tokens,
                                int ntok, double scale, double *lse /* [ntok][64] */,
                                double *D /* [ntok][64] */, double *dq /* [ntok][64][128] */) {
    if (check_cu(cu, ndocs) || topk < 1) return 1;
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
        int *keys = NULL;
        double *z = NULL, *dp = NULL;
        size_t cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < ntok; ++i) {
            int t = tokens[i];
            int d = doc_of(cu, ndocs, t);
            if (d < 0) { bad |= 1; continue; }
            int start = cu[d];
            size_t need = (size_t)(t - start + 1);
            if (need > cap) {
                cap = need;
                keys = (int *)realloc(keys, cap * sizeof *keys);
                z = (double *)realloc(z, cap * sizeof *z);
                dp = (double *)realloc(dp, cap * sizeof *dp);
            }
            for (int g = 0; g < ORC_KVH; ++g) {
                const int32_t *row = q2k + ((size_t)t * ORC_KVH + g) * topk;
                int nk = 0;
                for (int j = start; j <= t; ++j)
                    if (key_selected(row, topk, start, j, t)) keys[nk++] = j;
                for (int hh = 0; hh < ORC_GROUP; ++hh) {
                    int h = g * ORC_GROUP + hh;
                    const uint16_t *qr = q + ((size_t)t * ORC_QH + h) * ORC_D;
                    const uint16_t *dor = dout + ((size_t)t * ORC_QH + h) * ORC_D;
                    double *dqr = dq + ((size_t)i * ORC_QH + h) * ORC_D;
                    for (int x = 0; x < ORC_D; ++x) dqr[x] = 0.0;
                    if (nk == 0) {
                        lse[(size_t)i * ORC_QH + h] = -INFINITY;
                        D[(size_t)i * ORC_QH + h] = 0.0;
                        continue;
                    }
                    double zmax = -INFINITY;
                    for (int a = 0; a < nk; ++a) {
                        const uint16_t *kr = k + ((size_t)keys[a] * ORC_KVH + g) * ORC_D;
                        z[a] = scale * dot_bf16(qr, kr);
                        if (z[a] > zmax) zmax = z[a];
                    }
                    double sum = 0.0;
                    for (int a = 0; a < nk; ++a) sum += exp(z[a] - zmax);
                    double l = zmax + log(sum);
                    double Dth = 0.0;
                    for (int a = 0; a < nk; ++a) {
                        const uint16_t *vr = v + ((size_t)keys[a] * ORC_KVH + g) * ORC_D;
                        dp[a] = dot_bf16(dor, vr);
                        Dth += exp(z[a] - l) * dp[a];
                    }
                    for (int a = 0; a < nk; ++a) {
                        double ds = exp(z[a] - l) * (dp[a] - Dth);
                        const uint16_t *kr = k + ((size_t)keys[a] * ORC_KVH + g) * ORC_D;
                        for (int x = 0; x < ORC_D; ++x) dqr[x] += scale * ds * bf16_value(kr[x]);
                    }
                    lse[(size_t)i * ORC_QH + h] = l;
                    D[(size_t)i * ORC_QH + h] = Dth;
                }
            }
        }
        free(keys);
        free(z);
        free(dp);
    }
    return bad ? 2 : 0;
}

/* Phase 2, per listed key j and KV head g: dk and dv summed over the query
 * rows whose key set holds j (tokens t >= j of j's document whose row lists
 * j's block).  lse and D are phase 1's values indexed by token [T][64]; only
 * the rows of those tokens are read. */
int oracle_attend_backward_keys(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const uint16_t *dout, const int32_t *q2k /* [T][4][topk] */,
                                int topk, const int32_t *cu, int ndocs, const double *lse,
                                const double *D, double scale, const int32_t *keys, int nkeys,
                                double *dk /* [nkeys][4][128] */, double *dv /* [nkeys][4][128] */) {
    if (check_cu(cu, ndocs) || topk < 1) return 1;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < nkeys; ++i)
        for (int g = 0; g < ORC_KVH; ++g) {
            int j = keys[i];
            double *dkr = dk + ((size_t)i * ORC_KVH + g) * ORC_D;
            double *dvr = dv + ((size_t)i * ORC_KVH + g) * ORC_D;
            for (int x = 0; x < ORC_D; ++x) dkr[x] = dvr[x] = 0.0;
            int d = doc_of(cu, ndocs, j);
            if (d < 0) { bad |= 1; continue; }
            int start = cu[d], end = cu[d + 1];
            const uint16_t *kr = k + ((size_t)j * ORC_KVH + g) * ORC_D;
            const uint16_t *vr = v + ((size_t)j * ORC_KVH + g) * ORC_D;
            for (int t = j; t < end; ++t) {
                const int32_t *row = q2k + ((size_t)t * ORC_KVH + g) * topk;
                if (!key_selected(row, topk, start, j, t)) continue;
                for (int hh = 0; hh < ORC_GROUP; ++hh) {
                    int h = g * ORC_GROUP + hh;
                    const uint16_t *qr = q + ((size_t)t * ORC_QH + h) * ORC_D;
                    const uint16_t *dor = dout + ((size_t)t * ORC_QH + h) * ORC_D;
                    double p = exp(scale * dot_bf16(qr, kr) - lse[(size_t)t * ORC_QH + h]);
                    double ds = p * (dot_bf16(dor, vr) - D[(size_t)t * ORC_QH + h]);
                    for (int x = 0; x < ORC_D; ++x) {
                        dkr[x] += scale * ds * bf16_value(qr[x]);
                        dvr[x] += p * bf16_value(dor[x]);
                    }
                }
            }
        }
    return bad ? 2 : 0;
}

/* ---- paged decode --------------------------------------------------------- */

/* Physical slot of logical key j of request r: the K/V cache and the side
 * index-K cache share the slot ([TRT] class description). */
static size_t slot_of(const int32_t *pt, int max_pages, int r, int j) {
    return (size_t)pt[(size_t)r * max_pages + j / ORC_BS] * ORC_BS + (size_t)(j % ORC_BS);
}

static int check_decode(const int32_t *ctx, int B, int max_pages) {
    for (int r = 0; r < B; ++r)
        if (ctx[r] < 1 || (ctx[r] + ORC_BS - 1) / ORC_BS > max_pages) return 1;
    return 0;
}

/* Query block of each decode request: the query is token L-1. */
int oracle_decode_query_blocks(const int32_t *ctx, int B, int32_t *c_out) {
    for (int r = 0; r < B; ++r) {
        if (ctx[r] < 1) return 1;
        c_out[r] = (ctx[r] - 1) / ORC_BS;
    }
    return 0;
}

/* Decode scores: request r of length L is one document evaluated only at its
 * last token t = L-1, keys read through the page table. */
int oracle_decode_scores(const void *iq /* [B,4,128] */, const void *ikc /* [slots,1,128] */,
                         int dtype, const int32_t *pt, int max_pages, const int32_t *ctx,
                         int B, int nb_max, double *S /* [B][4][nb_max] */) {
    if (check_decode(ctx, B, max_pages)) return 1;
    for (int r = 0; r < B; ++r)
        if ((ctx[r] - 1) / ORC_BS >= nb_max) return 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int r = 0; r < B; ++r)
        for (int h = 0; h < ORC_IH; ++h) {
            int L = ctx[r], t = L - 1, c = t / ORC_BS;
            double *row = S + ((size_t)r * ORC_IH + h) * nb_max;
            for (int b = 0; b < nb_max; ++b) row[b] = -INFINITY;
            for (int b = 0; b <= c; ++b) {
                double best = -INFINITY;
                for (int j = b * ORC_BS; j < (b + 1) * ORC_BS && j <= t; ++j) {
                    size_t slot = slot_of(pt, max_pages, r, j);
                    double dot = 0.0;
                    for (int x = 0; x < ORC_D; ++x)
                        dot += index_elem(iq, dtype, ((size_t)r * ORC_IH + h) * ORC_D + x) *
                               index_elem(ikc, dtype, slot * ORC_D + x);
                    if (dot > best) best = dot;
                }
                row[b] = best;
            }
        }
    return 0;
}

/* Decode attention for query head h of request r over the keys j <= L-1
 * whose block j div 128 appears in q2k row (h/16, r). */
int oracle_decode_attend(const uint16_t *q /* [B,64,128] */, const uint16_t *kc,
                         const uint16_t *vc /* [slots,4,128] */, const int32_t *pt,
                         int max_pages, const int32_t *ctx, int B,
                         const int32_t *q2k /* [B][4][topk] */, int topk, double scale,
                         double *out /* [B][64][128] */) {
    if (check_decode(ctx, B, max_pages) || topk < 1) return 1;
#pragma omp parallel
    {
        const uint16_t **krows = NULL, **vrows = NULL;
        double *z = NULL;
        size_t cap = 0;
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int r = 0; r < B; ++r)
            for (int g = 0; g < ORC_KVH; ++g) {
                int L = ctx[r];
                if ((size_t)L > cap) {
                    cap = (size_t)L;
                    krows = (const uint16_t **)realloc((void *)krows, cap * sizeof *krows);
                    vrows = (const uint16_t **)realloc((void *)vrows, cap * sizeof *vrows);
                    z = (double *)realloc(z, cap * sizeof *z);
                }
                const int32_t *row = q2k + ((size_t)r * ORC_KVH + g) * topk;
                int nkeys = 0;
                for (int j = 0; j < L; ++j) {
                    int blk = j / ORC_BS, sel = 0;
                    for (int s = 0; s < topk; ++s) sel |= (row[s] == blk);
                    if (!sel) continue;
                    size_t slot = slot_of(pt, max_pages, r, j);
                    krows[nkeys] = kc + (slot * ORC_KVH + g) * ORC_D;
                    vrows[nkeys] = vc + (slot * ORC_KVH + g) * ORC_D;
                    ++nkeys;
                }
                for (int hh = 0; hh < ORC_GROUP; ++hh) {
                    int h = g * ORC_GROUP + hh;
                    attend_keys(q + ((size_t)r * ORC_QH + h) * ORC_D, krows, vrows, nkeys, scale,
                                z, out + ((size_t)r * ORC_QH + h) * ORC_D);
                }
            }
        free((void *)krows);
        free((void *)vrows);
        free(z);
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
