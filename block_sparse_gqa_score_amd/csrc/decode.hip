// Paged decode: selection and sparse GQA attention for one query token per
// request, over a paged K/V cache plus a side index-K cache that shares its
// slots (TensorRT-LLM "MiniMaxM3SparseAttentionConfig", class description;
// vLLM "vllm.models.minimax_m3.amd.sparse_attention_nvfp4", decode path).
// Request r with context length L is one document evaluated at its last
// position L-1; logical key j lives in slot pt[r, j/128]*128 + j%128.
//
// Kernels (one pass over the caches, HBM-bound):
//   decode_scores_stream_kernel - bf16 index keys: persistent one-wave
//       workgroups over equal ranges of the flattened page list, half pages
//       double-buffered in registers, MFMA 16x16x32 against the 4 index
//       heads, slots >= L masked, per-page max.
//   decode_scores_kernel - E4M3 index keys: one wave per (request, page),
//       MFMA 16x16x128 with unit scales.
//   decode_attend_stream_kernel - one workgroup per 8 selected slots of a
//       (KV head, request) (fewer for small batches, so the grid still
//       covers the CUs).  Each wave first selects the row's blocks from
//       the scores: the R-th largest score is bisected on order-preserving
//       score bits with wave-wide counts, over the few candidates at or
//       above the R-th largest lane maximum (compacted one per lane), or
//       over all candidates when ties leave too many; then an ascending
//       ballot-compacted emit.  Ties go to the lower block id, and forced
//       init/local blocks are always kept.  Then it streams its 32 keys of the
//       next block through its own LDS ring while computing the current one:
//       S^T = K Q^T and O^T = V^T P^T on MFMA 16x16x32 (16 query heads = N),
//       with an online softmax across the blocks; the 4 waves are merged in
//       LDS into one (O, m, l) partial per workgroup.
//   decode_combine_kernel - per (request, KV head): log-sum-exp merge of the
//       row's partials (one per attention workgroup) in fixed order, bf16
//       output (or, for the MXFP8 variant, that bf16 output encoded as E4M3
//       + E8M0 per 32 values).
#include "msa_internal.hpp"
#include "mxfp8.hpp"

namespace msa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDecPagesPerWg = 1;  // pages (one wave each) per score workgroup
}  // namespace

// ---------------------------------------------------------------------------
// G4: per-page index scores
// ---------------------------------------------------------------------------
template <bool kFp8, int kPpw>  // kPpw pages (one wave each) per workgroup
__global__ __launch_bounds__(64 * kPpw) void decode_scores_kernel(
    const uint8_t *__restrict__ iq, const uint8_t *__restrict__ ikc, const int32_t *__restrict__ pt,
    int max_pages, const int32_t *__restrict__ ctx, int max_ctx, int nb_max, float *__restrict__ S) {
    const int r = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pi = blockIdx.x * kPpw + wave;
    // the page-table entry is fetched together with the context length (an
    // entry past the context is in bounds and simply unused)
    const int page = pt[size_t(r) * max_pages + min(pi, max_pages - 1)];
    const int L = min(ctx[r], max_ctx);  // <= 0: an empty request, nothing to score
    asm volatile("" ::"v"(page), "v"(L));  // keep the two loads ahead of the branch
    const int nb = L > 0 ? (L + kBlock - 1) / kBlock : 0;
    if (pi >= nb) return;
    const int n = lane & 15, qd = lane >> 4;
    // a negative page id marks an absent block: its keys are read from page 0
    // (in bounds) and its score is -inf
    const size_t slot0 = size_t(max(page, 0)) * kBlock;
    constexpr int kRowBytes = kFp8 ? 128 : 256;
    const uint8_t *kbase = ikc + slot0 * kRowBytes;
    const uint8_t *qrow = iq + (size_t(r) * kIdxHeads + (n & 3)) * kRowBytes;

    f32x4 acc[8];
    if constexpr (kFp8) {
        // lane (m, qd) holds bytes 32qd..32qd+31 of its row (k order is ours).
        u32x4 qa = n < kIdxHeads ? *(const u32x4 *)(qrow + 32 * qd) : u32x4{0, 0, 0, 0};
        u32x4 qc = n < kIdxHeads ? *(const u32x4 *)(qrow + 32 * qd + 16) : u32x4{0, 0, 0, 0};
        const i32x8 qb = {(int)qa[0], (int)qa[1], (int)qa[2], (int)qa[3],
                          (int)qc[0], (int)qc[1], (int)qc[2], (int)qc[3]};
        u32x4 ka[8], kc[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const uint8_t *src = kbase + (16 * mt + n) * kRowBytes + 32 * qd;
            ka[mt] = *(const u32x4 *)src;
            kc[mt] = *(const u32x4 *)(src + 16);
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const i32x8 a = {(int)ka[mt][0], (int)ka[mt][1], (int)ka[mt][2], (int)ka[mt][3],
                             (int)kc[mt][0], (int)kc[mt][1], (int)kc[mt][2], (int)kc[mt][3]};
            acc[mt] = mfma_16x16x128_e4m3(a, qb, f32x4{});
        }
    } else {
        // lane (m, qd), step ks holds 16-byte chunk 4ks + qd of its row (the
        // four lanes of a row read 64 contiguous bytes per instruction).
        bf16x8 qb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[ks] = n < kIdxHeads
                         ? __builtin_bit_cast(bf16x8, *(const u32x4 *)(qrow + 16 * (4 * ks + qd)))
                         : bf16x8{};
        u32x4 ka[8][4];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                ka[mt][ks] = *(const u32x4 *)(kbase + (16 * mt + n) * kRowBytes + 16 * (4 * ks + qd));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            acc[mt] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc[mt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, ka[mt][ks]), qb[ks], acc[mt]);
        }
    }
    // lane (n, qd) holds slots 16mt + 4qd + i of column n (index head n < 4)
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = pi * kBlock + 16 * mt + 4 * qd + i;
            mx = fmaxf(mx, j < L ? acc[mt][i] : -INFINITY);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (page < 0) mx = -INFINITY;
    if (qd == 0 && n < kIdxHeads) S[(size_t(r) * kIdxHeads + n) * nb_max + pi] = mx;
}

// Streaming variant for bf16 index keys: kScoreWaves persistent one-wave
// workgroups share the flattened list of pages of all requests, each taking
// an equal contiguous range of whole pages.  A page is contracted as two
// half pages (64 keys); the wave double-buffers half pages in registers (the
// next one loads while the current one is contracted) and stores the page's
// scores after its second half.
namespace {
constexpr int kScoreWaves = 2048;

struct HalfPage {
    u32x4 k[4][4];  // [M-tile][k-step]: keys 16mt + n of the half page, chunk 4ks + qd
    bool absent;    // negative page id: the keys came from page 0 and do not count
};

// Pages of request r; a context length <= 0 marks an empty request (none).
__device__ __forceinline__ int pages_of(const int32_t *ctx, int r, int max_ctx) {
    const int L = min(ctx[r], max_ctx);
    return L > 0 ? (L + kBlock - 1) / kBlock : 0;
}
}  // namespace

__global__ __launch_bounds__(64) void decode_scores_stream_kernel(
    const uint16_t *__restrict__ iq, const uint16_t *__restrict__ ikc, const int32_t *__restrict__ pt,
    int max_pages, const int32_t *__restrict__ ctx, int max_ctx, int B, int nb_max, float *__restrict__ S) {
    const int lane = threadIdx.x;
    const int n = lane & 15, qd = lane >> 4;
    // total pages (a wave scan per 64 requests) and this wave's page range [p0, p1)
    int total = 0;
    for (int base = 0; base < B; base += 64) {
        int x = base + lane < B ? pages_of(ctx, base + lane, max_ctx) : 0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
        total += x;
    }
    const int wid = blockIdx.x;
    const int p0 = int((int64_t(total) * wid) / kScoreWaves);
    const int p1 = int((int64_t(total) * (wid + 1)) / kScoreWaves);
    if (p0 >= p1) return;
    // request r holding global page p0, and p0's page index within it
    int r = 0, before = 0;
    for (int base = 0; base < B; base += 64) {
        const int rr = base + lane;
        const int cnt = rr < B ? pages_of(ctx, rr, max_ctx) : 0;
        int x = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        const int excl = before + x - cnt;  // pages before request rr
        const uint64_t m = __ballot(rr < B && excl <= p0 && p0 < excl + cnt);
        if (m) {
            const int src = __ffsll((long long)m) - 1;
            r = base + src;
            before = __shfl(excl, src);
            break;
        }
        before += __shfl(x, 63);
    }
    int Lr = min(ctx[r], max_ctx);  // >= 1: request r holds page p0
    int npr = (Lr + kBlock - 1) / kBlock;

    auto load_q = [&](int rr, bf16x8 (&qb)[4]) {
        const uint16_t *qrow = iq + (size_t(rr) * kIdxHeads + (n & 3)) * kDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[ks] = n < kIdxHeads ? __builtin_bit_cast(bf16x8, *(const u32x4 *)(qrow + 8 * (4 * ks + qd)))
                                   : bf16x8{};
    };
    auto load_half = [&](int rr, int pg, int half, HalfPage &h) {
        const int page = pt[size_t(rr) * max_pages + pg];
        h.absent = page < 0;
        const uint16_t *kbase = ikc + (size_t(max(page, 0)) * kBlock + 64 * half) * kDim;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                h.k[mt][ks] = *(const u32x4 *)(kbase + (16 * mt + n) * kDim + 8 * (4 * ks + qd));
    };
    // max over the half page's keys < L for index head column n
    auto half_max = [&](const HalfPage &h, const bf16x8 (&qb)[4], int pg, int half, int L) {
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma_16x16x32(__builtin_bit_cast(bf16x8, h.k[mt][ks]), qb[ks], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = pg * kBlock + 64 * half + 16 * mt + 4 * qd + i;
                mx = fmaxf(mx, j < L ? acc[i] : -INFINITY);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        return h.absent ? -INFINITY : mx;
    };

    bf16x8 qb[4];
    load_q(r, qb);
    int pg = p0 - before;  // page of request r
    HalfPage h0, h1;
    load_half(r, pg, 0, h0);
    for (int p = p0; p < p1; ++p) {
        // first half (in h0); the second half loads meanwhile
        load_half(r, pg, 1, h1);
        float pmax = half_max(h0, qb, pg, 0, Lr);
        // next page's first half loads while the second half is contracted
        int rn = r, pgn = pg + 1;
        if (pgn == npr && p + 1 < p1) {  // the next non-empty request holds page p + 1
            pgn = 0;
            do { ++rn; } while (pages_of(ctx, rn, max_ctx) == 0);
        }
        if (p + 1 < p1) load_half(rn, pgn, 0, h0);
        pmax = fmaxf(pmax, half_max(h1, qb, pg, 1, Lr));
        if (qd == 0 && n < kIdxHeads) S[(size_t(r) * kIdxHeads + n) * nb_max + pg] = pmax;
        if (rn != r) {
            r = rn;
            Lr = min(ctx[r], max_ctx);
            npr = (Lr + kBlock - 1) / kBlock;
            load_q(r, qb);
        }
        pg = pgn;
    }
}

hipError_t launch_decode_scores(const void *iq, const void *ikc, bool fp8, const int32_t *pt,
                                int max_pages, const int32_t *ctx, int B, int max_ctx, int nb_max, float *S,
                                hipStream_t stream) {
    // one page per 64-thread workgroup: measured against 2, 4, 8 and 16 pages
    // per workgroup, the finest grain spreads the uneven request lengths best
    const dim3 grid(ceil_div(nb_max, kDecPagesPerWg), B);
    if (fp8)
        hipLaunchKernelGGL((decode_scores_kernel<true, kDecPagesPerWg>), grid, dim3(64 * kDecPagesPerWg), 0,
                           stream, (const uint8_t *)iq, (const uint8_t *)ikc, pt, max_pages, ctx, max_ctx,
                           nb_max, S);
    else
        hipLaunchKernelGGL(decode_scores_stream_kernel, dim3(kScoreWaves), dim3(64), 0, stream,
                           (const uint16_t *)iq, (const uint16_t *)ikc, pt, max_pages, ctx, max_ctx, B, nb_max,
                           S);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// G5: top-k per (request, index head), one wave each
// ---------------------------------------------------------------------------
// Number of lanes whose predicate holds, summed over the wave (scalar).
__device__ __forceinline__ int wave_count(bool pred) { return __popcll(__ballot(pred)); }

// Selection for one (request, index head) row by one wave: forced blocks
// plus the R = topk - forced highest-scoring candidates (ties to the lower
// block id), ascending, then -1.  The R-th largest order value is found by
// bisection on its bits with wave-wide counts.  out holds kMaxTopk + 128
// entries: the row, a dump slot per lane, then 64 entries of working space
// (out[0..63] also serves as working space before the row is written).
template <int kCpl>  // candidates per lane: blocks lane + 64*i
__device__ __forceinline__ void select_row(const float *__restrict__ srow, int nb_max, int c, int topk,
                                           int init, int local, int lane, int32_t *out) {
    const int R = topk - forced_count(c, init, local);
    // Every lane loads all its entries of the row at once (the index clamped
    // into the row; entries past c are never candidates): a conditional load
    // per candidate would wait for each in turn.
    float sv[kCpl];
#pragma unroll
    for (int i = 0; i < kCpl; ++i) sv[i] = srow[min(lane + 64 * i, nb_max - 1)];
    // order bits of each non-forced candidate; 0 marks "not a candidate"
    uint32_t u[kCpl];
#pragma unroll
    for (int i = 0; i < kCpl; ++i) {
        const int b = lane + 64 * i;
        u[i] = (b <= c && !is_forced(b, c, init, local)) ? max(float_order_bits(sv[i]), 1u) : 0u;
    }
    // Number of candidates >= x over the wave: each lane counts its own, and
    // the lane counts (< 2^kBits) are summed one bit at a time with ballots.
    constexpr int kBits = kCpl < 2 ? 1 : kCpl < 4 ? 2 : kCpl < 8 ? 3 : kCpl < 16 ? 4 : kCpl < 32 ? 5
                        : kCpl < 64 ? 6 : kCpl < 128 ? 7 : 8;
    auto count_ge = [&](uint32_t x) {
        int cl = 0;
#pragma unroll
        for (int i = 0; i < kCpl; ++i) cl += u[i] >= x ? 1 : 0;
        int tot = 0;
#pragma unroll
        for (int k = 0; k < kBits; ++k) tot += wave_count((cl >> k) & 1) << k;
        return tot;
    };
    // thr = largest x with #{u >= x} >= R, the R-th largest order value.
    //
    // Fast path: the R lanes whose own maxima are the R largest each hold a
    // distinct candidate >= lb, the R-th largest lane maximum, so thr >= lb
    // and every candidate that decides thr is >= lb.  Those (typically about
    // R of them) are compacted one per lane into out[0..63], and thr is
    // bisected over them with one compare per step.  The counts #{>= x} it
    // sees equal the full row's for every x >= lb and are >= R below lb, so
    // it yields the same thr.  More than 64 of them (ties), or fewer than R
    // lanes with a candidate, take the general path over all candidates.
    const uint64_t below = (1ull << lane) - 1ull;
    auto select1 = [&](uint32_t v) {  // R-th largest of one value per lane
        uint32_t t = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t trial = t | (1u << bit);
            if (wave_count(v >= trial) >= R) t = trial;
        }
        return t;
    };
    uint32_t thr = 0;
    if (R > 0) {
        uint32_t lm = 0;
#pragma unroll
        for (int i = 0; i < kCpl; ++i) lm = max(lm, u[i]);
        const uint32_t lb = select1(lm);
        if (lb > 0) {
            int kept = 0;
#pragma unroll
            for (int i = 0; i < kCpl; ++i) {
                const bool keep = u[i] >= lb;
                const uint64_t m = __ballot(keep);
                const int pos = kept + __popcll(m & below);
                if (keep && pos < 64) {
                    out[pos] = int32_t(u[i]);
                    out[kMaxTopk + 64 + pos] = lane + 64 * i;
                }
                kept += __popcll(m);
            }
            if (kept <= 64) {
                const uint32_t v0 = uint32_t(out[lane]);
                const int b0 = out[kMaxTopk + 64 + lane];
                const uint32_t v = lane < kept ? v0 : 0u;
                thr = select1(v);
                // The survivors are in ascending block order, and every
                // non-forced block lies between the forced head (< init) and
                // tail (> c - local).  So the row is the head, the taken
                // survivors in order, then the tail.
                const int n_gt_fast = wave_count(v > thr);
                const bool tie = v != 0u && v == thr;
                const int tie_rank = __popcll(__ballot(tie) & below);
                const bool take = v > thr || (tie && tie_rank < R - n_gt_fast);
                const int n_head = min(init, c + 1);
                const int tail_lo = local > 0 ? max(c - local + 1, n_head) : c + 1;
                const int pos = n_head + __popcll(__ballot(take) & below);
                if (take) out[pos] = b0;
                for (int j = lane; j < n_head; j += 64) out[j] = j;
                for (int j = lane; tail_lo + j <= c; j += 64) out[n_head + R + j] = tail_lo + j;
                return;
            }
        }
    }
    // General path: bisected on the high 16 bits first.  When exactly R
    // candidates reach that prefix, the R-th largest is their minimum;
    // otherwise (ties in the prefix) the bisection continues over the low
    // 16 bits.
    int n_gt = 0;  // #{u > thr}
    if (R > 0) {
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t trial = thr | (1u << bit);
            if (count_ge(trial) >= R) thr = trial;
        }
        if (count_ge(thr) == R) {
            uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
            for (int i = 0; i < kCpl; ++i) mn = u[i] >= thr ? min(mn, u[i]) : mn;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mn = min(mn, uint32_t(__shfl_xor(int(mn), o)));
            thr = mn;
        } else {
            for (int bit = 15; bit >= 0; --bit) {
                const uint32_t trial = thr | (1u << bit);
                if (count_ge(trial) >= R) thr = trial;
            }
        }
        n_gt = thr != 0xFFFFFFFFu ? count_ge(thr + 1u) : 0;
    }
    const int ties_wanted = R > 0 ? R - n_gt : 0;  // equal-to-threshold picks, lowest ids first
    int ties_seen = 0, emitted = 0;
    // ascending emit; a lane that takes nothing writes its own dump slot
    // out[kMaxTopk + lane], so the stores need no branch
#pragma unroll
    for (int i = 0; i < kCpl; ++i) {
        const int b = lane + 64 * i;
        const bool forced = b <= c && is_forced(b, c, init, local);
        const bool tie = R > 0 && u[i] != 0 && u[i] == thr;
        const uint64_t tie_mask = __ballot(tie);
        const int tie_rank = ties_seen + __popcll(tie_mask & below);
        ties_seen += __popcll(tie_mask);
        const bool take = forced || (R > 0 && u[i] != 0 && (u[i] > thr || (tie && tie_rank < ties_wanted)));
        const uint64_t take_mask = __ballot(take);
        const int pos = emitted + __popcll(take_mask & below);
        out[(take && pos < topk) ? pos : kMaxTopk + lane] = b;
        emitted += __popcll(take_mask);
    }
    for (int i = emitted + lane; i < topk; i += 64) out[i] = -1;
}

// ---------------------------------------------------------------------------
// G6: attention over one selected block per workgroup
// ---------------------------------------------------------------------------
namespace {
constexpr int kRowB = kDim * 2;          // 256-byte K/V row of one head
constexpr int kWaveVBytes = 32 * kRowB;  // 32 keys per wave

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte chunk c of V row r sits at chunk position c ^ vswz(r); any 16
// consecutive rows map one chunk to 16 distinct positions.
__device__ __forceinline__ int vswz(int r) { return r & 15; }
}  // namespace

// Two E4M3FN bytes (the low or high 16 bits of w) -> two bf16, packed (exact:
// every E4M3 value is a bf16 value).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// ---------------------------------------------------------------------------
// G6: streaming attention, one workgroup per 8 slots of a row
// ---------------------------------------------------------------------------
namespace {
constexpr int kStreamSlots = 8;  // selected slots per workgroup (at most)
// Per wave: two stages of one block's K rows + V rows (bf16: 2 x 16 KiB;
// E4M3: 2 x 8 KiB of bytes plus an 8 KiB bf16 V buffer for the transposing
// reads).
template <bool kFp8Kv> struct StreamLayout {
    static constexpr int kRowBytes = kFp8Kv ? kDim : 2 * kDim;    // one K or V row
    static constexpr int kHalf = 32 * kRowBytes;                   // 32 rows
    static constexpr int kStage = 2 * kHalf;                       // K rows, V rows
    static constexpr int kVbf = kFp8Kv ? 2 * kStage : 0;           // offset of the bf16 V buffer
    static constexpr int kWave = 2 * kStage + (kFp8Kv ? kWaveVBytes : 0);
    static constexpr int kCopies = kStage / 1024;                  // one-KiB copies per block
};

// HBM -> LDS copy of 16 bytes per lane (lane l writes lds_dst + 16l), from
// asm so that the compiler does not wait for it before unrelated LDS reads;
// completion is awaited with explicit vmcnt.
__device__ __forceinline__ void stream_copy(const void *src, uint8_t *lds_dst) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)lds_dst);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
}  // namespace

// Workgroup (sg, g, r): slots spw*sg .. spw*sg+spw-1 of row (KV head g,
// request r), spw <= 8 slots per workgroup;
// 4 waves, wave w owns keys 32w..32w+31 of every selected block.  Each wave
// streams its K and V rows of the next block into its own 2-stage LDS ring
// while it computes the current one (no workgroup barrier until the end):
//   S^T[32 x 16] = K . Q^T   (K rows read from LDS as the MFMA A operand),
//   an online softmax across the blocks, O^T += V^T . P^T (V^T by
//   transposing LDS reads); the 4 waves' partials are merged at the end
//   into one (O, m, l) partial of the workgroup.
// Both row buffers keep 16-byte chunk c of row rr at position c ^ (rr & 15).
// kFp8Kv: E4M3 caches; K is widened to bf16 as it is read, and each wave's
// V rows are widened once into a bf16 buffer in the layout above (E4M3
// values are exact in bf16; k_scale is folded into scale_log2 and v_scale
// multiplies the partial O).  Byte rows keep 16-byte chunk c of row rr at
// position c ^ (rr & 7).
template <bool kFp8Kv, int kCpl>
__global__ __launch_bounds__(256) void decode_attend_stream_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kc_, const void *__restrict__ vc_,
    const int32_t *__restrict__ pt, int max_pages, const int32_t *__restrict__ ctx, int max_ctx, int B,
    const float *__restrict__ S, int nb_max, int topk, int init, int local, int spw, int nparts, float scale_log2,
    float v_scale, float *__restrict__ part_o, float *__restrict__ part_ml, int32_t *__restrict__ q2k_out) {
    using SL = StreamLayout<kFp8Kv>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // 4 waves x 2 stages x (K, V)
    __shared__ float s_m[4][16], s_l[4][16];
    __shared__ int32_t s_sel[4][kMaxTopk + 128];  // per wave: the row, dump slots, working space
    const int sg = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, qd = lane >> 4;
    const int L = min(ctx[r], max_ctx);
    if (L <= 0) {
        // an empty (padding) request: nothing is read; an empty partial
        // (m = -inf, l = 0, O = 0) makes its output row zero, and its q2k
        // row is all -1
        if (q2k_out && sg == 0 && tid < topk) q2k_out[(size_t(g) * B + r) * topk + tid] = -1;
        float *po = part_o + ((size_t(r) * kKvHeads + g) * nparts + sg) * (kGroup * kDim);
        float *pml = part_ml + ((size_t(r) * kKvHeads + g) * nparts + sg) * (kGroup * 2);
        *(f32x4 *)(po + 8 * tid) = f32x4{};
        *(f32x4 *)(po + 8 * tid + 4) = f32x4{};
        if (tid < kGroup) {
            pml[2 * tid] = -INFINITY;
            pml[2 * tid + 1] = 0.f;
        }
        return;
    }
    const int c = (L - 1) / kBlock;
    const int key0 = 32 * wave;
    uint8_t *ring = smem + wave * SL::kWave;

    // Q^T operand: lane (n = head, qd), step ks: 16-byte chunk 4ks + qd
    // (loaded first, so that its latency overlaps the selection)
    const uint16_t *qrow = q + (size_t(r) * kHeads + g * kGroup + n) * kDim;
    bf16x8 qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qrow + 8 * (4 * ks + qd)));

    // The page-table entries of the row's candidates (block lane + 64i in
    // register i, as the scores are held), loaded before the selection so
    // that their latency overlaps it; an entry past the row is clamped and
    // never used.  Above 8 candidates per lane (where the extra loads cost
    // more than the round trip they save) the chosen blocks' entries are
    // loaded after the selection instead.
    constexpr bool kPtRegs = kCpl <= 8;
    int ptv[kPtRegs ? kCpl : 1];
    if constexpr (kPtRegs) {
#pragma unroll
        for (int i = 0; i < kCpl; ++i) ptv[i] = pt[size_t(r) * max_pages + min(lane + 64 * i, max_pages - 1)];
    }
    // The row's selection from the scores of index head g: every wave computes
    // the same row into its own LDS slots, so no barrier is needed.
    select_row<kCpl>(S + (size_t(r) * kIdxHeads + g) * nb_max, nb_max, c, topk, init, local, lane, s_sel[wave]);
    __builtin_amdgcn_wave_barrier();
    if (q2k_out && sg == 0 && wave == 0 && lane < topk) q2k_out[(size_t(g) * B + r) * topk + lane] = s_sel[0][lane];
    // the workgroup's slots (wave-uniform): block id, or -1 when unselected
    // or absent (a negative page id: nothing of it is read), and the block's
    // physical page
    int bsel[kStreamSlots], bpage[kStreamSlots];
#pragma unroll
    for (int j = 0; j < kStreamSlots; ++j) {
        const int s = sg * spw + j;
        const int b = (j < spw && s < topk) ? __builtin_amdgcn_readfirstlane(s_sel[wave][s]) : -1;
        const int bb = (b >= 0 && b <= c) ? b : -1;
        int page = -1;
        if (bb >= 0) {
            if constexpr (kPtRegs) {
                int x = ptv[0];
#pragma unroll
                for (int i = 1; i < kCpl; ++i) x = (bb >> 6) == i ? ptv[i] : x;
                page = __builtin_amdgcn_readlane(x, bb & 63);
            } else {
                page = __builtin_amdgcn_readfirstlane(pt[size_t(r) * max_pages + bb]);
            }
        }
        bsel[j] = page >= 0 ? bb : -1;
        bpage[j] = page;
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): q is in before any copy is issued
    // copies of slot j into stage st: K rows key0..key0+31 (8 one-KiB copies)
    // then V rows (8); rows past L re-read the last valid row (masked)
    auto issue = [&](int j, int st) {
        const int b = bsel[j];
        const size_t slot0 = size_t(max(bpage[j], 0)) * kBlock;
        const int kmax = L - 1 - b * kBlock;
        uint8_t *kb = ring + st * SL::kStage;
        constexpr int kRowsPerCopy = 1024 / SL::kRowBytes;  // 4 (bf16) or 8 (E4M3)
        constexpr int kChunksPerRow = SL::kRowBytes / 16;
#pragma unroll
        for (int i = 0; i < SL::kCopies / 2; ++i) {
            const int rr = kRowsPerCopy * i + lane / kChunksPerRow;
            const int chunk = (lane % kChunksPerRow) ^ (kFp8Kv ? (rr & 7) : vswz(rr));
            const size_t off = ((slot0 + min(key0 + rr, kmax)) * kKvHeads + g) * SL::kRowBytes + 16 * chunk;
            stream_copy((const uint8_t *)kc_ + off, kb + i * 1024);
            stream_copy((const uint8_t *)vc_ + off, kb + SL::kHalf + i * 1024);
        }
    };


    float m_run = -INFINITY, l_run = 0.f;  // per head column n (log2 domain)
    f32x4 oacc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{};
    const int gi = lane & 15;
    if (bsel[0] >= 0) issue(0, 0);
#pragma unroll
    for (int j = 0; j < kStreamSlots; ++j) {
        const bool next = j + 1 < kStreamSlots && bsel[j + 1] >= 0;
        if (next) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage (j+1)&1 was last read at slot j-1
            issue(j + 1, (j + 1) & 1);
        }
        if (bsel[j] < 0) continue;
        // slot j's copies have landed (the next slot's may still be in flight)
        if (next) {
            if constexpr (kFp8Kv) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const uint8_t *kb = ring + (j & 1) * SL::kStage;
        const uint8_t *vt = kFp8Kv ? ring + SL::kVbf : kb + SL::kHalf;
        const int kmax = L - 1 - bsel[j] * kBlock;
        if constexpr (kFp8Kv) {
            // widen this wave's 32 V rows into the bf16 buffer: lane -> row
            // lane/2, byte chunks 4(lane%2)..+3 (16 E4M3 values each)
            const uint8_t *vr = kb + SL::kHalf;
            uint8_t *vb = ring + SL::kVbf;
            const int rr = lane >> 1;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int c = 4 * (lane & 1) + cc;
                const u32x4 x = *(const u32x4 *)(vr + rr * SL::kRowBytes + ((c ^ (rr & 7)) << 4));
                u32x4 lo, hi;
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    lo[2 * w] = e4m3x2_to_bf16x2<false>(x[w]);
                    lo[2 * w + 1] = e4m3x2_to_bf16x2<true>(x[w]);
                    hi[2 * w] = e4m3x2_to_bf16x2<false>(x[2 + w]);
                    hi[2 * w + 1] = e4m3x2_to_bf16x2<true>(x[2 + w]);
                }
                *(u32x4 *)(vb + rr * kRowB + (((2 * c) ^ vswz(rr)) << 4)) = lo;
                *(u32x4 *)(vb + rr * kRowB + (((2 * c + 1) ^ vswz(rr)) << 4)) = hi;
            }
        }
        // S^T: M-tile mt = keys key0 + 16mt + m (row 16mt + m of the buffer)
        f32x4 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = f32x4{};
            const int rr = 16 * mt + n;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 ka;
                if constexpr (kFp8Kv) {
                    // 8 E4M3 values: the half (4ks + qd) % 2 of byte chunk (4ks + qd) / 2
                    const int e = 4 * ks + qd;
                    const u32x2 x = *(const u32x2 *)(kb + rr * SL::kRowBytes + ((((e >> 1) ^ (rr & 7)) << 4) | ((e & 1) << 3)));
                    ka = __builtin_bit_cast(bf16x8, u32x4{e4m3x2_to_bf16x2<false>(x[0]), e4m3x2_to_bf16x2<true>(x[0]),
                                                          e4m3x2_to_bf16x2<false>(x[1]), e4m3x2_to_bf16x2<true>(x[1])});
                } else {
                    ka = __builtin_bit_cast(bf16x8, *(const u32x4 *)(kb + rr * kRowB + (((4 * ks + qd) ^ vswz(rr)) << 4)));
                }
                sacc[mt] = mfma_16x16x32(ka, qb[ks], sacc[mt]);
            }
        }
        // online softmax over this block's keys 16mt + 4qd + i for head n
        float mloc = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = key0 + 16 * mt + 4 * qd + i <= kmax;
                const float z = ok ? sacc[mt][i] * scale_log2 : -INFINITY;
                sacc[mt][i] = z;
                mloc = fmaxf(mloc, z);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float base = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - base);  // 0 while m_run is -inf
        float psum = 0.f;
        bf16x8 pb;  // P^T operand: keys 4qd + e (tile 0) then 16 + 4qd + e (tile 1)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = __builtin_amdgcn_exp2f(sacc[mt][i] - base);
                psum += pv;
                pb[4 * mt + i] = (__bf16)pv;
            }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // O^T = alpha O^T + V^T . P^T (transposing reads as in the one-block kernel)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            i16x4 t[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int rr = 16 * h + 4 * qd + (gi >> 2);
                const int col = 16 * dt + 4 * (gi & 3);
                const int pos = ((col >> 3) ^ vswz(rr)) << 4;
                t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(vt + rr * kRowB + pos + ((col & 7) << 1)));
            }
            const i16x8 ab = {t[0][0], t[0][1], t[0][2], t[0][3], t[1][0], t[1][1], t[1][2], t[1][3]};
            oacc[dt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, ab), pb, oacc[dt] * alpha);
        }
    }
    // wave partial O^T -> LDS (the start of the wave's own ring, no longer read)
    float *so = (float *)ring;  // [16 heads][128 d] (8 KiB)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) so[n * kDim + 16 * dt + 4 * qd + i] = oacc[dt][i];
    if (qd == 0) {
        s_m[wave][n] = m_run;
        s_l[wave][n] = l_run;
    }
    __syncthreads();
    // merge the 4 waves: thread -> (head hh, 8 d)
    const int hh = tid >> 4, d0 = (tid & 15) * 8;
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) { mw[w] = s_m[w][hh]; M = fmaxf(M, mw[w]); }
    const float baseM = M == -INFINITY ? 0.f : M;
    float sc[4], l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        sc[w] = __builtin_amdgcn_exp2f(mw[w] - baseM);
        l += sc[w] * s_l[w][hh];
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float *src = (const float *)(smem + w * SL::kWave) + hh * kDim + d0;
        const f32x4 a = *(const f32x4 *)src, c4 = *(const f32x4 *)(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[e] += sc[w] * a[e];
            o[4 + e] += sc[w] * c4[e];
        }
    }
    if constexpr (kFp8Kv) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= v_scale;
    }
    // this workgroup's (O, m, l) partial; the combine kernel merges the row's partials
    float *po = part_o + (size_t(r) * kKvHeads + g) * nparts * (kGroup * kDim);
    float *pml = part_ml + (size_t(r) * kKvHeads + g) * nparts * (kGroup * 2);
    *(f32x4 *)(po + sg * (kGroup * kDim) + hh * kDim + d0) = f32x4{o[0], o[1], o[2], o[3]};
    *(f32x4 *)(po + sg * (kGroup * kDim) + hh * kDim + d0 + 4) = f32x4{o[4], o[5], o[6], o[7]};
    if ((tid & 15) == 0) {
        pml[sg * (kGroup * 2) + 2 * hh] = M;
        pml[sg * (kGroup * 2) + 2 * hh + 1] = l;
    }
}

// ---------------------------------------------------------------------------
// G7: merge the topk partials of each (request, KV head) in fixed block order
// ---------------------------------------------------------------------------
// One 64-thread workgroup per (d quarter, KV head, request): thread ->
// (head tid/4, 8 of the quarter's 32 d).
// The thread's 8 d of one head, with the 3 neighbouring lanes (tid/4 equal),
// are exactly one 32-value MXFP8 block of the output row [64 * 128]: block
// (head, d quarter).
// kP: the partial count rounded up to a power of two; partials t >= topk
// re-read the last one and weigh nothing, so every load is unconditional and
// all of them are in flight together.
template <bool kMx, int kP>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float *__restrict__ part_o,
                                                            const float *__restrict__ part_ml,
                                                            int topk, uint16_t *__restrict__ out,
                                                            uint8_t *__restrict__ out_q,
                                                            uint8_t *__restrict__ out_scale) {
    const int dq = blockIdx.x, g = blockIdx.y, r = blockIdx.z, tid = threadIdx.x;
    const size_t base = (size_t(r) * kKvHeads + g) * topk;
    const int hh = tid >> 2, d0 = 32 * dq + (tid & 3) * 8;  // head, 8 d
    float mt[kP], lt[kP];
    f32x4 oa[kP], ob[kP];
#pragma unroll
    for (int t = 0; t < kP; ++t) {
        const int tt = min(t, topk - 1);
        const float *ml = part_ml + (base + tt) * (kGroup * 2) + 2 * hh;
        const float *src = part_o + (base + tt) * (kGroup * kDim) + hh * kDim + d0;
        const float m = ml[0], l = ml[1];
        mt[t] = t < topk ? m : -INFINITY;
        lt[t] = t < topk ? l : 0.f;
        oa[t] = *(const f32x4 *)src;
        ob[t] = *(const f32x4 *)(src + 4);
    }
    float M = -INFINITY;
#pragma unroll
    for (int t = 0; t < kP; ++t) M = fmaxf(M, mt[t]);
    const float baseM = M == -INFINITY ? 0.f : M;
    f32x4 na = {}, nb = {};
    float den = 0.f;
#pragma unroll
    for (int t = 0; t < kP; ++t) {
        const float w = mt[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mt[t] - baseM);
        den += w * lt[t];
        na += w * oa[t];
        nb += w * ob[t];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    bf16x8 o8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o8[e] = (__bf16)(na[e] * inv);
        o8[4 + e] = (__bf16)(nb[e] * inv);
    }
    const size_t row = size_t(r) * kHeads + g * kGroup + hh;  // (request, query head)
    if constexpr (kMx) {
        const u32x4 w = __builtin_bit_cast(u32x4, o8);  // element 2j in the low half of word j
        uint16_t bits[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bits[2 * j] = uint16_t(w[j] & 0xFFFFu);
            bits[2 * j + 1] = uint16_t(w[j] >> 16);
        }
        uint32_t sc;
        const uint64_t codes = mxfp8_encode8(bits, sc);
        *(uint64_t *)(out_q + row * kDim + d0) = codes;
        if ((tid & 3) == 0) out_scale[row * (kDim / 32) + dq] = uint8_t(sc);
    } else {
        *(bf16x8 *)(out + row * kDim + d0) = o8;
    }
}

// partials per (request, KV head): one per attention workgroup (8 slots)
// Selected slots per attention workgroup: 8, or fewer when the batch is too
// small for (requests x KV heads x ceil(topk/8)) workgroups to cover the 256
// CUs (at batch 8, topk 16: 2 slots, 256 workgroups instead of 64).
int decode_slots_per_wg(int topk, int B) {
    int spw = kStreamSlots;
    while (spw > 1 && B * kKvHeads * ceil_div(topk, spw) < 256) spw >>= 1;
    return spw;
}

int decode_parts(int topk, int B) { return ceil_div(topk, decode_slots_per_wg(topk, B)); }

hipError_t launch_decode_attend(const uint16_t *q, const void *kc, const void *vc, bool fp8kv, float k_scale,
                                float v_scale, const int32_t *pt, int max_pages, const int32_t *ctx,
                                int max_ctx, int B, const float *S, int nb_max, int topk, int init, int local,
                                float scale, float *partial, int32_t *q2k_out, hipStream_t stream) {
    const int spw = decode_slots_per_wg(topk, B);
    const int nparts = ceil_div(topk, spw);
    float *part_o = partial;
    float *part_ml = partial + size_t(B) * kKvHeads * nparts * kGroup * kDim;
    const dim3 grid(nparts, kKvHeads, B);
    const int cpl = ceil_div(nb_max, 64);
#define MSA_ATTEND_CASE(N)                                                                                   \
    if (cpl <= N) {                                                                                          \
        if (fp8kv)                                                                                           \
            hipLaunchKernelGGL((decode_attend_stream_kernel<true, N>), grid, dim3(256),                      \
                               size_t(4) * StreamLayout<true>::kWave, stream, q, kc, vc, pt, max_pages, ctx, \
                               max_ctx, B, S, nb_max, topk, init, local, spw, nparts, scale * kLog2e * k_scale, \
                               v_scale, part_o, part_ml, q2k_out);                                          \
        else                                                                                                 \
            hipLaunchKernelGGL((decode_attend_stream_kernel<false, N>), grid, dim3(256),                     \
                               size_t(4) * StreamLayout<false>::kWave, stream, q, kc, vc, pt, max_pages, ctx, \
                               max_ctx, B, S, nb_max, topk, init, local, spw, nparts, scale * kLog2e, 1.0f,  \
                               part_o, part_ml, q2k_out);                                                   \
        return hipGetLastError();                                                                            \
    }
    MSA_ATTEND_CASE(1)
    MSA_ATTEND_CASE(2)
    MSA_ATTEND_CASE(4)
    MSA_ATTEND_CASE(8)
    MSA_ATTEND_CASE(16)
    MSA_ATTEND_CASE(32)
    MSA_ATTEND_CASE(64)
    MSA_ATTEND_CASE(128)
#undef MSA_ATTEND_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const float *partial, int B, int topk, bool fp8kv, uint16_t *out,
                                 uint8_t *out_q, uint8_t *out_scale, hipStream_t stream) {
    topk = decode_parts(topk, B);  // partials per (request, KV head)
    const float *part_o = partial;
    const float *part_ml = partial + size_t(B) * kKvHeads * topk * kGroup * kDim;
#define MSA_COMBINE_CASE(P)                                                                          \
    if (topk <= P) {                                                                                 \
        if (out_q)                                                                                   \
            hipLaunchKernelGGL((decode_combine_kernel<true, P>), dim3(4, kKvHeads, B), dim3(64), 0, stream, \
                               part_o, part_ml, topk, out, out_q, out_scale);                        \
        else                                                                                         \
            hipLaunchKernelGGL((decode_combine_kernel<false, P>), dim3(4, kKvHeads, B), dim3(64), 0, stream, \
                               part_o, part_ml, topk, out, out_q, out_scale);                        \
        return hipGetLastError();                                                                    \
    }
    MSA_COMBINE_CASE(1)
    MSA_COMBINE_CASE(2)
    MSA_COMBINE_CASE(4)
    MSA_COMBINE_CASE(8)
    MSA_COMBINE_CASE(16)
#undef MSA_COMBINE_CASE
    return hipErrorInvalidValue;
}

}  // namespace msa
