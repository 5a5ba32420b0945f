// Index-branch block selection for packed-document prefill.
//
// Method (TensorRT-LLM "MiniMaxM3SparseAttentionConfig", class description
// and the sparse_* fields; NeMo AutoModel minimax_m3_vl.msa,
// MSAMicrobatch.select_blocks): every 128-key block of the query's own
// document is scored by the largest raw dot product between the query's
// index vector (per index head) and the single shared index key, over the
// block's keys at or before the query; blocks 0..init-1 and the last
// `local` blocks up to the query's own block are forced; the remaining
// top-k slots take the best-scoring other blocks; ids are document-local,
// ascending, padded with -1.
//
// Kernels:
//   doc_setup_kernel    - sanitised document spans + tile prefix counts
//                         (for the scorer also the prefix counts of its
//                         (tile, key block) work items).
//   block_scores_kernel - S^T = K . IQ^T on MFMA (bf16 32x32x16 or E4M3
//                         32x32x64 with unit scales), fused causal mask and
//                         per-block row max for (tile, key block) items; a
//                         tile is 64 query tokens x 4 index heads of one
//                         document and its items are blocks 0..c.  Two
//                         workgroups per CU, each taking an equal contiguous
//                         range of all items; each key block is copied from
//                         global memory into LDS (swizzled, double-buffered)
//                         while the item before it is computed.
//   topk_prefill_kernel - one lane per (head, token) row: top-R insertion
//                         over 32-bit order keys of the scores, then an
//                         ascending emit pass that takes every candidate
//                         above the R-th key and the first (lowest-id)
//                         candidates equal to it, up to the quota.
#include "attend_common.hpp"

namespace msa {

// ---------------------------------------------------------------------------
// G0: document spans and tile offsets
// ---------------------------------------------------------------------------
// Tiles of a document of len tokens when every 128-token query block is cut
// into ceil(128/tile) tiles of near-equal size (a partial last block into
// ceil(rest/tile)); equal to ceil(len/tile) whenever tile divides 128.
__device__ __forceinline__ int tiles_in_doc(int len, int tile) {
    const int per_block = (kBlock + tile - 1) / tile;
    const int rest = len % kBlock;
    return (len / kBlock) * per_block + (rest + tile - 1) / tile;
}

// Block-scorer work of a document of len tokens: its kScoreTile-token tiles,
// tile j in query block j/2, each scored against blocks 0..j/2.  With m = nt/2,
// tiles 0..2m-1 hold 2(1 + 2 + ... + m) = m(m+1) (tile, block) pairs, and an
// odd last tile m + 1 more.
__device__ __forceinline__ int score_work_in_doc(int len) {
    const int nt = tiles_in_doc(len, kScoreTile);
    const int m = nt >> 1;
    return m * (m + 1) + ((nt & 1) ? m + 1 : 0);
}

__global__ __launch_bounds__(1024) void doc_setup_kernel(const int32_t *__restrict__ cu, int ndocs,
                                                         int T, int max_seqlen, int tile_a,
                                                         int tile_b, DocSpan *__restrict__ docs,
                                                         int32_t *__restrict__ off_a,
                                                         int32_t *__restrict__ off_b) {
    __shared__ int wsum_a[16], wsum_b[16];
    __shared__ int carry_a, carry_b;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry_a = 0;
        carry_b = 0;
        off_a[0] = 0;
        if (off_b) off_b[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < ndocs; base += 1024) {
        const int d = base + tid;
        int na = 0, nb = 0;
        if (d < ndocs) {
            int s = min(max(cu[d], 0), T);
            int e = min(max(cu[d + 1], s), T);
            int len = min(e - s, max_seqlen);
            docs[d] = DocSpan{s, len};
            na = tiles_in_doc(len, tile_a);
            // tile_b < 0: the block scorer's (tile, block) pairs instead of tiles
            nb = tile_b > 0 ? tiles_in_doc(len, tile_b) : tile_b < 0 ? score_work_in_doc(len) : 0;
        }
        // inclusive wave scans
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int ya = __shfl_up(na, o), yb = __shfl_up(nb, o);
            if (lane >= o) { na += ya; nb += yb; }
        }
        if (lane == 63) { wsum_a[wave] = na; wsum_b[wave] = nb; }
        __syncthreads();
        int pa = carry_a, pb = carry_b;
        for (int w = 0; w < wave; ++w) { pa += wsum_a[w]; pb += wsum_b[w]; }
        if (d < ndocs) {
            off_a[d + 1] = pa + na;
            if (off_b) off_b[d + 1] = pb + nb;
        }
        __syncthreads();
        if (tid == 1023) { carry_a = pa + na; carry_b = pb + nb; }
        __syncthreads();
    }
}

hipError_t launch_doc_setup(const int32_t *cu, int ndocs, int T, int max_seqlen, int tile_a,
                            int tile_b, DocSpan *docs, int32_t *off_a, int32_t *off_b,
                            hipStream_t stream) {
    hipLaunchKernelGGL(doc_setup_kernel, dim3(1), dim3(1024), 0, stream, cu, ndocs, T, max_seqlen,
                       tile_a, tile_b, docs, off_a, off_b);
    return hipGetLastError();
}

// Tile t of a prefix-count array off[0..ndocs]: the document d with
// off[d] <= t < off[d+1] (uniform across the workgroup).
__device__ __forceinline__ int tile_doc(const int32_t *off, int ndocs, int t) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// G1: block scores
// ---------------------------------------------------------------------------
template <bool kFp8>
struct ScoreLayout {
    static constexpr int kRowBytes = kFp8 ? 128 : 256;           // one index row
    static constexpr int kChunks = kRowBytes / 16;               // 16-byte chunks per row
    static constexpr int kRowsPerCopy = 1024 / kRowBytes;        // rows per one-KiB copy
    static constexpr int kCopiesPerWave = kBlock * kRowBytes / 1024 / 4;
    static constexpr int kBufBytes = kBlock * kRowBytes;
};

// LDS position of 16-byte chunk c of key row r: c ^ sswz(r).  The 16 rows a
// quarter-wave reads at one chunk then land on 16 distinct bank groups (bf16:
// 256-byte rows; E4M3: 128-byte rows, two rows per bank cycle).
template <bool kFp8>
__device__ __forceinline__ int sswz(int r) {
    return kFp8 ? ((r >> 1) & 7) : (r & 15);
}

static_assert(kScoreTile * 2 == kBlock, "two scorer tiles per query block");

// Tile j and block b of a document's local work index x (tiles in order,
// each over its blocks 0..j/2): tiles 2m and 2m+1 start at m(m+1) and
// m(m+1) + m + 1.
__device__ __forceinline__ void score_work_at(int x, int &j, int &b) {
    int m = int((__builtin_sqrtf(4.f * float(x) + 1.f) - 1.f) * 0.5f);
    while (m > 0 && m * (m + 1) > x) --m;
    while ((m + 1) * (m + 2) <= x) ++m;
    const int rem = x - m * (m + 1);
    const bool second = rem >= m + 1;
    j = 2 * m + (second ? 1 : 0);
    b = second ? rem - (m + 1) : rem;
}

template <bool kFp8>
__global__ __launch_bounds__(256, 2) void block_scores_kernel(
    const uint8_t *__restrict__ iq, const uint8_t *__restrict__ ik, const DocSpan *__restrict__ docs,
    const int32_t *__restrict__ tile_off, const int32_t *__restrict__ work_off, int ndocs, int T, int nb_max,
    float *__restrict__ S) {
    using L = ScoreLayout<kFp8>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // two key blocks

    // The work is the list of (tile, key block) pairs: documents in order, a
    // document's tiles in order, a tile's blocks 0..c.  Workgroup w takes the
    // w-th of gridDim.x equal contiguous ranges, so that the two workgroups of
    // every CU run (two waves per SIMD) until the end.
    const int total = work_off[ndocs];
    const int bid = blockIdx.x, nwg = gridDim.x;
    const int g0 = int((int64_t(total) * bid) / nwg);
    const int g1 = int((int64_t(total) * (bid + 1)) / nwg);
    if (g0 >= g1) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hb = lane >> 5;

    // position of a work item: document d, its tile j (query block c = j/2),
    // key block b
    struct Pos {
        int d, j, b;
    };
    auto locate = [&](int g) {
        Pos p;
        p.d = tile_doc(work_off, ndocs, g);
        score_work_at(g - work_off[p.d], p.j, p.b);
        return p;
    };
    // the item after p (items within [g0, g1) only: a document with work left)
    auto next = [&](Pos p) {
        if (p.b < p.j / 2) {
            ++p.b;
        } else if (p.j + 1 < tile_off[p.d + 1] - tile_off[p.d]) {
            ++p.j;
            p.b = 0;
        } else {
            do { ++p.d; } while (work_off[p.d + 1] == work_off[p.d]);
            p.j = 0;
            p.b = 0;
        }
        return p;
    };

    // Key block b of tile p -> LDS buffer buf: wave w issues copies
    // kCopiesPerWave*w .. (one KiB each, kRowsPerCopy rows); lane l of a copy
    // fills row l / kChunks at position l % kChunks, i.e. chunk
    // (l % kChunks) ^ sswz.  Rows at or past the tile's key end occur only in
    // its own query block, where the causal mask drops them: they re-read the
    // row before that end, in the document.
    auto issue_block = [&](const Pos &p, int buf) {
        const DocSpan doc = docs[p.d];
        // rows past the tile's last key (only in its diagonal block) repeat that key
        const int last = min(doc.len, (p.j + 1) * kScoreTile) - 1 - p.b * kBlock;
        const uint8_t *base = ik + size_t(doc.start + p.b * kBlock) * L::kRowBytes;
#pragma unroll
        for (int i = 0; i < L::kCopiesPerWave; ++i) {
            const int cp = L::kCopiesPerWave * wave + i;
            const int r = L::kRowsPerCopy * cp + lane / L::kChunks;
            const int chunk = (lane % L::kChunks) ^ sswz<kFp8>(r);
            copy_to_lds_s(base, uint32_t(min(r, last) * L::kRowBytes + 16 * chunk),
                          smem + buf * L::kBufBytes + cp * 1024);
        }
    };

    // Index-query operand (B) of the current tile, in registers.  Column n of
    // N-tile nt is row (token p0+16*wave+8*nt+n/4, head n%4).
    constexpr int kSteps = kFp8 ? 2 : 8;
    typedef typename std::conditional<kFp8, i32x8, bf16x8>::type Frag;
    Frag qb[2][kSteps];
    auto load_q = [&](const DocSpan &doc, int p0) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int p = p0 + 16 * wave + 8 * nt + n / 4;
            const bool ok = p < doc.len;
            const size_t row = size_t(doc.start + (ok ? p : 0)) * kIdxHeads + (n & 3);
            const uint8_t *src = iq + row * L::kRowBytes;
#pragma unroll
            for (int ks = 0; ks < kSteps; ++ks) {
                if constexpr (kFp8) {
                    u32x4 lo = ok ? *(const u32x4 *)(src + 64 * ks + 32 * hb) : u32x4{0, 0, 0, 0};
                    u32x4 hi = ok ? *(const u32x4 *)(src + 64 * ks + 32 * hb + 16) : u32x4{0, 0, 0, 0};
                    qb[nt][ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                } else {
                    u32x4 v = ok ? *(const u32x4 *)(src + 2 * (16 * ks + 8 * hb)) : u32x4{0, 0, 0, 0};
                    qb[nt][ks] = __builtin_bit_cast(bf16x8, v);
                }
            }
        }
    };

    // A fragment of M-tile mt, k-step ks: row 32mt + n, this lane's 16 (bf16)
    // or 32 (E4M3) bytes of the step
    auto load_frag = [&](const uint8_t *kb, int mt, int ks) {
        const int r = 32 * mt + n;
        const uint8_t *row = kb + r * L::kRowBytes;
        if constexpr (kFp8) {
            const int c0 = 4 * ks + 2 * hb;
            const u32x4 lo = *(const u32x4 *)(row + ((c0 ^ sswz<kFp8>(r)) << 4));
            const u32x4 hi = *(const u32x4 *)(row + (((c0 + 1) ^ sswz<kFp8>(r)) << 4));
            return Frag{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else {
            return __builtin_bit_cast(bf16x8, *(const u32x4 *)(row + (((2 * ks + hb) ^ sswz<kFp8>(r)) << 4)));
        }
    };

    Pos cur = locate(g0);
    issue_block(cur, 0);
    int tile_d = -1, tile_j = -1;  // the tile whose query operand is in qb
    DocSpan doc{0, 0};
    int p0 = 0, c = 0;

    // Item loop: at the barrier of item g its copies have landed (each wave
    // waited for its own) and every wave is done with item g-1, whose buffer
    // then receives item g+1 while item g is computed.
    for (int g = g0; g < g1; ++g) {
        if (cur.d != tile_d || cur.j != tile_j) {  // a new tile (workgroup-uniform)
            tile_d = cur.d;
            tile_j = cur.j;
            doc = docs[cur.d];
            p0 = cur.j * kScoreTile;
            c = cur.j / 2;
            load_q(doc, p0);
        }
        const int b = cur.b;
        const Pos nxt = g + 1 < g1 ? next(cur) : cur;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's copies of item g (and its loads, stores)
        barrier_keep_prefetch();
        if (g + 1 < g1) issue_block(nxt, (g + 1 - g0) & 1);
        const uint8_t *kb = smem + ((g - g0) & 1) * L::kBufBytes;

        // K-step by k-step over the 4 M-tiles (32 keys each): the fragment of
        // step s + kD is read from LDS before step s's MFMAs are issued, and
        // M-tile mt-1's max (its accumulators are complete by then) is taken
        // in chunks after the first steps of mt; scheduling fences keep that
        // order.  Lane (n, hb) of an N-tile accumulator holds keys
        // 32mt + 8(r/4) + 4hb + r%4 of column n.  The query's own block
        // (b == c) drops the keys past each column's token.
        float mxv[2] = {-INFINITY, -INFINITY};
        auto item = [&](auto diag_tag) {
            constexpr bool kDiag = decltype(diag_tag)::value;
            constexpr int kD = 3;                      // fragment read distance (steps)
            constexpr int kSt = 4 * kSteps;            // steps per item
            constexpr int kChunk = kSteps >= 4 ? 4 : kSteps;  // steps carrying a part of the max
            constexpr int kRows = 16 / kChunk;         // accumulator rows per part
            Frag fr[kD + 1];
            f32x16 acc[2][2];
            // rows [kRows*part, kRows*(part+1)) of M-tile mt's accumulators into the max
            auto max_part = [&](int mt, int part, const f32x16 (&a)[2]) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int p = p0 + 16 * wave + 8 * nt + n / 4;
#pragma unroll
                    for (int rr = 0; rr < kRows; ++rr) {
                        const int r = kRows * part + rr;
                        if constexpr (kDiag) {
                            const int kp = b * kBlock + 32 * mt + 8 * (r >> 2) + 4 * hb + (r & 3);
                            mxv[nt] = fmaxf(mxv[nt], kp > p ? -INFINITY : a[nt][r]);
                        } else {
                            mxv[nt] = fmaxf(mxv[nt], a[nt][r]);
                        }
                    }
                }
            };
#pragma unroll
            for (int st = 0; st < kD; ++st) fr[st] = load_frag(kb, st / kSteps, st % kSteps);
#pragma unroll
            for (int st = 0; st < kSt; ++st) {
                const int mt = st / kSteps, ks = st % kSteps;
                if (st + kD < kSt) fr[(st + kD) % (kD + 1)] = load_frag(kb, (st + kD) / kSteps, (st + kD) % kSteps);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const f32x16 cin = ks == 0 ? f32x16{} : acc[mt & 1][nt];
                    if constexpr (kFp8)
                        acc[mt & 1][nt] = mfma_32x32x64_e4m3(fr[st % (kD + 1)], qb[nt][ks], cin);
                    else
                        acc[mt & 1][nt] = mfma_32x32x16(fr[st % (kD + 1)], qb[nt][ks], cin);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (mt > 0 && ks < kChunk) max_part(mt - 1, ks, acc[(mt - 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int part = 0; part < kChunk; ++part) max_part(3, part, acc[1]);
        };
        if (b == c)
            item(std::true_type{});
        else
            item(std::false_type{});
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int p = p0 + 16 * wave + 8 * nt + n / 4;
            const float mx = fmaxf(mxv[nt], __shfl_xor(mxv[nt], 32));
            if (hb == 0 && p < doc.len)
                S[(size_t(n & 3) * nb_max + b) * T + doc.start + p] = mx;
        }
        cur = nxt;
    }
}

hipError_t launch_block_scores(const void *iq, const void *ik, bool fp8, const DocSpan *docs,
                               const int32_t *tile_off, const int32_t *work_off, int ndocs, int T,
                               int max_seqlen, float *S, hipStream_t stream) {
    const int nb_max = ceil_div(max_seqlen, kBlock);
    // two workgroups per CU, all resident at once, each with an equal share
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        ncu = 256;
    const int grid = 2 * ncu;
    if (fp8) {
        const size_t lds = 2 * ScoreLayout<true>::kBufBytes;  // two key blocks
        hipLaunchKernelGGL(block_scores_kernel<true>, dim3(grid), dim3(256), lds, stream,
                           (const uint8_t *)iq, (const uint8_t *)ik, docs, tile_off, work_off, ndocs, T,
                           nb_max, S);
    } else {
        const size_t lds = 2 * ScoreLayout<false>::kBufBytes;
        hipLaunchKernelGGL(block_scores_kernel<false>, dim3(grid), dim3(256), lds, stream,
                           (const uint8_t *)iq, (const uint8_t *)ik, docs, tile_off, work_off, ndocs, T,
                           nb_max, S);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// G2: forced blocks + top-k
// ---------------------------------------------------------------------------
// Insert `key` into the descending multiset top[0..15] (the smallest falls
// off): a min/max exchange per slot, two ALU ops each.
__device__ __forceinline__ void topk_insert(uint32_t (&top)[kMaxTopk], uint32_t key) {
#pragma unroll
    for (int i = 0; i < kMaxTopk; ++i) {
        const uint32_t hi = max(top[i], key);
        key = min(top[i], key);
        top[i] = hi;
    }
}

__device__ __forceinline__ uint32_t topk_at(const uint32_t (&top)[kMaxTopk], int i) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) v = (j == i) ? top[j] : v;
    return v;
}

// The R largest (score, lower block id first) keys are: every candidate whose
// score key exceeds the R-th largest score key `thr`, plus the first
// R - #(> thr) candidates in ascending block order whose key equals `thr`.
// So the scan keeps only the 32-bit score keys (ties need no id), and the
// emit pass hands out the tie quota in block order.  Empty slots hold 0; if a
// row has fewer than R candidates, thr = 0 and the quota covers every
// candidate whose key is 0, so all candidates are taken.
__global__ __launch_bounds__(256) void topk_prefill_kernel(const float *__restrict__ S,
                                                           const DocSpan *__restrict__ docs,
                                                           int ndocs, int T, int nb_max, int topk,
                                                           int init, int local,
                                                           int32_t *__restrict__ q2k) {
    // A row's work grows with its query block.  Workgroups x of heads h and
    // h + 2 are dispatched 2 * gridDim.x apart and tend to share a CU, so
    // heads 2 and 3 take the tiles in reverse order: a CU then pairs a late
    // (heavy) tile with an early (light) one.
    const int h = blockIdx.y;
    const int tile = h >= 2 ? int(gridDim.x) - 1 - int(blockIdx.x) : int(blockIdx.x);
    const int t = tile * 256 + threadIdx.x;
    if (t >= T) return;
    int32_t *out = q2k + (size_t(h) * T + t) * topk;
    const int d = find_doc(docs, ndocs, t);
    if (d < 0) {
        for (int i = 0; i < topk; ++i) out[i] = -1;
        return;
    }
    const int c = (t - docs[d].start) / kBlock;
    const int R = topk - forced_count(c, init, local);
    const float *row = S + size_t(h) * nb_max * T + t;  // row[b*T]

    uint32_t top[kMaxTopk];
#pragma unroll
    for (int i = 0; i < kMaxTopk; ++i) top[i] = 0;
    // candidates are read 32 at a time, all loads issued before they are
    // used (one load per candidate in a dependent loop waits a full memory
    // latency each), and the next 32 are loaded while the current ones are
    // processed; the loads are unconditional, with the block index clamped
    // into the scores' nb_max rows (entries past c are never used)
    constexpr int kChunk = 32;
    auto load_chunk = [&](float (&dst)[kChunk], int b0) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) dst[j] = row[size_t(min(b0 + j, nb_max - 1)) * T];
    };
    float sa[kChunk], sb[kChunk];
    if (R > 0) {
        auto scan = [&](const float (&sv)[kChunk], int b0) {
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const int b = b0 + j;
                if (b <= c && !is_forced(b, c, init, local)) topk_insert(top, float_order_bits(sv[j]));
            }
        };
        load_chunk(sa, 0);
        for (int b0 = 0; b0 <= c; b0 += 2 * kChunk) {
            load_chunk(sb, b0 + kChunk);
            scan(sa, b0);
            if (b0 + kChunk > c) break;
            load_chunk(sa, b0 + 2 * kChunk);
            scan(sb, b0 + kChunk);
        }
    }
    // R <= 0: the forced blocks fill the row and no candidate is taken
    const uint32_t thr = R > 0 ? topk_at(top, R - 1) : ~0u;
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < kMaxTopk; ++i) n_gt += (i < R && top[i] > thr) ? 1 : 0;
    int quota = R > 0 ? R - n_gt : 0;
    int k = 0;
    auto emit = [&](const float (&sv)[kChunk], int b0) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int b = b0 + j;
            bool take = false;
            if (b <= c) {
                if (is_forced(b, c, init, local)) {
                    take = true;
                } else if (R > 0) {
                    const uint32_t key = float_order_bits(sv[j]);
                    const bool tie = key == thr && quota > 0;
                    quota -= tie ? 1 : 0;
                    take = key > thr || tie;
                }
            }
            if (take && k < topk) out[k++] = b;
        }
    };
    load_chunk(sa, 0);
    for (int b0 = 0; b0 <= c && k < topk; b0 += 2 * kChunk) {
        load_chunk(sb, b0 + kChunk);
        emit(sa, b0);
        if (b0 + kChunk > c || k >= topk) break;
        load_chunk(sa, b0 + 2 * kChunk);
        emit(sb, b0 + kChunk);
    }
    for (; k < topk; ++k) out[k] = -1;
}

hipError_t launch_topk_prefill(const float *S, const DocSpan *docs, int ndocs, int T, int nb_max,
                               int topk, int init, int local, int32_t *q2k, hipStream_t stream) {
    hipLaunchKernelGGL(topk_prefill_kernel, dim3(ceil_div(T, 256), kIdxHeads), dim3(256), 0, stream,
                       S, docs, ndocs, T, nb_max, topk, init, local, q2k);
    return hipGetLastError();
}

}  // namespace msa
