// Backward of the sparse GQA prefill attention for a fixed selection.
//
// Method (NeMo AutoModel minimax_m3_vl.msa, _SparseAttention.backward: bf16
// grad_out [tokens,64,128] -> dq [tokens,64,128], dk and dv [tokens,4,128];
// the selection is a hard top-k and carries no gradient).  With P the
// forward's softmax rows, rebuilt from the saved log-sum-exp, dP = dO.v,
// D = rowsum(dO * O) and dS = P (dP - D), over each row's selected keys:
//   dq = scale dS K,   dk = scale dS^T Q,   dv = P^T dO.
//
// Kernels:
//   bwd_hist_kernel, bwd_colscan_kernel, bwd_scan_kernel, bwd_fill_kernel
//       - inverse of q2k: for every (KV head g, document block) the tokens
//       whose row selects the block, ascending, in O(T * topk): per-tile
//       counts, a scan over the tiles and of the list lengths (and chunk
//       counts), then a fill that ranks a tile's tokens by LDS lane masks;
//       no atomics on global memory, so the lists, and every sum taken over
//       them, are the same on every run.
//   bwd_dq_kernel       - query-major: a workgroup takes 16 tokens of one
//       query block (8 waves x 2 tokens) and streams the union of their
//       selected blocks as 32-key units (K rows, V rows) through a 9-slot
//       LDS ring as the forward does: no workgroup barrier, every unit has an
//       LDS state word (claimed bit, count of the waves that still need it)
//       and every slot a ready flag (the id of the unit whose copies last
//       landed there, copied after the unit's 16 copies); each wave walks
//       only the units its tokens need and claims its next one ahead.  Per
//       unit S^T = K Q^T, dP^T = V dO^T, P^T and dS^T in registers, then
//       dQ^T += K^T dS^T with K^T taken by transposing LDS reads.  Its
//       prologue also computes D = rowsum(dO * O) in fp32 for its rows and
//       stores it for dK/dV, which runs after it.
//   bwd_dkdv_kernel     - key-major: one workgroup per chunk of kBwdChunk
//       tokens of one block's list; 8 waves x 16 keys (two waves per SIMD)
//       hold their K and V rows as MFMA operands; per step of 4 tokens (64
//       query rows of the KV
//       group, with their lse and D, staged in a 4-step LDS ring) S = Q K^T,
//       dP = dO V^T, dS, then
//       dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T taken by
//       transposing LDS reads; one fp32 partial (dK, dV) per chunk, or the
//       final bf16 dk, dv when the block's list is a single chunk.
//   bwd_reduce_kernel   - per block with several chunks, the partials summed
//       in chunk order into bf16 dk, dv (a single-chunk block is written by
//       its chunk; keys that no query attends to get zeros).
#include "attend_common.hpp"

namespace msa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowB = kDim * 2;  // bytes of one bf16 row of 128

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read of a 4 x 16 bf16 block: lane j of each 16-lane group
// receives column j of the 4 rows its group addressed (lane i of the group
// supplies row i/4, columns 4(i%4)..+3).
__device__ __forceinline__ i16x4 read_tr(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
}

// Two transposing reads (rows e of the first, then of the second) as one
// 8-element bf16 MFMA operand.
__device__ __forceinline__ bf16x8 join_tr(const i16x4 &a, const i16x4 &b) {
    const i16x8 x = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, x);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
}  // namespace

// ---------------------------------------------------------------------------
// Inverse of q2k: per (KV head, document block) the selecting tokens
// ---------------------------------------------------------------------------
// List li = g * nb_max + Bg holds, ascending, the tokens whose row for KV
// head g selects document block Bg (the blocks of all documents numbered by
// blk_off): the entries b of the row with 0 <= b <= the token's own block,
// each once, as the attention takes them.  Built in O(T * topk): per tile of
// 256 tokens a count of each list's tokens (bwd_hist_kernel), a scan over
// the tiles (bwd_colscan_kernel: each list's tokens in earlier tiles), the
// lists' offsets (bwd_scan_kernel), and a fill (bwd_fill_kernel) in which a
// token's rank within its tile comes from 64-bit LDS masks of the lanes
// that select each block, one mask per wave.  No step depends on timing, so
// the lists, and every sum taken over them, are the same on every run.
constexpr int kListTile = 256;  // tokens per tile, one per thread
constexpr int kListWin = 1024;  // blocks per LDS window

// Token t's counted entries for KV head g as global block numbers
// (blk_off[d] + b), -1 in the other slots.
__device__ __forceinline__ void row_blocks(const int32_t *__restrict__ q2k, int topk, int T,
                                           const DocSpan *__restrict__ docs,
                                           const int32_t *__restrict__ blk_off, int ndocs, int g, int t,
                                           int (&bg)[kMaxTopk]) {
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) bg[j] = -1;
    if (t >= T) return;
    int lo = 0, hi = ndocs - 1;  // the document: the last whose start <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (docs[mid].start <= t) lo = mid; else hi = mid - 1;
    }
    const int c = (t - docs[lo].start) / kBlock;
    const int base = blk_off[lo];
    const int32_t *r = q2k + (size_t(g) * T + t) * topk;
    int b[kMaxTopk];
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) b[j] = j < topk ? r[j] : -1;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
        bool dup = false;
#pragma unroll
        for (int i = 0; i < j; ++i) dup |= b[i] == b[j];
        if (b[j] >= 0 && b[j] <= c && !dup) bg[j] = base + b[j];
    }
}

// Workgroup (tile, g): hist[tile][g * nb_max + Bg] = the tile's tokens in list (g, Bg).
__global__ __launch_bounds__(kListTile) void bwd_hist_kernel(const int32_t *__restrict__ q2k, int topk, int T,
                                                             const DocSpan *__restrict__ docs,
                                                             const int32_t *__restrict__ blk_off, int ndocs,
                                                             int nb_max, int nlists, int32_t *__restrict__ hist) {
    __shared__ int s_h[kListWin];
    const int tile = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    int bg[kMaxTopk];
    row_blocks(q2k, topk, T, docs, blk_off, ndocs, g, tile * kListTile + tid, bg);
    for (int w0 = 0; w0 < nb_max; w0 += kListWin) {
        for (int i = tid; i < kListWin; i += kListTile) s_h[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j)
            if (bg[j] >= w0 && bg[j] < w0 + kListWin) atomicAdd(&s_h[bg[j] - w0], 1);
        __syncthreads();
        for (int i = tid; i < kListWin && w0 + i < nb_max; i += kListTile)
            hist[size_t(tile) * nlists + g * nb_max + w0 + i] = s_h[i];
        __syncthreads();
    }
}

// Thread li: hist[tile][li] becomes the exclusive prefix over the tiles,
// cnt[li] the list's length.
__global__ __launch_bounds__(256) void bwd_colscan_kernel(int32_t *__restrict__ hist, int ntiles, int nlists,
                                                          int32_t *__restrict__ cnt) {
    const int li = blockIdx.x * 256 + threadIdx.x;
    if (li >= nlists) return;
    constexpr int kBatch = 16;  // loads in flight together
    int run = 0;
    for (int t0 = 0; t0 < ntiles; t0 += kBatch) {
        int x[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) x[i] = t0 + i < ntiles ? hist[size_t(t0 + i) * nlists + li] : 0;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (t0 + i < ntiles) hist[size_t(t0 + i) * nlists + li] = run;
            run += x[i];
        }
    }
    cnt[li] = run;
}

// Workgroup (tile, g): each of the tile's entries written at its list's
// offset + the tokens of earlier tiles + the earlier tokens of its tile.
__global__ __launch_bounds__(kListTile) void bwd_fill_kernel(const int32_t *__restrict__ q2k, int topk, int T,
                                                             const DocSpan *__restrict__ docs,
                                                             const int32_t *__restrict__ blk_off, int ndocs,
                                                             int nb_max, int nlists, const int32_t *__restrict__ hist,
                                                             const int32_t *__restrict__ list_off,
                                                             int32_t *__restrict__ lists) {
    constexpr int kWaves = kListTile / 64;
    __shared__ unsigned long long s_m[kWaves][kListWin];  // lanes of wave w selecting block w0 + x
    const int tile = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int t = tile * kListTile + tid;
    int bg[kMaxTopk];
    row_blocks(q2k, topk, T, docs, blk_off, ndocs, g, t, bg);
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int w0 = 0; w0 < nb_max; w0 += kListWin) {
        for (int i = tid; i < kWaves * kListWin; i += kListTile) (&s_m[0][0])[i] = 0ull;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j)
            if (bg[j] >= w0 && bg[j] < w0 + kListWin) atomicOr(&s_m[wave][bg[j] - w0], 1ull << lane);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMaxTopk; ++j) {
            if (bg[j] < w0 || bg[j] >= w0 + kListWin) continue;
            const int x = bg[j] - w0;
            int rank = __popcll(s_m[wave][x] & below);
            for (int w = 0; w < wave; ++w) rank += __popcll(s_m[w][x]);
            const int li = g * nb_max + bg[j];
            lists[list_off[li] + hist[size_t(tile) * nlists + li] + rank] = t;
        }
        __syncthreads();
    }
}

// Exclusive scans of n list lengths: list_off[0..n] and chunk_off[0..n]
// (kBwdChunk tokens per chunk).  One workgroup.
__global__ __launch_bounds__(1024) void bwd_scan_kernel(const int32_t *__restrict__ cnt, int n,
                                                        int32_t *__restrict__ list_off,
                                                        int32_t *__restrict__ chunk_off) {
    __shared__ int wsum_a[16], wsum_b[16];
    __shared__ int carry_a, carry_b;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry_a = carry_b = 0;
        list_off[0] = chunk_off[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < n; base += 1024) {
        const int i = base + tid;
        int a = i < n ? cnt[i] : 0;
        int c = (a + kBwdChunk - 1) / kBwdChunk;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int ya = __shfl_up(a, o), yc = __shfl_up(c, o);
            if (lane >= o) { a += ya; c += yc; }
        }
        if (lane == 63) { wsum_a[wave] = a; wsum_b[wave] = c; }
        __syncthreads();
        int pa = carry_a, pc = carry_b;
        for (int w = 0; w < wave; ++w) { pa += wsum_a[w]; pc += wsum_b[w]; }
        if (i < n) {
            list_off[i + 1] = pa + a;
            chunk_off[i + 1] = pc + c;
        }
        __syncthreads();
        if (tid == 1023) { carry_a = pa + a; carry_b = pc + c; }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// dQ (query-major)
// ---------------------------------------------------------------------------
namespace {
constexpr int kQTok = kAttnTile;                      // 16 tokens per workgroup
constexpr int kQWaves = kQTok / 2;                    // 8 waves, 2 tokens each
constexpr int kQThreads = 64 * kQWaves;               // 512
constexpr int kUnitsPerBlock = kBlock / kAttnUnit;    // 4
constexpr int kHalfBytes = kAttnUnit * kRowB;         // 8 KiB: 32 K rows (or V rows)
constexpr int kQUnitBytes = 2 * kHalfBytes;           // K rows, then V rows
constexpr int kQRing = 2 * kUnitsPerBlock + 1;        // 9 slots (144 KiB)
static_assert(kQRing * kQUnitBytes <= 144 * 1024, "ring must leave LDS for the union tables");
constexpr int kQMaxUnion = kQTok * kMaxTopk;               // distinct blocks of a tile at most (256)
constexpr int kQMaxUnits = kUnitsPerBlock * kQMaxUnion;    // ring units of a tile at most
// Unit state words in LDS: bits 0-7 count the waves that still have to read
// the unit, kQClaimed marks its copies issued.  Whether they have landed is
// read from the ring slot's flag.
constexpr uint32_t kQClaimed = 0x100u;
constexpr int kQSpinLimit = 1 << 14;  // polls before a wait gives up (never reached in a correct run)

// Unit ids 0..kQMaxUnits-1 in device memory: the source of the ready flags'
// copies (a slot's flag holds the id of the unit whose copies last landed).
struct QUnitIds {
    int v[kQMaxUnits];
    constexpr QUnitIds() : v() {
        for (int i = 0; i < kQMaxUnits; ++i) v[i] = i;
    }
};
__device__ const QUnitIds kQUnitIds = QUnitIds();

// Row r = 8a + 4m + e (a, e < 4) of a 32-row half, 16-byte chunk c
// (d 8c..8c+7), sits at chunk position c ^ swz32(r), swz32 = 4e + 2(a%2) +
// a/2.  The 16 rows one plain operand read touches (a, e < 4, m fixed) map
// to 16 distinct positions, and the 8 rows of a transposing read's 32-lane
// half (a in {0, 1} or {2, 3}, e < 4, m = h) to 8 distinct position pairs
// (swz32 / 2 = 2e + a%2 differs).
__device__ __forceinline__ int swz32(int r) { return ((r & 3) << 2) | ((r >> 2) & 2) | ((r >> 4) & 1); }

struct DqState {
    bf16x8 qb[2][4];   // Q^T operand of each token (column n = head n)
    bf16x8 dob[2][4];  // dO^T operand
    f32x4 acc[2][8];   // dQ^T: lane holds d = 16dt + 4grp + i of head n
    float lse2[2];     // log2-domain log-sum-exp of head n
    float dsum[2];     // D of head n
};

// One ring unit (unit q of its block, K rows at Ku, V rows after them) for
// one wave (kA0 / kA1: which tokens compute; kDiag: the query's own block,
// causal mask, tokens from act_rt).
template <bool kA0, bool kA1, bool kDiag>
__device__ __forceinline__ void dq_unit(DqState &st, const uint8_t *Ku, int q, const int (&k_row_off)[2], int nsw,
                                        int grp, const int (&tr_row)[2], const int (&tr_x)[2], int tr_lo, int keyb,
                                        const bool (&act_rt)[2], const int (&my_p)[2], float scale_log2) {
    const bool act[2] = {kDiag ? act_rt[0] : kA0, kDiag ? act_rt[1] : kA1};
    const uint8_t *Vu = Ku + kHalfBytes;
    bf16x8 ka[4][2], va[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int off = k_row_off[mt] + (((4 * ks + grp) ^ nsw) << 4);
            ka[ks][mt] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Ku + off));
            va[ks][mt] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Vu + off));
        }
    // S^T and dP^T for this unit; lane (n, grp) holds keys 8grp + 4mt + i
    bf16x8 dsb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (!act[t]) continue;
        f32x4 s[2] = {f32x4{}, f32x4{}}, dp[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                s[mt] = mfma_16x16x32(ka[ks][mt], st.qb[t][ks], s[mt]);
                dp[mt] = mfma_16x16x32(va[ks][mt], st.dob[t][ks], dp[mt]);
            }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = !kDiag || keyb + kAttnUnit * q + 4 * mt + i <= my_p[t];
                const float p = ok ? __builtin_amdgcn_exp2f(s[mt][i] * scale_log2 - st.lse2[t]) : 0.f;
                dsb[t][4 * mt + i] = (__bf16)(p * (dp[mt][i] - st.dsum[t]));
            }
    }
    // dQ^T += K^T dS^T: K^T rows d = 16dt + j, keys 8grp + e from two
    // transposing reads of K rows 8grp..8grp+3 and 8grp+4..8grp+7
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 kt = join_tr(read_tr(Ku + tr_row[0] + (((2 * dt) ^ tr_x[0]) << 4) + tr_lo),
                                  read_tr(Ku + tr_row[1] + (((2 * dt) ^ tr_x[1]) << 4) + tr_lo));
#pragma unroll
        for (int t = 0; t < 2; ++t)
            if (act[t]) st.acc[t][dt] = mfma_16x16x32(kt, dsb[t], st.acc[t][dt]);
    }
}
}  // namespace

__global__ __launch_bounds__(kQThreads) void bwd_dq_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ dout, const uint16_t *__restrict__ o, const float *__restrict__ lse,
    float *__restrict__ Dsum, const int32_t *__restrict__ q2k, int topk, const DocSpan *__restrict__ docs,
    const int32_t *__restrict__ tile_off, int ndocs, int T, float scale, float scale_log2,
    uint16_t *__restrict__ dq) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr int kEntries = kQTok * kMaxTopk;
    static_assert(kQThreads >= kEntries, "one thread per (token, slot) pair");
    // The union tables (s_id, s_first, s_mask, s_ublk, s_umask) are dead once
    // the walk starts; their space then holds the waves' visit lists.
    constexpr int kVisits = kUnitsPerBlock * 2 * kMaxTopk;  // visits of a wave at most
    static_assert(kQWaves * kVisits <= 5 * kEntries, "visit lists fit the union tables");
    __shared__ int s_tab[5 * kEntries];
    int *const s_id = s_tab, *const s_first = s_tab + kEntries, *const s_mask = s_tab + 2 * kEntries;
    int *const s_ublk = s_tab + 3 * kEntries, *const s_umask = s_tab + 4 * kEntries;
    uint32_t *const s_vis = reinterpret_cast<uint32_t *>(s_tab);  // [kQWaves][kVisits]
    __shared__ int s_nu;
    __shared__ uint32_t s_unit[kQMaxUnits];     // per ring unit: claimed bit | waves still to read it
    __shared__ int s_wlist[kQWaves][2 * kMaxTopk];  // per wave: the union blocks it needs, ascending
    __shared__ int s_flag[kQRing][64];          // per ring slot: id of the unit that has landed there

    // XCD-aware order, as in the forward: XCD x serves KV head x/2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, xslot = bid >> 3;
    const int g = xcd >> 1;
    const int tile = 16 * (xslot >> 3) + 8 * (xcd & 1) + (xslot & 7);
    if (tile >= tile_off[ndocs]) return;
    const int d = prefix_doc(tile_off, ndocs, tile);
    const int nt_doc = tile_off[d + 1] - tile_off[d];
    const int local_tile = nt_doc - 1 - (tile - tile_off[d]);
    const DocSpan doc = docs[d];
    const int p0 = local_tile * kQTok;
    const int c = p0 / kBlock;
    const int ntok = min(kQTok, doc.len - p0);
    const int p_last = p0 + ntok - 1;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int head = g * kGroup + n;

    int my_p[2];
    bool tok_ok[2];
    DqState st;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        my_p[t] = p0 + 2 * wave + t;
        tok_ok[t] = 2 * wave + t < ntok;
        const size_t row = size_t(doc.start + (tok_ok[t] ? my_p[t] : p0)) * kHeads + head;
        const uint16_t *qs = q + row * kDim, *ds = dout + row * kDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            st.qb[t][ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qs + 32 * ks + 8 * grp));
            st.dob[t][ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(ds + 32 * ks + 8 * grp));
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.acc[t][dt] = f32x4{};
        st.lse2[t] = lse[row] * kLog2e;
        // D = rowsum(dO * O) of row (token, head n): this lane's 32 of its
        // 128 products (d = 32ks + 8grp .. +7), then the 4 lanes of the row.
        // dK/dV (launched after this kernel) reads it from Dsum.
        const uint16_t *os = o + row * kDim;
        float dsp = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 ob = __builtin_bit_cast(bf16x8, *(const u32x4 *)(os + 32 * ks + 8 * grp));
#pragma unroll
            for (int j = 0; j < 8; ++j) dsp += float(st.dob[t][ks][j]) * float(ob[j]);
        }
        dsp += __shfl_xor(dsp, 16);
        dsp += __shfl_xor(dsp, 32);
        st.dsum[t] = dsp;
        if (grp == 0 && tok_ok[t]) Dsum[row] = dsp;
    }
    // use the loaded operands once here, so that the compiler's wait for them
    // sits before the block loop (a wait inside it would drain the prefetch)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(st.qb[t][ks]), "v"(st.dob[t][ks]));
        asm volatile("" ::"v"(st.lse2[t]), "v"(st.dsum[t]));
    }

    const int nu = tile_union(q2k, T, topk, g, doc.start + p0, ntok, c, tid, s_id, s_first, s_mask,
                              s_ublk, s_umask, &s_nu);
    const int last_units =
        (nu > 0 && s_ublk[nu - 1] == c) ? (p_last - c * kBlock) / kAttnUnit + 1 : kUnitsPerBlock;
    // Ring order, unit-major: unit 0 of every union block (ascending), then
    // unit 1, and so on.  Only existing units are numbered: the query's own
    // block, last in the union, stops at the unit of the tile's last token.
    // Any kQRing consecutive units then span kQRing blocks, most of which
    // several waves need; in block-major order a window spans two or three
    // blocks that only some waves need, and the others wait for ring slots.
    const int nunits = kUnitsPerBlock * (nu - 1) + last_units;
    auto unit_id = [&](int qq, int bi) { return qq * nu - max(0, qq - last_units) + bi; };

    // Unit copies, all 16 issued by the wave that claims the unit: copy
    // pair i fills K rows and V rows 4i..4i+3 (lane l: row 4i + l/16,
    // position l%16, i.e. chunk (l%16) ^ swz32(row)), from the unit's first
    // row in scalar registers and a 32-bit lane offset.  Rows past p_last
    // re-read row p_last.  A 17th copy puts the unit's id into
    // the slot's flag: a wave's copies land in issue order, so the flag shows
    // the rows landed.
    auto issue_unit = [&](int vu, int ub, int qq) {
        uint8_t *slot = smem + (vu % kQRing) * kQUnitBytes;
        const int key0 = ub * kBlock + qq * kAttnUnit;
        const size_t row0 = (size_t(doc.start + key0) * kKvHeads + g) * kDim;
        const int lim = p_last - key0;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
            const int r = 4 * ii + (lane >> 4);
            const uint32_t voff = uint32_t(min(r, lim) * (kKvHeads * kRowB) + (((lane & 15) ^ swz32(r)) << 4));
            copy_to_lds_s(k + row0, voff, slot + ii * 1024);
            copy_to_lds_s(v + row0, voff, slot + kHalfBytes + ii * 1024);
        }
        const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)&s_flag[vu % kQRing][0]);
        asm volatile("global_load_lds_dword %0, off" ::"v"(&kQUnitIds.v[vu]), "{m0}"(m0) : "memory");
    };

    // Unit counts (the waves whose tokens selected the unit's block; units of
    // the query's own block past the tile's last token do not exist) and each
    // wave's list of the blocks it needs, ascending.
    for (int u = tid; u < nunits; u += kQThreads) {
        const int u1 = u - last_units * nu;
        const int bi = u1 < 0 ? u % nu : u1 % max(nu - 1, 1);
        const int m = s_umask[bi];
        int nw = 0;
#pragma unroll
        for (int w = 0; w < kQWaves; ++w) nw += ((m >> (2 * w)) & 3) ? 1 : 0;
        s_unit[u] = uint32_t(nw);
    }
    int nwb = 0;
    for (int u0 = 0; u0 < nu; u0 += 64) {
        const int u = min(u0 + lane, nu - 1);
        const bool mine = u0 + lane < nu && ((s_umask[u] >> (2 * wave)) & 3);
        const uint64_t mm = __ballot(mine);
        if (mine) s_wlist[wave][nwb + __popcll(mm & ((1ull << lane) - 1ull))] = u;
        nwb += __popcll(mm);
    }
    for (int i = tid; i < kQRing * 64; i += kQThreads) (&s_flag[0][0])[i] = -1;
    __syncthreads();
    // The wave's visits in ring order (lane k holds its k-th list block, for
    // each of the block's units): the unit's id (bits 0-9), its index in the
    // block (bits 10-11), the wave's tokens that selected the block (bits
    // 12-13) and the block's id (bits 14-31).  The walk reads them from LDS
    // one visit ahead: a list held in VGPRs was spilled, and each scratch
    // reload's vmcnt wait drained the copies the wave had issued ahead.
    static_assert(kQMaxUnits <= 1024 && kBwdMaxTokens / kBlock <= (1 << 18), "visit entry fields");
    const int lw = (nwb > 0 && s_wlist[wave][nwb - 1] == nu - 1) ? last_units : kUnitsPerBlock;
    const int nvis = nwb > 0 ? kUnitsPerBlock * (nwb - 1) + lw : 0;
    int bi = 0;
    uint32_t e = 0u;
    if (lane < nwb) {
        bi = s_wlist[wave][lane];
        e = uint32_t((s_umask[bi] >> (2 * wave)) & 3) << 12 | uint32_t(s_ublk[bi]) << 14;
    }
    __syncthreads();  // every wave has read the union tables
    if (lane < nwb) {
        const int nq = lane == nwb - 1 ? lw : kUnitsPerBlock;
        for (int qq = 0; qq < nq; ++qq)
            s_vis[wave * kVisits + qq * nwb - max(0, qq - lw) + lane] = uint32_t(unit_id(qq, bi)) | uint32_t(qq) << 10 | e;
    }

    // Lane-constant LDS offsets.  Plain reads: M-tile mt row n is key
    // 8(n/4) + 4mt + n%4, whose swz32 is nsw.  Transposing reads h = 0, 1:
    // this lane supplies row 8grp + 4h + n/4, columns 16dt + 4(n%4)..+3.
    int k_row_off[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) k_row_off[mt] = (8 * (n >> 2) + 4 * mt + (n & 3)) * kRowB;
    const int nsw = swz32(8 * (n >> 2) + (n & 3));
    int tr_row[2], tr_x[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 8 * grp + 4 * h + (n >> 2);
        tr_row[h] = r * kRowB;
        tr_x[h] = swz32(r) ^ ((n & 3) >> 1);
    }
    const int tr_lo = (n & 1) * 8;

    // Unit state, read by every lane (LDS broadcast); changed by lane 0.
    auto unit_word = [&](int u) {
        return __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&s_unit[u], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
    };
    // Slot u % kQRing is free for unit u once every wave needing unit u - kQRing is done with it.
    auto fillable = [&](int u) { return u < kQRing || (unit_word(u - kQRing) & 0xFFu) == 0u; };
    auto try_claim = [&](int u) {
        uint32_t old = kQClaimed;
        if (lane == 0) old = __hip_atomic_fetch_or(&s_unit[u], kQClaimed, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        return (__builtin_amdgcn_readfirstlane(old) & kQClaimed) == 0u;
    };
    auto landed = [&](int u) {
        return __builtin_amdgcn_readfirstlane(
                   __hip_atomic_load(&s_flag[u % kQRing][lane], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) == u;
    };
    // Wait until unit u has landed; claim and copy it when nobody has and its
    // slot is free.  Every wait is bounded (kQSpinLimit polls).
    auto acquire = [&](int u, int ub, int qq) {
        for (int spin = 0; spin < kQSpinLimit; ++spin) {
            if (landed(u)) return;
            const uint32_t wd = unit_word(u);
            if (!(wd & kQClaimed) && fillable(u) && try_claim(u)) issue_unit(u, ub, qq);
            __builtin_amdgcn_s_sleep(1);
        }
    };

    // The wave's walk over its visits, in ring order.  Before computing a
    // unit it claims the next one it needs, when that unit's slot is free,
    // and issues its copies, which land during the compute; the slowest wave
    // can always claim its next unit, since every unit kQRing places earlier
    // was needed only by waves at or beyond it.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): operands are in (no copy issued yet)
    uint32_t nx = nvis > 0 ? __builtin_amdgcn_readfirstlane(s_vis[wave * kVisits]) : 0u;
#pragma unroll 1
    for (int i = 0; i < nvis; ++i) {
        const uint32_t x = nx;
        const int u = x & 1023u, qq = (x >> 10) & 3u, b = int(x >> 14);
        const bool act[2] = {tok_ok[0] && ((x >> 12) & 1u), tok_ok[1] && ((x >> 13) & 1u)};
        // One LDS round trip: u's flag, the next visit, the next unit's
        // state and the state of the unit before it in its slot.
        nx = i + 1 < nvis ? __builtin_amdgcn_readfirstlane(s_vis[wave * kVisits + i + 1]) : 0u;
        const int vn = i + 1 < nvis ? int(nx & 1023u) : -1;
        const int vs = vn >= 0 ? vn : u;
        const int vp = vn >= kQRing ? vn - kQRing : u;
        const int fl = __hip_atomic_load(&s_flag[u % kQRing][lane], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t wv = __hip_atomic_load(&s_unit[vs], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t wp = __hip_atomic_load(&s_unit[vp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(fl) != u) acquire(u, b, qq);
        // claim the next unit ahead (a unit only this wave needs is marked
        // with a non-returning atomic)
        const uint32_t wvs = __builtin_amdgcn_readfirstlane(wv);
        if (vn >= 0 && !(wvs & kQClaimed) && (vn < kQRing || (__builtin_amdgcn_readfirstlane(wp) & 0xFFu) == 0u)) {
            const int nb = int(nx >> 14), nqq = (nx >> 10) & 3u;
            if ((wvs & 0xFFu) == 1u) {
                if (lane == 0) __hip_atomic_fetch_or(&s_unit[vn], kQClaimed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                issue_unit(vn, nb, nqq);
            } else if (try_claim(vn)) {
                issue_unit(vn, nb, nqq);
            }
        }
        const int keyb = b * kBlock + 8 * grp;
        const uint8_t *Ku = smem + (u % kQRing) * kQUnitBytes;
        if (b == c)
            dq_unit<true, true, true>(st, Ku, qq, k_row_off, nsw, grp, tr_row, tr_x, tr_lo, keyb, act, my_p,
                                      scale_log2);
        else if (act[0] && act[1])
            dq_unit<true, true, false>(st, Ku, qq, k_row_off, nsw, grp, tr_row, tr_x, tr_lo, keyb, act, my_p,
                                       scale_log2);
        else if (act[0])
            dq_unit<true, false, false>(st, Ku, qq, k_row_off, nsw, grp, tr_row, tr_x, tr_lo, keyb, act, my_p,
                                        scale_log2);
        else if (act[1])
            dq_unit<false, true, false>(st, Ku, qq, k_row_off, nsw, grp, tr_row, tr_x, tr_lo, keyb, act, my_p,
                                        scale_log2);
        // done reading unit u
        if (lane == 0) __hip_atomic_fetch_sub(&s_unit[u], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every copy this wave issued has landed

#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (!tok_ok[t]) continue;
        uint16_t *dst = dq + (size_t(doc.start + my_p[t]) * kHeads + head) * kDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (__bf16)(st.acc[t][dt][i] * scale);
            *(bf16x4 *)(dst + 16 * dt + 4 * grp) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// dK, dV (key-major)
// ---------------------------------------------------------------------------
namespace {
constexpr int kKvTok = 4;                      // tokens per step
constexpr int kKvRows = kKvTok * kGroup;       // 64 query rows per step
constexpr int kStageBytes = kKvRows * kRowB;   // 16 KiB of Q (or dO) rows
constexpr int kStageAll = 2 * kStageBytes + 2 * kKvRows * 4;  // Q, dO, lse, D of one step
constexpr int kStages = 4;                     // LDS ring: steps s+1..s+3 stream in during step s
constexpr int kKvWaves = 8;                    // waves per workgroup, two per SIMD
constexpr int kKeyTiles = kBlock / (16 * kKvWaves);  // 16-key tiles per wave (1)

// HBM -> LDS copy of 4 bytes per lane (lane l writes lds_dst + 4l).
__device__ __forceinline__ void copy_dword_to_lds(const void *src, uint8_t *lds_dst) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)lds_dst);
    asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// Wait until at most n (<= 31) of this wave's copies are outstanding.
__device__ __forceinline__ void wait_copies32(int n) {
#define MSA_W(i) case i: asm volatile("s_waitcnt vmcnt(" #i ")" ::: "memory"); break;
    switch (n) {
        MSA_W(1) MSA_W(2) MSA_W(3) MSA_W(4) MSA_W(5) MSA_W(6) MSA_W(7) MSA_W(8) MSA_W(9) MSA_W(10)
        MSA_W(11) MSA_W(12) MSA_W(13) MSA_W(14) MSA_W(15) MSA_W(16) MSA_W(17) MSA_W(18) MSA_W(19)
        MSA_W(20) MSA_W(21) MSA_W(22) MSA_W(23) MSA_W(24) MSA_W(25) MSA_W(26) MSA_W(27) MSA_W(28)
        MSA_W(29) MSA_W(30) MSA_W(31)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef MSA_W
}

// Row r (0..63) of a staged Q / dO tile, chunk c at position c ^ swz16(r),
// swz16(r) = 2 (r mod 8) + (r / 8 mod 2): the 16 rows 16rt + m of a plain
// operand read map to 16 distinct positions, and a transposing read's
// 32-lane half (rows 16h + 4grp + e for two grp) touches 8 rows x 2 chunks
// at 16 distinct positions, so neither read conflicts in the LDS banks.
__device__ __forceinline__ int swz16(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
}  // namespace

__global__ __launch_bounds__(64 * kKvWaves) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ Dsum,
    const DocSpan *__restrict__ docs, const int32_t *__restrict__ blk_off, int ndocs, int nb_max,
    const int32_t *__restrict__ lists, const int32_t *__restrict__ list_off,
    const int32_t *__restrict__ chunk_off, int nlists, float scale, float scale_log2,
    float *__restrict__ part, uint16_t *__restrict__ dk, uint16_t *__restrict__ dv) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // kStages x (Q, dO, lse, D)
    const int ci = blockIdx.x;
    if (ci >= chunk_off[nlists]) return;
    int lo = 0, hi = nlists - 1;  // list li: the last with chunk_off[li] <= ci
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= ci) lo = mid; else hi = mid - 1;
    }
    const int li = lo;
    const int g = li / nb_max, Bg = li - g * nb_max;
    const int d = prefix_doc(blk_off, ndocs, Bg);
    const DocSpan doc = docs[d];
    const int b = Bg - blk_off[d];
    const int e0 = list_off[li] + (ci - chunk_off[li]) * kBwdChunk;
    const int ne = min(kBwdChunk, list_off[li + 1] - e0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, grp = lane >> 4;

    // this wave's keys kb + 16kt + n as B operands (col = key, k chunk 4ks + grp)
    const int kb = b * kBlock + 16 * kKeyTiles * wave;
    bf16x8 kreg[kKeyTiles][4], vreg[kKeyTiles][4];
#pragma unroll
    for (int kt = 0; kt < kKeyTiles; ++kt) {
        const int kp = min(kb + 16 * kt + n, doc.len - 1);
        const size_t row = (size_t(doc.start + kp) * kKvHeads + g) * kDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kreg[kt][ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(k + row + 8 * (4 * ks + grp)));
            vreg[kt][ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(v + row + 8 * (4 * ks + grp)));
        }
    }
    // use the operands once here, so that the compiler's wait for them sits
    // before the step loop (a wait inside it would also drain the prefetch)
#pragma unroll
    for (int kt = 0; kt < kKeyTiles; ++kt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(kreg[kt][ks]), "v"(vreg[kt][ks]));
    f32x4 dkt[kKeyTiles][8], dvt[kKeyTiles][8];  // [key tile][d tile]: key 16kt + n, d 16dt + 4grp + i
#pragma unroll
    for (int kt = 0; kt < kKeyTiles; ++kt)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dkt[kt][dt] = dvt[kt][dt] = f32x4{};

    // Stage s: tokens e0 + 4s .. +3 (past the list end: its last token,
    // masked).  32 one-KiB copies (16 of Q, 16 of dO rows), 4 per wave;
    // copy cc fills rows 4cc..4cc+3 = heads 4(cc%4).. of token cc/4.  Wave 0
    // also copies the 4 tokens' lse rows, wave 1 their D rows (64 floats,
    // [token][head]), so that the step loop issues no vector load of its own
    // (the compiler would wait for it, and with it for the whole prefetch).
    const int nsteps = (ne + kKvTok - 1) / kKvTok;
    constexpr int kCopiesPerWave = 32 / kKvWaves;
    const int per_stage = kCopiesPerWave + (wave < 2 ? 1 : 0);
    auto issue_stage = [&](int s, int buf) {
        uint8_t *st = smem + buf * kStageAll;
#pragma unroll
        for (int j = 0; j < kCopiesPerWave; ++j) {
            const int c = kCopiesPerWave * wave + j;
            const int cc = c & 15;
            const int r = 4 * cc + (lane >> 4);
            const int tok = lists[e0 + min(kKvTok * s + (cc >> 2), ne - 1)];
            const int ch = (lane & 15) ^ swz16(r);
            const uint16_t *src =
                (c < 16 ? q : dout) + (size_t(tok) * kHeads + g * kGroup + (r & 15)) * kDim + 8 * ch;
            copy_to_lds(src, st + (c < 16 ? 0 : kStageBytes) + cc * 1024);
        }
        if (wave < 2) {
            int t4[kKvTok];  // wave-uniform (scalar) loads; the lane picks its token
#pragma unroll
            for (int j = 0; j < kKvTok; ++j) t4[j] = lists[e0 + min(kKvTok * s + j, ne - 1)];
            const int tj = lane >> 4;
            const int tok = tj == 0 ? t4[0] : tj == 1 ? t4[1] : tj == 2 ? t4[2] : t4[3];
            const float *src = (wave == 0 ? lse : Dsum) + size_t(tok) * kHeads + g * kGroup + (lane & 15);
            copy_dword_to_lds(src, st + 2 * kStageBytes + wave * (kKvRows * 4));
        }
    };

    // lane-constant offsets: plain read of row 16rt + n, chunk 4ks + grp;
    // transposing read h supplies row 16(2s2 + h) + 4grp + n/4, cols 16dt + 4(n%4)
    const int a_off = n * kRowB;
    const int a_sw = swz16(n);
    int tr_row[2], tr_x[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 16 * h + 4 * grp + (n >> 2);
        tr_row[h] = r * kRowB;
        tr_x[h] = swz16(r) ^ ((n & 3) >> 1);
    }
    const int tr_lo = (n & 1) * 8;

    // queries' operands are in registers before the first copy is issued
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    for (int s = 0; s < min(nsteps, kStages - 1); ++s) issue_stage(s, s);
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s % kStages;
        if (s + kStages - 1 < nsteps) issue_stage(s + kStages - 1, (s + kStages - 1) % kStages);
        // copies complete in issue order: leave the later stages in flight
        wait_copies32(per_stage * (min(nsteps - 1, s + kStages - 1) - s));
        barrier_keep_prefetch();
        const uint8_t *Qs = smem + buf * kStageAll;
        const uint8_t *Ds = Qs + kStageBytes;
        const float *Ls = (const float *)(Qs + 2 * kStageBytes);
        const float *Dl = Ls + kKvRows;

        // per row tile rt (token 4s + rt): heads 4grp + i
        float lse2[4][4], dsum[4][4];
        int pos[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int e = kKvTok * s + rt;
            const int tok = lists[e0 + min(e, ne - 1)];
            pos[rt] = e < ne ? tok - doc.start : -1;  // -1: no key passes the mask
            const f32x4 l4 = *(const f32x4 *)(Ls + 16 * rt + 4 * grp);
            const f32x4 d4 = *(const f32x4 *)(Dl + 16 * rt + 4 * grp);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lse2[rt][i] = l4[i] * kLog2e;
                dsum[rt][i] = d4[i];
            }
        }
        // S = Q K^T and dP = dO V^T; lane holds key 16kt + n, rows 4grp + i
        bf16x8 pb[2][kKeyTiles], dsb[2][kKeyTiles];  // [k-step s2 = rt/2][kt]: rows 16rt + 4grp + i at 4(rt%2) + i
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 sacc[kKeyTiles] = {}, pacc[kKeyTiles] = {};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = 16 * rt * kRowB + a_off + (((4 * ks + grp) ^ a_sw) << 4);
                const bf16x8 qa = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Qs + off));
                const bf16x8 da = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Ds + off));
#pragma unroll
                for (int kt = 0; kt < kKeyTiles; ++kt) {
                    sacc[kt] = mfma_16x16x32(qa, kreg[kt][ks], sacc[kt]);
                    pacc[kt] = mfma_16x16x32(da, vreg[kt][ks], pacc[kt]);
                }
            }
            // Only a row whose token lies in the wave's keys (or a padding
            // row, pos -1) masks keys: a wave-uniform branch, so that the
            // other rows skip the compare and select per score.  A masked
            // score becomes -inf, whose exponential is 0.
            if (pos[rt] < kb + 16 * kKeyTiles - 1) {
#pragma unroll
                for (int kt = 0; kt < kKeyTiles; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (kb + 16 * kt + n > pos[rt]) sacc[kt][i] = -INFINITY;
            }
#pragma unroll
            for (int kt = 0; kt < kKeyTiles; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(sacc[kt][i] * scale_log2 - lse2[rt][i]);
                    pb[rt >> 1][kt][4 * (rt & 1) + i] = (__bf16)p;
                    dsb[rt >> 1][kt][4 * (rt & 1) + i] = (__bf16)(p * (pacc[kt][i] - dsum[rt][i]));
                }
        }
        // dV^T += dO^T P, dK^T += Q^T dS over the 64 rows (two k-steps of 32)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int o0 = 32 * s2 * kRowB + tr_row[0] + (((2 * dt) ^ tr_x[0]) << 4) + tr_lo;
                const int o1 = 32 * s2 * kRowB + tr_row[1] + (((2 * dt) ^ tr_x[1]) << 4) + tr_lo;
                const bf16x8 doT = join_tr(read_tr(Ds + o0), read_tr(Ds + o1));
                const bf16x8 qT = join_tr(read_tr(Qs + o0), read_tr(Qs + o1));
#pragma unroll
                for (int kt = 0; kt < kKeyTiles; ++kt) {
                    dvt[kt][dt] = mfma_16x16x32(doT, pb[s2][kt], dvt[kt][dt]);
                    dkt[kt][dt] = mfma_16x16x32(qT, dsb[s2][kt], dkt[kt][dt]);
                }
            }
        barrier_keep_prefetch();  // every wave is done with buf before it is refilled
    }

    if (chunk_off[li + 1] - chunk_off[li] == 1) {
        // the block's only chunk: its sums are final, written as bf16
#pragma unroll
        for (int kt = 0; kt < kKeyTiles; ++kt) {
            const int kp = kb + 16 * kt + n;
            if (kp >= doc.len) continue;
            const size_t row = (size_t(doc.start + kp) * kKvHeads + g) * kDim + 4 * grp;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                bf16x4 a, c;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = (__bf16)(dkt[kt][dt][i] * scale);
                    c[i] = (__bf16)dvt[kt][dt][i];
                }
                *(bf16x4 *)(dk + row + 16 * dt) = a;
                *(bf16x4 *)(dv + row + 16 * dt) = c;
            }
        }
        return;
    }
    float *pk = part + size_t(ci) * 2 * kBlock * kDim;
    float *pv = pk + kBlock * kDim;
#pragma unroll
    for (int kt = 0; kt < kKeyTiles; ++kt) {
        const int key = 16 * kKeyTiles * wave + 16 * kt + n;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            *(f32x4 *)(pk + key * kDim + 16 * dt + 4 * grp) = dkt[kt][dt] * scale;
            *(f32x4 *)(pv + key * kDim + 16 * dt + 4 * grp) = dvt[kt][dt];
        }
    }
}

// Workgroup (Bg, g, z): keys 16z..16z+15 of block Bg, KV head g.  A block
// with several chunks gets its partials summed in chunk order into bf16
// dk, dv; a block no row selects gets zeros; a single-chunk block was
// written by its chunk.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *__restrict__ part,
                                                         const int32_t *__restrict__ chunk_off,
                                                         const DocSpan *__restrict__ docs,
                                                         const int32_t *__restrict__ blk_off, int ndocs,
                                                         int nb_max, uint16_t *__restrict__ dk,
                                                         uint16_t *__restrict__ dv) {
    const int Bg = blockIdx.x, g = blockIdx.y, z = blockIdx.z;
    if (Bg >= blk_off[ndocs]) return;
    const int li = g * nb_max + Bg;
    const int c0 = chunk_off[li], c1 = chunk_off[li + 1];
    if (c1 - c0 == 1) return;
    const int d = prefix_doc(blk_off, ndocs, Bg);
    const DocSpan doc = docs[d];
    const int b = Bg - blk_off[d];
    const int nk = min(kBlock, doc.len - b * kBlock);
    const int tid = threadIdx.x;
    const int which = tid >> 7;            // 0: dk, 1: dv
    const int key = 16 * z + ((tid >> 3) & 15);
    const int col = 16 * (tid & 7);        // 16 consecutive d per thread
    f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
    for (int c = c0; c < c1; ++c) {
        const float *src = part + ((size_t(c) * 2 + which) * kBlock + key) * kDim + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += *(const f32x4 *)(src + 4 * j);
    }
    if (key < nk) {
        uint16_t *dst = (which == 0 ? dk : dv) + (size_t(doc.start + b * kBlock + key) * kKvHeads + g) * kDim + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (__bf16)acc[j][i];
            *(bf16x4 *)(dst + 4 * j) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
BwdLayout bwd_layout(int T, int ndocs, int topk) {
    BwdLayout L;
    L.nb_max = ceil_div(T, kBlock) + ndocs;
    L.nlists = kKvHeads * L.nb_max;
    const size_t pairs = size_t(kKvHeads) * size_t(T) * size_t(topk);
    L.max_chunks = int((pairs + kBwdChunk - 1) / kBwdChunk) + L.nlists;
    L.list_entries = pairs;
    L.ntiles = ceil_div(T, kListTile);
    return L;
}

hipError_t launch_bwd_lists(const int32_t *q2k, int topk, int T, const DocSpan *docs,
                            const int32_t *blk_off, int ndocs, const BwdLayout &L, int32_t *hist, int32_t *cnt,
                            int32_t *list_off, int32_t *chunk_off, int32_t *lists, hipStream_t stream) {
    const dim3 grid(L.ntiles, kKvHeads);
    hipLaunchKernelGGL(bwd_hist_kernel, grid, dim3(kListTile), 0, stream, q2k, topk, T, docs, blk_off, ndocs,
                       L.nb_max, L.nlists, hist);
    hipLaunchKernelGGL(bwd_colscan_kernel, dim3(ceil_div(L.nlists, 256)), dim3(256), 0, stream, hist, L.ntiles,
                       L.nlists, cnt);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, stream, (const int32_t *)cnt, L.nlists,
                       list_off, chunk_off);
    hipLaunchKernelGGL(bwd_fill_kernel, grid, dim3(kListTile), 0, stream, q2k, topk, T, docs, blk_off, ndocs,
                       L.nb_max, L.nlists, (const int32_t *)hist, (const int32_t *)list_off, lists);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                         const uint16_t *o, const float *lse, float *Dsum, const int32_t *q2k, int topk,
                         const DocSpan *docs, const int32_t *tile_off, int ndocs, int T, float scale,
                         uint16_t *dq, hipStream_t stream) {
    const int max_tiles = ceil_div(T, kQTok) + ndocs;
    const int grid = 8 * 8 * ceil_div(max_tiles, 16);
    const size_t lds = size_t(kQRing) * kQUnitBytes;
    static const bool fits = lds_fits(reinterpret_cast<const void *>(bwd_dq_kernel), lds);
    if (!fits) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(grid), dim3(kQThreads), lds, stream, q, k, v, dout, o, lse, Dsum,
                       q2k, topk, docs, tile_off, ndocs, T, scale, scale * kLog2e, dq);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                           const float *lse, const float *Dsum, const DocSpan *docs,
                           const int32_t *blk_off, int ndocs, const BwdLayout &L, const int32_t *lists,
                           const int32_t *list_off, const int32_t *chunk_off, float scale, float *part,
                           uint16_t *dk, uint16_t *dv, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(L.max_chunks), dim3(64 * kKvWaves), size_t(kStages) * kStageAll, stream,
                       q, k, v, dout, lse, Dsum,
                       docs, blk_off, ndocs, L.nb_max, lists, list_off, chunk_off, L.nlists, scale,
                       scale * kLog2e, part, dk, dv);
    return hipGetLastError();
}

hipError_t launch_bwd_reduce(const float *part, const int32_t *chunk_off, const DocSpan *docs,
                             const int32_t *blk_off, int ndocs, const BwdLayout &L, uint16_t *dk,
                             uint16_t *dv, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3(L.nb_max, kKvHeads, kBlock / 16), dim3(256), 0, stream, part, chunk_off,
                       docs, blk_off, ndocs, L.nb_max, dk, dv);
    return hipGetLastError();
}

}  // namespace msa
