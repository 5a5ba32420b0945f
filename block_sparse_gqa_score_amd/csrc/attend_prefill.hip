// Sparse GQA attention over the selected blocks, prefill on packed documents.
//
// Method (NeMo AutoModel minimax_m3_vl.msa, sparse_attention; TensorRT-LLM
// "MiniMaxM3SparseAttentionConfig", class description, step two): query
// head h of token t attends, with softmax over scale * q.k, to the keys of
// t's document at or before t whose document-local 128-key block appears in
// q2k row (h/16, t).
//
// Two kernels:
//   kv_units_kernel - K and V of every document re-laid per 32-key unit:
//       V^T [unit][KV head][d][32 keys], so that the PV operand is read from
//       LDS with plain 16-byte reads, and K [unit][KV head][32 keys][d], so
//       that a unit's K rows of one head are 8 KiB contiguous (in the input
//       they are 256 B apart from each other by the other heads' rows).  Keys
//       past the document end are 0 in both.
//   attend_prefill_kernel - workgroup = (KV head g, 16 consecutive tokens of
//       one document inside one 128-token block, so all share the query
//       block c); 8 waves, each owning 2 tokens x 16 heads.  The workgroup
//       walks the UNION of its tokens' selected blocks in ascending order as
//       32-key units (K rows 8 KiB + V^T rows 8 KiB), copied HBM -> LDS by
//       global_load_lds_dwordx4 into a 9-slot ring; the waves meet at one
//       barrier per union block, while the next five units stream in.  A
//       wave computes a block only for those of its two tokens that selected
//       it, as one chain over the block's 128 keys (one softmax step); the K
//       and V^T fragments it reads from LDS serve both tokens.  Blocks that a
//       single token selected skip the ring: that token's wave reads them
//       straight from memory, one 32-key unit in each ring iteration where it
//       has no token in the ring's block, and the rest after the ring.
//
// Per wave, token and 32-key unit (MFMA 16x16x32 bf16, key rows m, head
// columns n):
//   S^T[32 x 16] = K . Q^T       2 M-tiles x 4 k-steps; M-tile mt row i is key
//                                 8(i/4) + 4mt + i%4, so lane (n, grp) holds
//                                 keys 8grp..8grp+7 of column n in order;
//   causal mask in the query's own block, online softmax in the exp2 domain
//   with lazy rescaling (the reference max only moves when it grows by more
//   than 2^8), P^T packed to bf16 straight from the accumulators,
//   O^T[128 x 16] += V^T . P^T   8 d-tiles x 1 k-step.
#include "attend_common.hpp"

namespace msa {

namespace {
constexpr int kTok = kAttnTile;                        // 16 tokens per workgroup
constexpr int kWaves = kTok / 2;                       // 8 waves, 2 tokens each
constexpr int kThreads = 64 * kWaves;                  // 512
constexpr int kUnitsPerBlock = kBlock / kAttnUnit;     // 4
constexpr int kKUnitBytes = kAttnUnit * kDim * 2;      // 8 KiB of K rows
constexpr int kVUnitBytes = kDim * kAttnUnit * 2;      // 8 KiB of V^T rows
constexpr int kUnitBytes = kKUnitBytes + kVUnitBytes;  // 16 KiB
constexpr int kRing = 9;  // LDS ring slots of one unit each (144 KiB)
constexpr int kLoadsPerWave = kUnitBytes / 1024 / kWaves;  // 2 one-KiB copies
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;  // rescale only when the max grows by > 2^8
constexpr int kSharedMin = 2;     // union blocks this many tokens selected go through the ring

static_assert(kLoadsPerWave == 2, "unit copy split assumes 2 copies per wave");
static_assert(kRing == 2 * kUnitsPerBlock + 1, "one unit of the block after next streams ahead");
static_assert(kRing * kUnitBytes <= 144 * 1024, "ring must leave LDS for the union tables");

// K unit in LDS: row r (key), 16-byte chunk c (d 8c..8c+7) at slot
// 16r + (c ^ kswz(r)).  The 16 lanes of an operand read hold rows
// 8a + 4mt + b (a, b < 4), whose kswz values are the 16 distinct 4a + b.
__device__ __forceinline__ int kswz(int r) { return (((r >> 3) & 3) << 2) | (r & 3); }
// V^T unit in LDS: row d, chunk c (keys 8c..8c+7) at slot 4d + (c ^ vswz(d));
// 16 consecutive rows at one chunk cover all 16 chunk positions of 256 B.
__device__ __forceinline__ int vswz(int d) { return (d >> 2) & 3; }

// Per-wave state: query operands and running softmax of the wave's two
// tokens (column n of each is head n of the KV group).
struct WaveState {
    bf16x8 qb[2][4];
    f32x4 acc_o[2][8];
    float m_ref[2];  // raw-score reference of the exponentials
    float l_run[2];
};

// One union block for one wave.  kA0/kA1: which tokens compute (fixed at
// compile time, so the whole chain is straight-line code the scheduler can
// overlap: LDS reads of unit q+1 run under the MFMAs of unit q).  kDiag:
// the query's own block, with nq <= 4 units, the causal mask, and the
// active tokens taken from act_rt at run time.
template <bool kA0, bool kA1, bool kDiag>
__device__ __forceinline__ void attend_block(WaveState &st, const uint8_t *smem, int ustart, int nq,
                                             const int (&k_row_off)[2], int v_off, int n, int grp,
                                             int keyb, const bool (&act_rt)[2],
                                             const int (&my_p)[2], float scale_log2) {
    const bool act[2] = {kDiag ? act_rt[0] : kA0, kDiag ? act_rt[1] : kA1};
    // S^T for the block: unit q, M-tile mt of token t
    f32x4 sacc[2][kUnitsPerBlock][2];
#pragma unroll
    for (int q = 0; q < kUnitsPerBlock; ++q) {
        if (kDiag && q >= nq) break;
        const uint8_t *Ku = smem + ((ustart + q) % kRing) * kUnitBytes;
        bf16x8 ka[4][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                ka[ks][mt] = __builtin_bit_cast(
                    bf16x8, *(const u32x4 *)(Ku + k_row_off[mt] + (((4 * ks + grp) ^ n) << 4)));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (!act[t]) continue;
            sacc[t][q][0] = f32x4{};
            sacc[t][q][1] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    sacc[t][q][mt] = mfma_16x16x32(ka[ks][mt], st.qb[t][ks], sacc[t][q][mt]);
        }
    }

    // online softmax over the block's keys; this lane holds keys
    // keyb + 32q + e (e < 8) of head column n
    bf16x8 pb[2][kUnitsPerBlock];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (!act[t]) continue;
        float sv[kUnitsPerBlock][8];
#pragma unroll
        for (int q = 0; q < kUnitsPerBlock; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[q][e] = sacc[t][q][e >> 2][e & 3];
        if (kDiag) {  // causal mask; also drops units q >= nq
#pragma unroll
            for (int q = 0; q < kUnitsPerBlock; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sv[q][e] = keyb + kAttnUnit * q + e <= my_p[t] ? sv[q][e] : -INFINITY;
        }
        float mloc = sv[0][0];
#pragma unroll
        for (int q = 0; q < kUnitsPerBlock; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) mloc = fmaxf(mloc, sv[q][e]);
        mloc = row_max4(mloc);
        // lazy reference: move it (and rescale) only on a large increase
        const bool grow = mloc > st.m_ref[t] &&
                          (st.m_ref[t] == -INFINITY || (mloc - st.m_ref[t]) * scale_log2 > kLazyLog2);
        if (__ballot(grow)) {
            const float m_new = grow ? mloc : st.m_ref[t];
            const float alpha = st.m_ref[t] == -INFINITY
                                    ? 0.f
                                    : __builtin_amdgcn_exp2f((st.m_ref[t] - m_new) * scale_log2);
            st.l_run[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) st.acc_o[t][dt] *= alpha;
            st.m_ref[t] = m_new;
        }
        const float mb = st.m_ref[t] == -INFINITY ? 0.f : st.m_ref[t] * scale_log2;
        float psum = 0.f;
#pragma unroll
        for (int q = 0; q < kUnitsPerBlock; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = __builtin_amdgcn_exp2f(sv[q][e] * scale_log2 - mb);
                psum += pv;
                pb[t][q][e] = (__bf16)pv;
            }
        st.l_run[t] += psum;
    }

    // O^T += V^T . P^T, unit by unit
#pragma unroll
    for (int q = 0; q < kUnitsPerBlock; ++q) {
        if (kDiag && q >= nq) break;
        const uint8_t *Vu = smem + ((ustart + q) % kRing) * kUnitBytes + kKUnitBytes;
        bf16x8 va[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            va[dt] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Vu + 1024 * dt + v_off));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (!act[t]) continue;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                st.acc_o[t][dt] = mfma_16x16x32(va[dt], pb[t][q], st.acc_o[t][dt]);
        }
    }
}

}  // namespace

namespace {
// Unit q of a block b < c for token t of a wave, read straight from memory
// (the per-unit K rows and V^T rows are contiguous in the MFMA operand
// layouts), with the lazy online softmax.  Used for blocks a single token of
// the tile selected, which would otherwise hold the whole workgroup at a
// barrier for one wave's work.
template <int t>
__device__ __forceinline__ void attend_unit_global(WaveState &st, const uint16_t *__restrict__ ku,
                                                   const uint16_t *__restrict__ vt, int g, int uoff, int b,
                                                   int q, int n, int grp, float scale_log2) {
    {
        f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const uint16_t *src = ku + ((size_t(uoff + kUnitsPerBlock * b + q) * kKvHeads + g) * kAttnUnit +
                                        8 * (n >> 2) + 4 * mt + (n & 3)) * kDim;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                sacc[mt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, *(const u32x4 *)(src + 8 * (4 * ks + grp))),
                                         st.qb[t][ks], sacc[mt]);
        }
        const uint16_t *vsrc = vt + ((size_t(uoff + kUnitsPerBlock * b + q) * kKvHeads + g) * kDim + n) * kAttnUnit + 8 * grp;
        bf16x8 va[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) va[dt] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(vsrc + 16 * dt * kAttnUnit));
        float mloc = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) mloc = fmaxf(mloc, sacc[e >> 2][e & 3]);
        mloc = row_max4(mloc);
        const bool grow = mloc > st.m_ref[t] &&
                          (st.m_ref[t] == -INFINITY || (mloc - st.m_ref[t]) * scale_log2 > kLazyLog2);
        if (__ballot(grow)) {
            const float m_new = grow ? mloc : st.m_ref[t];
            const float alpha = st.m_ref[t] == -INFINITY
                                    ? 0.f
                                    : __builtin_amdgcn_exp2f((st.m_ref[t] - m_new) * scale_log2);
            st.l_run[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) st.acc_o[t][dt] *= alpha;
            st.m_ref[t] = m_new;
        }
        const float mb = st.m_ref[t] == -INFINITY ? 0.f : st.m_ref[t] * scale_log2;
        float psum = 0.f;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pv = __builtin_amdgcn_exp2f(sacc[e >> 2][e & 3] * scale_log2 - mb);
            psum += pv;
            pb[e] = (__bf16)pv;
        }
        st.l_run[t] += psum;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.acc_o[t][dt] = mfma_16x16x32(va[dt], pb, st.acc_o[t][dt]);
    }
}
}  // namespace

// ---------------------------------------------------------------------------
// K, V -> per-unit K and V^T
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_units_kernel(const uint16_t *__restrict__ k,
                                                       const uint16_t *__restrict__ v,
                                                       const DocSpan *__restrict__ docs,
                                                       const int32_t *__restrict__ unit_off, int ndocs,
                                                       uint16_t *__restrict__ ku, uint16_t *__restrict__ vt) {
    __shared__ uint16_t tile[kAttnUnit][kDim + 2];
    const int U = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    if (U >= unit_off[ndocs]) return;
    const int d = prefix_doc(unit_off, ndocs, U);
    const DocSpan doc = docs[d];
    const int key0 = (U - unit_off[d]) * kAttnUnit;
    // 32 rows x 16 chunks of 16 bytes, 2 per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int id = tid + 256 * i, r = id >> 4, ch = id & 15;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key0 + r < doc.len)
            x = *(const u32x4 *)(v + (size_t(doc.start + key0 + r) * kKvHeads + g) * kDim + 8 * ch);
        u32x4 kx = {0u, 0u, 0u, 0u};
        if (key0 + r < doc.len)
            kx = *(const u32x4 *)(k + (size_t(doc.start + key0 + r) * kKvHeads + g) * kDim + 8 * ch);
        *(u32x4 *)(ku + ((size_t(U) * kKvHeads + g) * kAttnUnit + r) * kDim + 8 * ch) = kx;
        uint32_t *dst = (uint32_t *)&tile[r][8 * ch];  // 4-byte aligned (row pitch 260 B)
        dst[0] = x[0];
        dst[1] = x[1];
        dst[2] = x[2];
        dst[3] = x[3];
    }
    __syncthreads();
    // 128 rows (d) x 4 chunks (8 keys) of 16 bytes, 2 per thread; a wave
    // writes 1 KiB contiguous
    uint16_t *dst = vt + (size_t(U) * kKvHeads + g) * kDim * kAttnUnit;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int id = tid + 256 * i, dd = id >> 2, ch = id & 3;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = uint32_t(tile[8 * ch + 2 * j][dd]) | (uint32_t(tile[8 * ch + 2 * j + 1][dd]) << 16);
        *(u32x4 *)(dst + dd * kAttnUnit + 8 * ch) = o;
    }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attend_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ ku, const uint16_t *__restrict__ vt,
    const int32_t *__restrict__ q2k, int topk, const DocSpan *__restrict__ docs,
    const int32_t *__restrict__ tile_off, const int32_t *__restrict__ unit_off, int ndocs, int T,
    float scale_log2, uint16_t *__restrict__ out, float *__restrict__ lse) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr int kEntries = kTok * kMaxTopk;  // 256 (token, slot) pairs
    static_assert(kThreads >= kEntries, "one thread per (token, slot) pair");
    __shared__ int s_id[kEntries];
    __shared__ int s_first[kEntries];
    __shared__ int s_mask[kEntries];
    __shared__ int s_ublk[kEntries];
    __shared__ int s_umask[kEntries];
    __shared__ int s_sblk[kEntries];   // the ring's blocks: shared ones and the query's own
    __shared__ int s_smask[kEntries];
    __shared__ int s_nu, s_ns;

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; XCD x
    // serves KV head x/2 and alternate groups of 8 tiles (one 128-token query
    // block) of that head, longest first, so the tiles sharing a query block
    // share one L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, xslot = bid >> 3;
    const int g = xcd >> 1;
    const int tile = 16 * (xslot >> 3) + 8 * (xcd & 1) + (xslot & 7);
    if (tile >= tile_off[ndocs]) return;
    const int d = prefix_doc(tile_off, ndocs, tile);
    const int nt_doc = tile_off[d + 1] - tile_off[d];
    const int local_tile = nt_doc - 1 - (tile - tile_off[d]);
    const DocSpan doc = docs[d];
    const int uoff = unit_off[d];
    const int p0 = local_tile * kTok;
    const int c = p0 / kBlock;
    const int ntok = min(kTok, doc.len - p0);
    const int p_last = p0 + ntok - 1;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int n = lane & 15, grp = lane >> 4;

    // ---- this wave's tokens and their query operands (column n = head n)
    const int head = g * kGroup + n;
    int my_p[2];
    bool tok_ok[2];
    WaveState st;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        my_p[t] = p0 + 2 * wave + t;
        tok_ok[t] = 2 * wave + t < ntok;
        const uint16_t *src =
            q + (size_t(doc.start + (tok_ok[t] ? my_p[t] : p0)) * kHeads + head) * kDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            st.qb[t][ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + 32 * ks + 8 * grp));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.acc_o[t][dt] = f32x4{};
        st.m_ref[t] = -INFINITY;
        st.l_run[t] = 0.f;
    }

    // ---- union of the tile's selected blocks (ascending, with token masks)
    const int nu = tile_union(q2k, T, topk, g, doc.start + p0, ntok, c, tid, s_id, s_first, s_mask,
                              s_ublk, s_umask, &s_nu);
    // Split the union: blocks at least kSharedMin tokens selected, and the
    // query's own block, go through the LDS ring (ascending); a block one
    // token selected is read by that token's wave straight from memory.
    if (wave == 0) {
        int base = 0;
        for (int u0 = 0; u0 < nu; u0 += 64) {
            const int u = u0 + lane;
            const bool sh = u < nu && (__popc(s_umask[u]) >= kSharedMin || s_ublk[u] == c);
            const uint64_t m = __ballot(sh);
            if (sh) {
                const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
                s_sblk[pos] = s_ublk[u];
                s_smask[pos] = s_umask[u];
            }
            base += __popcll(m);
        }
        if (lane == 0) s_ns = base;
    }
    __syncthreads();
    const int ns = s_ns;
    // ---- blocks a single token of the tile selected (never the query's own
    // block): that token's wave alone, straight from memory, one unit at a
    // time in the ring iterations where the wave has no token in the ring's
    // block, and the rest after the ring (the online softmax takes blocks in
    // any order).  The wave lists them as 2b + t, at most kMaxTopk per token.
    __shared__ int s_dlist[kTok / 2][2 * kMaxTopk];
    int nd = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (!tok_ok[t]) continue;
        const int bit = 1 << (2 * wave + t);
        for (int u0 = 0; u0 < nu; u0 += 64) {
            const int u = min(u0 + lane, nu - 1);
            const int um = s_umask[u], ub = s_ublk[u];
            const bool dir = u0 + lane < nu && (um & bit) && ub != c && __popc(um) < kSharedMin;
            const uint64_t m = __ballot(dir);
            if (dir) s_dlist[wave][nd + __popcll(m & ((1ull << lane) - 1ull))] = 2 * ub + t;
            nd += __popcll(m);
        }
    }
    const int nd_units = kUnitsPerBlock * nd;
    int di = 0;

    // 32-key units: 4 per ring block, except that the query's own block c
    // (always last when present) stops at the unit holding p_last.
    const int last_units =
        (ns > 0 && s_sblk[ns - 1] == c) ? (p_last - c * kBlock) / kAttnUnit + 1 : kUnitsPerBlock;
    const int nunits = ns > 0 ? kUnitsPerBlock * (ns - 1) + last_units : 0;

    // ---- HBM -> LDS unit copies: 16 one-KiB copies per unit.  Copy i < 8
    // fills K rows 4i..4i+3 (lane l: row 4i + l/16, slot position l%16, i.e.
    // chunk (l%16) ^ kswz(row)); copy i >= 8 fills V^T rows 16(i-8)..+15
    // (lane l: row 16(i-8) + l/4, chunk (l%4) ^ vswz(row)).  Both come from
    // the per-unit copies, whose rows past the document end are zero.
    auto issue_copy = [&](int vu, int ub, int i) {
        const int qq = vu & 3;
        uint8_t *slot = smem + (vu % kRing) * kUnitBytes;
        if (i < 8) {
            const int r = 4 * i + (lane >> 4);
            const int ch = (lane & 15) ^ kswz(r);
            const size_t unit = size_t(uoff + ub * kUnitsPerBlock + qq);
            const uint16_t *src = ku + ((unit * kKvHeads + g) * kAttnUnit + r) * kDim + 8 * ch;
            copy_to_lds(src, slot + i * 1024);
        } else {
            const int jv = i - 8;
            const int dd = 16 * jv + (lane >> 2);
            const int ch = (lane & 3) ^ vswz(dd);
            const size_t unit = size_t(uoff + ub * kUnitsPerBlock + qq);
            const uint16_t *src = vt + ((unit * kKvHeads + g) * kDim + dd) * kAttnUnit + 8 * ch;
            copy_to_lds(src, slot + kKUnitBytes + jv * 1024);
        }
    };
    // Wave w issues copies 2w and 2w+1 of every unit.
    auto issue_unit = [&](int vu) {
        const int ub = __builtin_amdgcn_readfirstlane(s_sblk[vu >> 2]);
        issue_copy(vu, ub, 2 * wave);
        issue_copy(vu, ub, 2 * wave + 1);
    };

    // Lane-constant LDS byte offsets of the operand reads.
    // K: M-tile mt row n is key 8(n/4) + 4mt + n%4, whose kswz is n.
    int k_row_off[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) k_row_off[mt] = (8 * (n >> 2) + 4 * mt + (n & 3)) * (kDim * 2);
    // V^T: d-tile dt reads row 16dt + n, chunk grp.
    const int v_off = 64 * n + 16 * (grp ^ vswz(n));

    // Block loop: union block u occupies units 4u..4u+nq-1 (nq < 4 only for
    // the query's own block).  At the barrier of block u its units have
    // landed (each wave waited for its own copies of them) and every wave is
    // done with block u-1; the ring then takes every unit up to 4u + 8, so
    // five units stream in during the compute.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): query operands are in (no copy issued yet)
    int issued = min(nunits, kRing);
    for (int vu = 0; vu < issued; ++vu) issue_unit(vu);
    for (int u = 0; u < ns || di < nd_units; ++u) {
        if (u >= ns) {  // past the ring (no more barriers): the wave's remaining units
            const int e = __builtin_amdgcn_readfirstlane(s_dlist[wave][di >> 2]);
            if (e & 1) attend_unit_global<1>(st, ku, vt, g, uoff, e >> 1, di & 3, n, grp, scale_log2);
            else attend_unit_global<0>(st, ku, vt, g, uoff, e >> 1, di & 3, n, grp, scale_log2);
            ++di;
            continue;
        }
        const int ustart = kUnitsPerBlock * u;
        const int nq = u == ns - 1 ? nunits - ustart : kUnitsPerBlock;
        wait_copies(2 * (issued - (ustart + nq)));  // copies complete in issue order
        barrier_keep_prefetch();

        const int b = __builtin_amdgcn_readfirstlane(s_sblk[u]);
        const int umask = __builtin_amdgcn_readfirstlane(s_smask[u]);
        const bool act[2] = {tok_ok[0] && ((umask >> (2 * wave)) & 1),
                             tok_ok[1] && ((umask >> (2 * wave + 1)) & 1)};
        // refill the slots of block u-1 (every wave is past it)
        for (const int ifront = min(nunits, ustart + kRing); issued < ifront; ++issued)
            issue_unit(issued);
        const int keyb = b * kBlock + 8 * grp;
        if (b == c)
            attend_block<true, true, true>(st, smem, ustart, nq, k_row_off, v_off, n, grp, keyb, act, my_p,
                                           scale_log2);
        else if (act[0] && act[1])
            attend_block<true, true, false>(st, smem, ustart, kUnitsPerBlock, k_row_off, v_off, n, grp, keyb,
                                            act, my_p, scale_log2);
        else if (act[0])
            attend_block<true, false, false>(st, smem, ustart, kUnitsPerBlock, k_row_off, v_off, n, grp,
                                             keyb, act, my_p, scale_log2);
        else if (act[1])
            attend_block<false, true, false>(st, smem, ustart, kUnitsPerBlock, k_row_off, v_off, n, grp,
                                             keyb, act, my_p, scale_log2);
        else if (di < nd_units) {  // no token in this block: one unit of the wave's own blocks
            const int e = __builtin_amdgcn_readfirstlane(s_dlist[wave][di >> 2]);
            if (e & 1) attend_unit_global<1>(st, ku, vt, g, uoff, e >> 1, di & 3, n, grp, scale_log2);
            else attend_unit_global<0>(st, ku, vt, g, uoff, e >> 1, di & 3, n, grp, scale_log2);
            ++di;
        }
    }

    // ---- epilogue: normalise and store bf16 (lane holds d = 16dt + 4grp + i)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float l_tot = row_sum4(st.l_run[t]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (lse && tok_ok[t] && grp == 0) {
            // sum_j e^(scale s_j) = 2^(m_ref * scale_log2) * l_tot
            const float mb = st.m_ref[t] == -INFINITY ? 0.f : st.m_ref[t] * scale_log2;
            lse[size_t(doc.start + my_p[t]) * kHeads + head] =
                l_tot > 0.f ? (mb + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
        }
        if (tok_ok[t]) {
            uint16_t *dst = out + (size_t(doc.start + my_p[t]) * kHeads + head) * kDim;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                bf16x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = (__bf16)(st.acc_o[t][dt][i] * inv);
                *(bf16x4 *)(dst + 16 * dt + 4 * grp) = o;
            }
        }
    }
}

// V^T per unit, then K per unit [unit][KV head][32 keys][d] (same size)
static size_t unit_elems(int T, int ndocs) {
    return (size_t(ceil_div(T, kAttnUnit)) + size_t(ndocs)) * kKvHeads * kDim * kAttnUnit;
}

size_t prefill_units_bytes(int T, int ndocs) { return 2 * unit_elems(T, ndocs) * 2; }

hipError_t launch_kv_units(const uint16_t *k, const uint16_t *v, const DocSpan *docs,
                           const int32_t *unit_off, int ndocs, int T, uint16_t *vt, hipStream_t stream) {
    const int max_units = ceil_div(T, kAttnUnit) + ndocs;  // document-aligned units (upper bound)
    hipLaunchKernelGGL(kv_units_kernel, dim3(max_units, kKvHeads), dim3(256), 0, stream, k, v, docs,
                       unit_off, ndocs, vt + unit_elems(T, ndocs), vt);
    return hipGetLastError();
}

hipError_t launch_attend_prefill(const uint16_t *q, const uint16_t *vt,
                                 const int32_t *q2k, int topk, const DocSpan *docs,
                                 const int32_t *tile_off, const int32_t *unit_off, int ndocs, int T,
                                 float scale, uint16_t *out, float *lse, hipStream_t stream) {
    const int max_tiles = ceil_div(T, kTok) + ndocs;  // document-aligned tiles (upper bound)
    const int grid = 8 * 8 * ceil_div(max_tiles, 16);  // 8 XCDs x slots
    const size_t lds = size_t(kRing) * kUnitBytes;
    hipLaunchKernelGGL(attend_prefill_kernel, dim3(grid), dim3(kThreads), lds, stream, q,
                       vt + unit_elems(T, ndocs), vt, q2k, topk, docs, tile_off, unit_off, ndocs, T,
                       scale * kLog2e, out, lse);
    return hipGetLastError();
}

}  // namespace msa
