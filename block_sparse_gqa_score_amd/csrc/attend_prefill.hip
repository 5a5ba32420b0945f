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
//   attend_prefill_kernel - workgroup = (KV head g, a tile of up to 24
//       consecutive tokens of one document inside one 128-token block, so all
//       share the query block c; a query block is cut into 6 near-equal
//       tiles); 8 waves, two per SIMD, each owning 3 token slots x 16 heads
//       (tile token i is slot i/8 of wave i%8): their Q^T operands stay in
//       VGPRs and their O^T accumulators in AGPRs.  The workgroup streams the
//       union of its tokens' selected blocks as 32-key units (K rows 8 KiB +
//       V^T rows 8 KiB) HBM -> LDS by global_load_lds_dwordx4 through a
//       9-slot ring, unit-major (unit 0 of every union block, ascending, then
//       unit 1, ...: any 9 consecutive units span 9 blocks, which most of the
//       waves need), with no workgroup barrier: every unit has an
//       LDS state word (claimed bit, count of the waves that still need it)
//       and every slot a flag, the id of the unit whose copies last landed
//       there (a 17th copy, of the id, issued after the unit's 16: a wave's
//       copies land in issue order).  Each wave walks only the units its
//       tokens need, in ring order, from a visit list built per tile.  A wave that needs a unit nobody has copied yet claims
//       it and issues its copies once every wave needing the unit 9 places
//       earlier is done with that slot; before computing a unit it claims its
//       next one the same way, so the copies land during the compute.  A unit
//       only one wave needs is claimed without a returning atomic.  A wave
//       computes a unit for those of its tokens that selected the block; the
//       K and V^T fragments it reads from LDS once serve all of them.  The
//       slowest wave can always claim its next unit, so the waits end; each
//       is also bounded by a poll limit.
//
// Per wave, token and 32-key unit (MFMA 16x16x32 bf16, key rows m, head
// columns n):
//   S^T[32 x 16] = K . Q^T       2 M-tiles x 4 k-steps; M-tile mt row i is key
//                                 8(i/4) + 4mt + i%4, so lane (n, grp) holds
//                                 keys 8grp..8grp+7 of column n in order;
//   causal mask in the tile's own units of the query block, online softmax
//   per unit in the exp2 domain with lazy rescaling (the reference max only
//   moves when it grows by more than 2^8), P^T packed to bf16 straight from
//   the accumulators,
//   O^T[128 x 16] += V^T . P^T   8 d-tiles x 1 k-step.
#include "attend_common.hpp"

namespace msa {

namespace {
constexpr int kTok = kFwdTile;                         // most tokens per workgroup
constexpr int kWaves = kFwdWaves;                      // waves per workgroup
constexpr int kTpw = kTok / kWaves;                    // token slots per wave
constexpr int kBitsPerWave = 32 / kWaves;              // a wave's field in a 32-bit token mask
constexpr int kTilesPerBlock = (kBlock + kTok - 1) / kTok;  // tiles per 128-token query block
constexpr int kThreads = 64 * kWaves;
constexpr int kUnitsPerBlock = kBlock / kAttnUnit;     // 4
constexpr int kKUnitBytes = kAttnUnit * kDim * 2;      // 8 KiB of K rows
constexpr int kVUnitBytes = kDim * kAttnUnit * 2;      // 8 KiB of V^T rows
constexpr int kUnitBytes = kKUnitBytes + kVUnitBytes;  // 16 KiB
constexpr int kRing = 9;  // LDS ring slots of one unit each (144 KiB, with the tables below < 160 KiB)
constexpr int kMaxUnion = kTok * kMaxTopk;             // distinct blocks of a tile at most
constexpr int kUnionListBytes = kMaxUnion * 8;         // (block, token mask) pairs
// Block-id window of the union's mask table (it shares the ring's LDS with
// the union list, before any copy is issued).
constexpr int kTableIds = (kRing * kUnitBytes - kUnionListBytes) / 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;  // rescale only when the max grows by > 2^8
constexpr int kMaxUnits = kUnitsPerBlock * kMaxUnion;  // ring units of a tile at most
// Unit state words in LDS: bits 0-7 count the waves that still have to read
// the unit, kClaimed marks its copy issued.  Whether the copy has landed is
// read from the ring slot's flag.
constexpr uint32_t kClaimed = 0x100u;
constexpr int kSpinLimit = 1 << 14;  // polls before a wait gives up (never reached in a correct run)

// Unit ids 0..kMaxUnits-1 in device memory: the source of the ready flags'
// copies (the flag of a ring slot holds the id of the unit whose data last
// landed there).
struct UnitIds {
    int v[kMaxUnits];
    constexpr UnitIds() : v() {
        for (int i = 0; i < kMaxUnits; ++i) v[i] = i;
    }
};
__device__ const UnitIds kUnitIds = UnitIds();

static_assert(kTpw * kWaves == kTok && kTpw <= kBitsPerWave && kTpw <= 8, "slots fit the mask fields");

// K unit in LDS: row r (key), 16-byte chunk c (d 8c..8c+7) at slot
// 16r + (c ^ kswz(r)).  The 16 lanes of an operand read hold rows
// 8a + 4mt + b (a, b < 4), whose kswz values are the 16 distinct 4a + b.
__device__ __forceinline__ int kswz(int r) { return (((r >> 3) & 3) << 2) | (r & 3); }
// V^T unit in LDS: row d, chunk c (keys 8c..8c+7) at slot 4d + (c ^ vswz(d));
// 16 consecutive rows at one chunk cover all 16 chunk positions of 256 B.
__device__ __forceinline__ int vswz(int d) { return (d >> 2) & 3; }

// Per-wave state: query operands and running softmax of the wave's 8
// tokens (column n of each is head n of the KV group).
struct WaveState {
    bf16x8 qb[kTpw][4];
    f32x4 acc_o[kTpw][8];
    float m_ref[kTpw];  // raw-score reference of the exponentials
    float l_run[kTpw];
};

// S^T of one unit for token t: K fragments ka (shared by the wave's tokens).
template <int t>
__device__ __forceinline__ void unit_scores(const WaveState &st, const bf16x8 (&ka)[4][2], f32x4 (&s)[2]) {
    s[0] = f32x4{};
    s[1] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s[mt] = mfma_16x16x32(ka[ks][mt], st.qb[t][ks], s[mt]);
}

// Online-softmax step of token t over one unit's 32 keys (this lane: keys
// e = 0..7 at unit offset 8grp + e, sacc[e/4][e%4]).  With `mask` (wave-
// uniform: the tile's own unit of the query block) keys past the token drop
// (block-relative key offset kofs + e > pos).  Returns P^T packed as the PV
// operand.
template <int t>
__device__ __forceinline__ bf16x8 unit_softmax(WaveState &st, const f32x4 (&sacc)[2], bool mask, int kofs,
                                               int pos, float scale_log2) {
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = sacc[e >> 2][e & 3];
    if (mask) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = kofs + e <= pos ? sv[e] : -INFINITY;
    }
    float mloc = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mloc = fmaxf(mloc, sv[e]);
    mloc = row_max4(mloc);
    // lazy reference: move it (and rescale) only on a large increase
    const bool grow = mloc > st.m_ref[t] &&
                      (st.m_ref[t] == -INFINITY || (mloc - st.m_ref[t]) * scale_log2 > kLazyLog2);
    if (__ballot(grow)) {
        const float m_new = grow ? mloc : st.m_ref[t];
        const float alpha =
            st.m_ref[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m_ref[t] - m_new) * scale_log2);
        st.l_run[t] *= alpha;
        // The accumulators live in AGPRs; pinning the value to AGPRs on both
        // sides of the multiply keeps the register allocator from moving the
        // whole O^T state to VGPRs around this rarely taken path.
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            f32x4 x = st.acc_o[t][dt];
            asm volatile("" : "+a"(x));
            x *= alpha;
            asm volatile("" : "+a"(x));
            st.acc_o[t][dt] = x;
        }
        st.m_ref[t] = m_new;
    }
    const float mb = st.m_ref[t] == -INFINITY ? 0.f : st.m_ref[t] * scale_log2;
    float psum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float pv = __builtin_amdgcn_exp2f(sv[e] * scale_log2 - mb);
        psum += pv;
        pb[e] = (__bf16)pv;
    }
    st.l_run[t] += psum;
    return pb;
}

// Scores and softmax of one unit for slot t, when the slot's token selected
// the block (act bit t); P^T goes to pb[t].
template <int t>
__device__ __forceinline__ void token_unit(WaveState &st, const bf16x8 (&ka)[4][2], bf16x8 (&pb)[kTpw],
                                           uint32_t act, bool mask, int kofs, int pos0, float scale_log2) {
    if constexpr (t < kTpw) {
        if (!((act >> t) & 1u)) return;
        f32x4 s[2];
        unit_scores<t>(st, ka, s);
        pb[t] = unit_softmax<t>(st, s, mask, kofs, pos0 + kWaves * t, scale_log2);
    }
}

// One ring unit for the wave's active tokens `act` (bit t = slot t of the
// wave, wave-uniform): K fragments read once from LDS, scores and softmax
// token by token, then V^T fragments read once and O^T += V^T P^T per token.
// mask: the tile's own unit of the query block (keys past a token drop).
__device__ __forceinline__ void ring_unit(WaveState &st, const uint8_t *Ku, uint32_t act, const int (&k_row_off)[2],
                                          int v_off, int n, int grp, bool mask, int kofs, int pos0,
                                          float scale_log2) {
    bf16x8 pb[kTpw];
    {
        bf16x8 ka[4][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                ka[ks][mt] = __builtin_bit_cast(bf16x8,
                                                *(const u32x4 *)(Ku + k_row_off[mt] + (((4 * ks + grp) ^ n) << 4)));
        token_unit<0>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
        token_unit<1>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
        token_unit<2>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
        token_unit<3>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
        token_unit<4>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
        token_unit<5>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
        token_unit<6>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
        token_unit<7>(st, ka, pb, act, mask, kofs, pos0, scale_log2);
    }
    const uint8_t *Vu = Ku + kKUnitBytes;
    bf16x8 va[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Vu + 1024 * dt + v_off));
#pragma unroll
    for (int t = 0; t < kTpw; ++t) {
        if (!((act >> t) & 1u)) continue;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.acc_o[t][dt] = mfma_16x16x32(va[dt], pb[t], st.acc_o[t][dt]);
    }
}

// Exclusive prefix sum over the workgroup of one int per thread; the total
// goes to *total.  s_w: kWaves ints of LDS.  Ends with a barrier.
__device__ __forceinline__ int block_exclusive_scan(int v, int tid, int *s_w, int *total) {
    const int lane = tid & 63, wave = tid >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_w[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? s_w[w] : 0;
        tot += s_w[w];
    }
    *total = tot;
    __syncthreads();
    return before + x - v;
}

// Union of the selected blocks of a tile of ntok <= 28 consecutive tokens
// (first token tok0, all in query block c of one document) for KV head g:
// ublk[0..nu) ascending, umask[u] bit kBitsPerWave (i % kWaves) + i / kWaves
// set when tile token i selected ublk[u] (token i belongs to wave
// i % kWaves, slot i / kWaves).
// Ids outside 0..c and -1 are dropped; repeats count once.  The 32-bit
// masks are gathered in an LDS table indexed by block id (windows of
// kTableIds ids), then compacted in ascending order.  Called by every
// thread of the workgroup; returns nu to all of them.
__device__ __forceinline__ int tile_union32(const int32_t *__restrict__ q2k, int T, int topk, int g, int tok0,
                                            int ntok, int c, int tid, uint32_t *table, int *ublk,
                                            uint32_t *umask, int *s_w) {
    int nu = 0;
    for (int b0 = 0; b0 <= c; b0 += kTableIds) {
        const int W = min(kTableIds, c + 1 - b0);
        for (int i = tid; i < W; i += kThreads) table[i] = 0u;
        __syncthreads();
        for (int e = tid; e < ntok * topk; e += kThreads) {  // consecutive entries: coalesced
            const int tok = e / topk;
            const int id = q2k[(size_t(g) * T + tok0) * topk + e];
            if (id >= b0 && id < b0 + W)
                atomicOr(&table[id - b0], 1u << (kBitsPerWave * (tok % kWaves) + tok / kWaves));
        }
        __syncthreads();
        const int per = (W + kThreads - 1) / kThreads;  // thread tid: ids [tid*per, tid*per+per)
        int cnt = 0;
        for (int i = 0; i < per; ++i) {
            const int idx = tid * per + i;
            cnt += (idx < W && table[idx] != 0u) ? 1 : 0;
        }
        int tot;
        int pos = nu + block_exclusive_scan(cnt, tid, s_w, &tot);
        for (int i = 0; i < per; ++i) {
            const int idx = tid * per + i;
            const uint32_t m = idx < W ? table[idx] : 0u;
            if (m != 0u) {
                ublk[pos] = b0 + idx;
                umask[pos] = m;
                ++pos;
            }
        }
        nu += tot;
        __syncthreads();
    }
    return nu;
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
    __shared__ int s_sblk[kMaxUnion];             // the ring's blocks (the tile's union), ascending
    __shared__ uint32_t s_smask[kMaxUnion];       // their token masks
    __shared__ uint32_t s_unit[kMaxUnits];        // per ring unit: state bits | waves still to read it
    __shared__ int s_wlist[kWaves][kTpw * kMaxTopk];  // per wave: the ring blocks it needs, ascending
    __shared__ int s_w[kWaves];
    __shared__ int s_flag[kRing][64];             // per ring slot: id of the unit that has landed there

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; XCD x
    // serves KV head x/2 and alternate groups of 5 tiles (one 128-token query
    // block) of that head, longest first, so the tiles sharing a query block
    // share one L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, xslot = bid >> 3;
    const int g = xcd >> 1;
    const int tile = 2 * kTilesPerBlock * (xslot / kTilesPerBlock) + kTilesPerBlock * (xcd & 1) +
                     xslot % kTilesPerBlock;
    if (tile >= tile_off[ndocs]) return;
    const int d = prefix_doc(tile_off, ndocs, tile);
    const int nt_doc = tile_off[d + 1] - tile_off[d];
    const int local_tile = nt_doc - 1 - (tile - tile_off[d]);
    const DocSpan doc = docs[d];
    const int uoff = unit_off[d];
    // tile i of query block c: positions [c*128 + Lb*i/nt, c*128 + Lb*(i+1)/nt)
    // of the block's Lb tokens cut into nt near-equal tiles
    const int nb_full = doc.len / kBlock;
    int c, ti, nt, Lb;
    if (local_tile < kTilesPerBlock * nb_full) {
        c = local_tile / kTilesPerBlock;
        ti = local_tile % kTilesPerBlock;
        Lb = kBlock;
        nt = kTilesPerBlock;
    } else {
        c = nb_full;
        ti = local_tile - kTilesPerBlock * nb_full;
        Lb = doc.len - kBlock * c;
        nt = (Lb + kTok - 1) / kTok;
    }
    const int r0 = Lb * ti / nt;                   // block-relative first position
    const int p0 = c * kBlock + r0;
    const int ntok = Lb * (ti + 1) / nt - r0;      // 1..28
    const int q_lo = r0 / kAttnUnit;               // own-block units q >= q_lo take the causal mask
    const int q_hi = (r0 + ntok - 1) / kAttnUnit;  // the own block stops at unit q_hi

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int n = lane & 15, grp = lane >> 4;
    // slot t of this wave is tile token kWaves t + wave, at position
    // p0 + kWaves t + wave
    const int pos0 = p0 + wave;

    // ---- this wave's tokens and their query operands (column n = head n)
    const int head = g * kGroup + n;
    WaveState st;
#pragma unroll
    for (int t = 0; t < kTpw; ++t) {
        const int p = kWaves * t + wave < ntok ? pos0 + kWaves * t : p0;
        const uint16_t *src = q + (size_t(doc.start + p) * kHeads + head) * kDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            st.qb[t][ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + 32 * ks + 8 * grp));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) st.acc_o[t][dt] = f32x4{};
        st.m_ref[t] = -INFINITY;
        st.l_run[t] = 0.f;
    }

    // ---- union of the tile's selected blocks (ascending, with token masks);
    // the table and the list live in the ring's LDS until the walk starts
    int *ublk = (int *)(smem + kRing * kUnitBytes - kUnionListBytes);
    uint32_t *umask = (uint32_t *)(ublk + kMaxUnion);
    const int nu = tile_union32(q2k, T, topk, g, doc.start + p0, ntok, c, tid, (uint32_t *)smem, ublk, umask, s_w);
    // The ring holds every union block, ascending; the query's own block c is
    // last when present and stops at the unit of the tile's last token.
    for (int u = tid; u < nu; u += kThreads) {
        s_sblk[u] = ublk[u];
        s_smask[u] = umask[u];
    }
    const int ns = nu;
    const int last_units = (ns > 0 && ublk[ns - 1] == c) ? q_hi + 1 : kUnitsPerBlock;
    // unit counts: the waves whose tokens selected the unit's block
    // Ring order: unit-major, unit q of every union block, then unit q + 1.
    // A window of kRing consecutive units then spans kRing blocks, needed by
    // most of the waves, instead of the two or three blocks of block-major
    // order, which only some of them need (in block-major order, waiting for
    // a slot took 40% of the waves' time).  Only existing units are numbered (the diagonal block,
    // last, stops at unit last_units - 1: passes q < last_units hold ns units,
    // later ones ns - 1), so a slot's previous occupant is always the unit
    // kRing places earlier.
    const int nunits = kUnitsPerBlock * (ns - 1) + last_units;
    auto unit_id = [&](int q, int bi) { return q * ns - max(0, q - last_units) + bi; };
    auto unit_block = [&](int u) {  // the unit's union block index
        const int u1 = u - last_units * ns;
        return u1 < 0 ? u % ns : u1 % max(ns - 1, 1);
    };
    for (int u = tid; u < nunits; u += kThreads) {
        const int bi = unit_block(u);
        const uint32_t m = umask[bi];
        int nw = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) nw += ((m >> (kBitsPerWave * w)) & ((1u << kBitsPerWave) - 1u)) ? 1 : 0;
        s_unit[u] = uint32_t(nw);
    }
    // each wave lists the ring blocks its tokens selected, ascending
    int nwb = 0;
    {
        const uint32_t wbits = ((1u << kBitsPerWave) - 1u) << (kBitsPerWave * wave);
        for (int u0 = 0; u0 < nu; u0 += 64) {
            const int u = min(u0 + lane, nu - 1);
            const bool mine = u0 + lane < nu && (umask[u] & wbits);
            const uint64_t m = __ballot(mine);
            if (mine) s_wlist[wave][nwb + __popcll(m & ((1ull << lane) - 1ull))] = u;
            nwb += __popcll(m);
        }
    }
    for (int i = tid; i < kRing * 64; i += kThreads) (&s_flag[0][0])[i] = -1;
    __syncthreads();  // lists, counts and flags are set; the union's LDS is free for the ring

    // Lane-constant LDS byte offsets of the operand reads.
    // K: M-tile mt row n is key 8(n/4) + 4mt + n%4, whose kswz is n.
    int k_row_off[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) k_row_off[mt] = (8 * (n >> 2) + 4 * mt + (n & 3)) * (kDim * 2);
    // V^T: d-tile dt reads row 16dt + n, chunk grp.
    const int v_off = 64 * n + 16 * (grp ^ vswz(n));
    const int tok_ok = (ntok - wave + kWaves - 1) / kWaves;  // slots t < tok_ok of this wave hold a token
    const uint32_t ok_mask = (1u << tok_ok) - 1u;
    // The wave's list in one VGPR, entry i in lane i (read back with
    // readlane): the wave's slots that selected the block (bits 0-2), its
    // ring block index (bits 3-11) and its id (bits 12-31).
    static_assert(kTpw <= 3 && kMaxUnion <= 512, "list entry fields");
    uint32_t wl = 0u;
    if (lane < nwb) {
        const int bi = s_wlist[wave][lane];
        wl = ((s_smask[bi] >> (kBitsPerWave * wave)) & ok_mask) | (uint32_t(bi) << 3) | (uint32_t(s_sblk[bi]) << 12);
    }

    // ---- HBM -> LDS copy of ring unit u (16 one-KiB copies, all issued by
    // the wave that claimed it) into slot u % kRing, copy i to slot byte
    // 1024 i.  Copy i < 8 fills K rows 4i..4i+3 (lane l: row 4i + l/16,
    // slot position l%16, i.e. chunk (l%16) ^ kswz(row)); copy i >= 8 fills
    // V^T rows 16(i-8)..+15 (lane l: row 16(i-8) + l/4, chunk
    // (l%4) ^ vswz(row)).  Both come from the per-unit copies (8 KiB per
    // unit and head in either), whose rows past the document end are zero.
    // (ub: the unit's block id, q: its 32-key unit within the block, both
    // known to the caller)
    auto issue_unit = [&](int u, int ub, int q) {
        const size_t unit = size_t(uoff + ub * kUnitsPerBlock + q) * kKvHeads + g;
        const uint16_t *ksrc = ku + unit * (kAttnUnit * kDim);
        const uint16_t *vsrc = vt + unit * (kAttnUnit * kDim);
        uint8_t *slot = smem + (u % kRing) * kUnitBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + (lane >> 4);
            copy_to_lds_s(ksrc, uint32_t(2 * (r * kDim + 8 * ((lane & 15) ^ kswz(r)))), slot + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int dd = 16 * i + (lane >> 2);
            copy_to_lds_s(vsrc, uint32_t(2 * (dd * kAttnUnit + 8 * ((lane & 3) ^ vswz(dd)))), slot + kKUnitBytes + i * 1024);
        }
        // Copies land in issue order: once the flag holds u, the data has landed.
        const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)&s_flag[u % kRing][0]);
        asm volatile("global_load_lds_dword %0, off" ::"v"(&kUnitIds.v[u]), "{m0}"(m0) : "memory");
    };
    // Unit state, read by every lane (LDS broadcast); changed by lane 0.
    auto unit_word = [&](int u) {
        return __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&s_unit[u], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
    };
    // Slot u % kRing is free for unit u once every wave needing unit u - kRing is done with it.
    auto fillable = [&](int u) { return u < kRing || (unit_word(u - kRing) & 0xFFu) == 0u; };
    auto try_claim = [&](int u) {
        uint32_t old = kClaimed;
        if (lane == 0) old = __hip_atomic_fetch_or(&s_unit[u], kClaimed, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        return (__builtin_amdgcn_readfirstlane(old) & kClaimed) == 0u;
    };
    auto landed = [&](int u) {
        return __builtin_amdgcn_readfirstlane(
                   __hip_atomic_load(&s_flag[u % kRing][lane], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) == u;
    };
    // Wait until unit u has landed; claim and copy it when nobody has and its
    // slot is free.  Every wait is bounded (kSpinLimit polls).
    auto acquire = [&](int u, int ub, int q) {
        for (int spin = 0; spin < kSpinLimit; ++spin) {
            if (landed(u)) return;
            const uint32_t wd = unit_word(u);
            if (!(wd & kClaimed) && fillable(u) && try_claim(u)) issue_unit(u, ub, q);
            __builtin_amdgcn_s_sleep(1);
        }
    };

    // ---- the wave's walk over its needed units, in ring order.  Before
    // computing a unit it claims the next one it needs, when that unit's slot
    // is free, and issues its copies, which land during the compute.
    // One visit: unit u (unit qq of list entry e's block) computed, with the
    // next unit v (vq of block vub) claimed ahead; v = -1: none.
    auto visit = [&](int u, uint32_t e, int qq, int v, int vub, int vq) {
        // keep every O^T accumulator in AGPRs across the walk (the register
        // allocator would otherwise carry some of them in VGPRs, which the
        // query operands and the working set need)
#pragma unroll
        for (int t = 0; t < kTpw; ++t)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) asm volatile("" : "+a"(st.acc_o[t][dt]));
        const uint32_t act = e & 7u;
        const bool own = int(e >> 12) == c;
        // One LDS round trip: u's flag, v's state and the state of the unit
        // before v in its slot (v = -1: none; below kRing: the slot is new).
        const int vs = v >= 0 ? v : u;
        const int vp = v >= kRing ? v - kRing : u;
        const int fl = __hip_atomic_load(&s_flag[u % kRing][lane], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t wv = __hip_atomic_load(&s_unit[vs], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t wp = __hip_atomic_load(&s_unit[vp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(fl) != u) acquire(u, int(e >> 12), qq);
        // claim v ahead when its slot is free: a unit that only this wave
        // needs (count 1, nobody has read it) is marked without a returning
        // atomic; a shared one goes to whichever wave claims it first
        const uint32_t wvs = __builtin_amdgcn_readfirstlane(wv);
        if (v >= 0 && !(wvs & kClaimed) && (v < kRing || (__builtin_amdgcn_readfirstlane(wp) & 0xFFu) == 0u)) {
            if ((wvs & 0xFFu) == 1u) {
                if (lane == 0) __hip_atomic_fetch_or(&s_unit[v], kClaimed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                issue_unit(v, vub, vq);
            } else if (try_claim(v)) {
                issue_unit(v, vub, vq);
            }
        }
        const uint8_t *Ku = smem + (u % kRing) * kUnitBytes;
        // the tile's own units of the query block: keys past each token drop
        if (act)
            ring_unit(st, Ku, act, k_row_off, v_off, n, grp, own && qq >= q_lo, kAttnUnit * qq + 8 * grp,
                      pos0 - c * kBlock, scale_log2);
        // done reading unit u: its slot may be refilled once every wave needing it is done
        if (lane == 0) __hip_atomic_fetch_sub(&s_unit[u], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // The wave's visits in ring order (ascending unit number), packed
    // u | k << 11 | q << 17 (unit q of list entry k's block), visit i in lane
    // i % 64 of vis0, vis1, vis2 (i / 64).  Pass q holds every entry except a
    // diagonal last one past its last unit, so (k, q) is visit
    // q nwb - max(0, q - lw) + k.  Written through LDS scratch at the start of
    // the ring (free until the walk), one KiB per wave.
    static_assert(kTpw * kMaxTopk * kUnitsPerBlock <= 192 && kUnitsPerBlock * kMaxUnion <= 2048, "visit fields");
    auto entry = [&](int k) { return __builtin_amdgcn_readlane(wl, k); };
    const int lw = nwb > 0 && int((entry(nwb - 1) >> 3) & 511u) == ns - 1 ? last_units : kUnitsPerBlock;
    const int nvis = nwb > 0 ? kUnitsPerBlock * (nwb - 1) + lw : 0;
    uint32_t vis0, vis1, vis2;  // three named registers (an array indexed at run time would go to scratch)
    {
        uint32_t *svis = (uint32_t *)(smem + wave * 1024);
        if (lane < nwb) {
            const int bi = (wl >> 3) & 511u;
            const int nq = lane == nwb - 1 ? lw : kUnitsPerBlock;
            for (int q = 0; q < nq; ++q) {
                const int i = q * nwb - max(0, q - lw) + lane;
                svis[i] = uint32_t(unit_id(q, bi)) | (uint32_t(lane) << 11) | (uint32_t(q) << 17);
            }
        }
        __builtin_amdgcn_wave_barrier();
        vis0 = svis[lane];
        vis1 = svis[64 + lane];
        vis2 = svis[128 + lane];
    }
    __syncthreads();  // every wave has its visits before any copy lands in the ring
    auto vis_at = [&](int i) {
        const uint32_t r = i < 64 ? vis0 : i < 128 ? vis1 : vis2;
        return __builtin_amdgcn_readlane(r, i & 63);
    };
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): query operands are in (no copy issued yet)
    for (int i = 0; i < nvis; ++i) {
        const uint32_t x = vis_at(i);
        int v = -1, vub = 0, vq = 0;
        if (i + 1 < nvis) {
            const uint32_t y = vis_at(i + 1);
            v = int(y & 2047u);
            vub = int(entry((y >> 11) & 63u) >> 12);
            vq = int(y >> 17);
        }
        visit(int(x & 2047u), entry((x >> 11) & 63u), int(x >> 17), v, vub, vq);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every copy this wave issued has landed

    // ---- epilogue: normalise and store bf16 (lane holds d = 16dt + 4grp + i)
#pragma unroll
    for (int t = 0; t < kTpw; ++t) {
        const float l_tot = row_sum4(st.l_run[t]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const bool ok = t < tok_ok;
        const size_t row = size_t(doc.start + pos0 + kWaves * t) * kHeads + head;
        if (lse && ok && grp == 0) {
            // sum_j e^(scale s_j) = 2^(m_ref * scale_log2) * l_tot
            const float mb = st.m_ref[t] == -INFINITY ? 0.f : st.m_ref[t] * scale_log2;
            lse[row] = l_tot > 0.f ? (mb + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
        }
        if (ok) {
            uint16_t *dst = out + row * kDim;
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
    // document-aligned tiles (upper bound): 5 per 128-token query block
    const int max_tiles = kTilesPerBlock * (ceil_div(T, kBlock) + ndocs);
    // 8 XCDs x slots; an XCD pair serves 2 groups of 5 tiles per 5 slots
    const int grid = 8 * kTilesPerBlock * ceil_div(max_tiles, 2 * kTilesPerBlock);
    const size_t lds = size_t(kRing) * kUnitBytes;
    static const bool fits = lds_fits(reinterpret_cast<const void *>(attend_prefill_kernel), lds);
    if (!fits) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attend_prefill_kernel, dim3(grid), dim3(kThreads), lds, stream, q,
                       vt + unit_elems(T, ndocs), vt, q2k, topk, docs, tile_off, unit_off, ndocs, T,
                       scale * kLog2e, out, lse);
    return hipGetLastError();
}

}  // namespace msa
