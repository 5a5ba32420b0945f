// Sparse GQA attention over the selected blocks, prefill on packed documents.
//
// Method (NeMo AutoModel minimax_m3_vl.msa, sparse_attention; TensorRT-LLM
// "MiniMaxM3SparseAttentionConfig", class description, step two): query
// head h of token t attends, with softmax over scale * q.k, to the keys of
// t's document at or before t whose document-local 128-key block appears in
// q2k row (h/16, t).
//
// Workgroup = (KV head g, 16 consecutive tokens of one document inside one
// 128-token block, so all share the query block c); 8 waves, each owning
// 2 tokens x 16 heads = 32 query columns.  The workgroup walks the UNION of
// its tokens' selected blocks in ascending order.  Each block's K and V
// (128 x 128 bf16 each, natural [key][d] layout, 16-byte chunks XOR-swizzled
// per row) are copied HBM -> LDS by global_load_lds_dwordx4 into a 2-stage
// ring: block u+1 streams in while block u is computed, with no register
// staging.  A wave whose two tokens did not select the block skips it.
//
// Per wave and block (key rows m, query columns n):
//   S^T[128 x 32] = K . Q^T   4 M-tiles x 8 k-steps of MFMA 32x32x16; the K
//                              operand is a 16-byte LDS read per lane.
//   mask (selected by the column's token; key <= query in the own block),
//   online softmax in the exp2 domain with lazy rescaling (the reference max
//   only moves when it grows by more than 2^8), P^T packed to bf16 from the
//   S^T accumulators,
//   O^T[128 x 32] += V^T . P^T   4 d-tiles x 8 k-steps of MFMA 32x32x16; the
//                              V^T operand comes from two ds_read_b64_tr_b16.
// The S^T accumulator gives lane (n, hb) the keys 8*(r/4) + 4*hb + r%4 of
// each 32-key tile, so PV step s consumes registers 8*(s%2)..8*(s%2)+7 of
// tile s/2: keys 16s + 4hb + e and 16s + 8 + 4hb + e (e < 4), exactly the
// two 4-row groups each transposing read returns for lane (d, hb).
#include "msa_internal.hpp"

namespace msa {

namespace {
constexpr int kTok = kAttnTile;        // 16 tokens per workgroup
constexpr int kWaves = kTok / 2;       // 8 waves
constexpr int kThreads = 64 * kWaves;  // 512
constexpr int kRowBytes = kDim * 2;    // 256
constexpr int kTileBytes = kBlock * kRowBytes;  // 32 KiB (K or V block)
constexpr int kStageBytes = 2 * kTileBytes;     // K + V
constexpr int kStages = 2;
constexpr int kLoadsPerWave = kStageBytes / 1024 / kWaves;  // 1 KiB per wave instruction
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;  // rescale only when the max grows by > 2^8

// Chunk position of 16-byte chunk c in row r is c ^ swz(r): 16 consecutive
// rows hit 16 distinct positions (K operand reads), and 8 consecutive rows x
// 4 consecutive chunks hit every position exactly twice (V^T reads).
__device__ __forceinline__ int swz(int r) {
    return (((r >> 1) & 3) << 2) | ((r & 1) << 1) | ((r >> 3) & 1);
}

__device__ __forceinline__ int tile_doc(const int32_t *off, int ndocs, int t) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Workgroup barrier that drains this wave's LDS operations but leaves its
// global->LDS prefetch in flight (a plain __syncthreads would also wait for
// every outstanding vector-memory operation).  Callers wait for the block
// they are about to read with an explicit vmcnt first.
__device__ __forceinline__ void barrier_keep_prefetch() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ i16x4 ds_read_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}
}  // namespace

__global__ __launch_bounds__(kThreads) void attend_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ q2k, int topk, const DocSpan *__restrict__ docs,
    const int32_t *__restrict__ tile_off, int ndocs, int T, float scale_log2,
    uint16_t *__restrict__ out) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr int kEntries = kTok * kMaxTopk;  // 256 (token, slot) pairs
    __shared__ int s_id[kEntries];
    __shared__ int s_first[kEntries];
    __shared__ int s_mask[kEntries];
    __shared__ int s_ublk[kEntries];
    __shared__ int s_umask[kEntries];
    __shared__ int s_nu;

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; XCD x
    // serves KV head x/2 and alternate groups of 8 tiles (one 128-token query
    // block) of that head, longest first, so the tiles sharing a query block
    // share one L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, xslot = bid >> 3;
    const int g = xcd >> 1;
    const int tile = 16 * (xslot >> 3) + 8 * (xcd & 1) + (xslot & 7);
    if (tile >= tile_off[ndocs]) return;
    const int d = tile_doc(tile_off, ndocs, tile);
    const int nt_doc = tile_off[d + 1] - tile_off[d];
    const int local_tile = nt_doc - 1 - (tile - tile_off[d]);
    const DocSpan doc = docs[d];
    const int p0 = local_tile * kTok;
    const int c = p0 / kBlock;
    const int ntok = min(kTok, doc.len - p0);
    const int p_last = p0 + ntok - 1;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int n = lane & 31, hb = lane >> 5;

    // ---- union of the tile's selected blocks (ascending, with token masks)
    if (tid == 0) s_nu = 0;
    if (tid < kEntries) {
        const int tok = tid >> 4, sl = tid & 15;
        int id = -1;
        if (tok < ntok && sl < topk) id = q2k[(size_t(g) * T + doc.start + p0 + tok) * topk + sl];
        s_id[tid] = (id >= 0 && id <= c) ? id : -1;
    }
    __syncthreads();
    if (tid < kEntries) {
        const int my = s_id[tid];
        int first = my >= 0, mask = 0;
        for (int j = 0; j < kEntries; ++j) {
            if (s_id[j] == my) {
                mask |= 1 << (j >> 4);
                if (j < tid) first = 0;
            }
        }
        s_first[tid] = first;
        s_mask[tid] = mask;
    }
    __syncthreads();
    if (tid < kEntries && s_first[tid]) {
        const int my = s_id[tid];
        int pos = 0;
        for (int j = 0; j < kEntries; ++j) pos += (s_first[j] && s_id[j] < my);
        s_ublk[pos] = my;
        s_umask[pos] = s_mask[tid];
        atomicAdd(&s_nu, 1);
    }
    __syncthreads();
    const int nu = s_nu;

    // ---- this wave's query operand: column n = (token 2*wave + n/16, head n%16)
    const int my_tok = 2 * wave + (n >> 4);
    const int my_p = p0 + my_tok;
    const bool tok_ok = my_tok < ntok;
    const int head = g * kGroup + (n & 15);
    bf16x8 qb[8];
    {
        const uint16_t *src = q + (size_t(doc.start + (tok_ok ? my_p : p0)) * kHeads + head) * kDim;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qb[ks] = tok_ok ? __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + 16 * ks + 8 * hb))
                            : bf16x8{};
    }

    // ---- HBM -> LDS block copy: 64 one-KiB instructions per block (K then V),
    // kLoadsPerWave per wave.  Instruction j' fills rows 4j'..4j'+3 of its tile;
    // lane l writes position l%16 of row 4j' + l/16, i.e. chunk (l%16)^swz(row).
    // Rows past the last query of the tile are never attended: they re-read
    // row p_last so that no load leaves the document.
    auto issue_block = [&](int b, int stage) {
        uint8_t *base = smem + stage * kStageBytes;
#pragma unroll
        for (int j = 0; j < kLoadsPerWave; ++j) {
            const int id = kLoadsPerWave * wave + j;  // 0..63
            const int part = id >> 5, row4 = id & 31;
            const int r = 4 * row4 + (lane >> 4);
            const int chunk = (lane & 15) ^ swz(r);
            const int kp = min(b * kBlock + r, p_last);
            const uint16_t *src = (part ? v : k) +
                                  (size_t(doc.start + kp) * kKvHeads + g) * kDim + 8 * chunk;
            __builtin_amdgcn_global_load_lds((const void *)src,
                                             (lds_void *)(base + part * kTileBytes + row4 * 1024),
                                             16, 0, 0);
        }
    };

    f32x16 acc_o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc_o[dt] = f32x16{};
    float m_ref = -INFINITY;  // raw-score reference of the exponentials
    float l_run = 0.f;

    // Lane-constant LDS byte offsets; the row parts that vary with the
    // unrolled loop indices (32mt, 64hf rows; 16s rows) are compile-time
    // immediates because swz() only depends on a row's low 4 bits.
    int k_off[8];                  // K operand: row n, chunk 2ks+hb
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) k_off[ks] = n * kRowBytes + (((2 * ks + hb) ^ swz(n)) << 4);
    int v_off[4][2];               // V^T operand: row 4*(G/2) + gi/4 (+8 h2), column 32dt + ...
    {
        const int G = lane >> 4, gi = lane & 15;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int row = 8 * h2 + 4 * (G >> 1) + (gi >> 2);
                const int col = 32 * dt + 16 * (G & 1) + 4 * (gi & 3);
                v_off[dt][h2] = row * kRowBytes + ((((col >> 3) ^ swz(row))) << 4) + ((col & 7) << 1);
            }
    }

    if (nu > 0) issue_block(s_ublk[0], 0);
    for (int u = 0; u < nu; ++u) {
        if (u + 1 < nu) {
            issue_block(s_ublk[u + 1], (u + 1) & 1);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerWave) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        barrier_keep_prefetch();  // block u is in LDS for every wave

        const int b = s_ublk[u];
        const int umask = s_umask[u];
        const uint8_t *Kt = smem + (u & 1) * kStageBytes;
        const uint8_t *Vt = Kt + kTileBytes;
        if ((umask >> (2 * wave)) & 3) {
            const bool sel = tok_ok && ((umask >> my_tok) & 1);
            // two 64-key halves, each a full S / softmax / PV round
#pragma unroll 1
            for (int hf = 0; hf < 2; ++hf) {
                const uint8_t *Kh = Kt + 64 * hf * kRowBytes;
                const uint8_t *Vh = Vt + 64 * hf * kRowBytes;
                f32x16 acc_s[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) acc_s[mt] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    bf16x8 a[2];
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
                        a[mt] = __builtin_bit_cast(
                            bf16x8, *(const u32x4 *)(Kh + 32 * mt * kRowBytes + k_off[ks]));
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) acc_s[mt] = mfma_32x32x16(a[mt], qb[ks], acc_s[mt]);
                }

                // Column mask (token did not select b) goes into the exp2
                // offset; the per-key causal mask is only needed in the
                // query's own block.
                float mloc = -INFINITY;
                if (b == c) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kp = b * kBlock + 64 * hf + 32 * mt + 8 * (r >> 2) + 4 * hb + (r & 3);
                            const float sv = kp <= my_p ? acc_s[mt][r] : -INFINITY;
                            acc_s[mt][r] = sv;
                            mloc = fmaxf(mloc, sv);
                        }
                } else {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, acc_s[mt][r]);
                }
                mloc = sel ? mloc : -INFINITY;
                mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
                // lazy reference: move it (and rescale) only on a large increase
                const bool grow = mloc > m_ref &&
                                  (m_ref == -INFINITY || (mloc - m_ref) * scale_log2 > kLazyLog2);
                if (__ballot(grow)) {
                    const float m_new = grow ? mloc : m_ref;
                    const float alpha = m_ref == -INFINITY
                                            ? 0.f
                                            : __builtin_amdgcn_exp2f((m_ref - m_new) * scale_log2);
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) acc_o[dt] *= alpha;
                    m_ref = m_new;
                }
                // unselected columns: offset +inf makes every exponential 0
                const float mb = !sel ? INFINITY : (m_ref == -INFINITY ? 0.f : m_ref * scale_log2);
                float psum = 0.f;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float pv = __builtin_amdgcn_exp2f(acc_s[mt][r] * scale_log2 - mb);
                        acc_s[mt][r] = pv;
                        psum += pv;
                    }
                l_run += psum;

#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {  // 16-key PV steps of this half
                    bf16x8 pb;
#pragma unroll
                    for (int i = 0; i < 8; ++i) pb[i] = (__bf16)acc_s[s4 >> 1][8 * (s4 & 1) + i];
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        i16x4 t[2];
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
                            t[h2] = ds_read_tr16(Vh + 16 * s4 * kRowBytes + v_off[dt][h2]);
                        const i16x8 ab = {t[0][0], t[0][1], t[0][2], t[0][3],
                                          t[1][0], t[1][1], t[1][2], t[1][3]};
                        acc_o[dt] = mfma_32x32x16(__builtin_bit_cast(bf16x8, ab), pb, acc_o[dt]);
                    }
                }
            }
        }
        barrier_keep_prefetch();  // stage u&1 is refilled by the next iteration's prefetch
    }

    // ---- epilogue: normalise and store bf16
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (tok_ok) {
        uint16_t *dst = out + (size_t(doc.start + my_p) * kHeads + head) * kDim;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * dt + 8 * r4 + 4 * hb;
                bf16x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc_o[dt][4 * r4 + i] * inv);
                *(bf16x4 *)(dst + d0) = o;
            }
    }
}

hipError_t launch_attend_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const int32_t *q2k, int topk, const DocSpan *docs,
                                 const int32_t *tile_off, int ndocs, int T, int max_seqlen,
                                 float scale, uint16_t *out, hipStream_t stream) {
    (void)max_seqlen;
    const int max_tiles = ceil_div(T, kTok) + ndocs;  // document-aligned tiles (upper bound)
    const int grid = 8 * 8 * ceil_div(max_tiles, 16);  // 8 XCDs x slots
    const size_t lds = size_t(kStages) * kStageBytes;
    hipLaunchKernelGGL(attend_prefill_kernel, dim3(grid), dim3(kThreads), lds, stream, q, k, v, q2k,
                       topk, docs, tile_off, ndocs, T, scale * kLog2e, out);
    return hipGetLastError();
}

}  // namespace msa
