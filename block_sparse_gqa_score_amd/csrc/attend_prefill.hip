// Sparse GQA attention over the selected blocks, prefill on packed documents.
//
// Method (NeMo AutoModel minimax_m3_vl.msa, sparse_attention; TensorRT-LLM
// "MiniMaxM3SparseAttentionConfig", class description, step two): query
// head h of token t attends, with softmax over scale * q.k, to the keys of
// t's document at or before t whose document-local 128-key block appears in
// q2k row (h/16, t).
//
// Workgroup = (KV head g, 8 consecutive tokens of one document, all inside
// one 128-token block so they share the query block c).  Its 4 waves each own
// 2 tokens x 16 heads = 32 query columns.  The workgroup walks the UNION of
// its 8 tokens' selected blocks in ascending order; each block's K (row
// major) and V (transposed, d-major) are staged once into LDS through
// coalesced 256-byte row loads and prefetched into registers one block
// ahead.  A wave whose two tokens did not select the block skips it.
//
// Per wave and block (key rows m, query columns n):
//   S^T[128 x 32] = K[128 x 128] . Q^T   4 M-tiles x 8 k-steps of MFMA 32x32x16
//   mask (selected by the column's token, key <= query in the own block),
//   online softmax in the exp2 domain, P^T packed to bf16 straight from the
//   S^T accumulators,
//   O^T[128 x 32] += V^T . P^T            4 d-tiles x 8 k-steps of MFMA 32x32x16
// The accumulator of S^T gives lane (n, hb) the keys 8*(r/4) + 4*hb + r%4 of
// each 32-key tile, so PV step s consumes registers 8*(s%2)..8*(s%2)+7 of
// tile s/2, i.e. keys 16s + 8*(i/4) + 4*hb + i%4; the V^T operand reads the
// same keys as two 4-key runs of the transposed LDS copy.
#include "msa_internal.hpp"

namespace msa {

namespace {
constexpr int kKPitch = kDim + 8;     // bf16 per K row in LDS   (272 B)
constexpr int kVPitch = kBlock + 4;   // bf16 per V^T row in LDS (264 B)
constexpr int kKBytes = kBlock * kKPitch * 2;
constexpr int kVBytes = kDim * kVPitch * 2;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int tile_doc(const int32_t *off, int ndocs, int t) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// 4 keys x 8 d (bf16) -> 8 d-rows x 4 keys: pick 16-bit halves.
__device__ __forceinline__ u32x2 pick_column(const u32x4 (&r)[4], int dpair, bool high) {
    // element (key kk, d = 2*dpair + high) of the 4 loaded rows
    uint32_t e[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) e[kk] = high ? (r[kk][dpair] >> 16) : (r[kk][dpair] & 0xFFFFu);
    return u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
}
}  // namespace

__global__ __launch_bounds__(256) void attend_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ q2k, int topk, const DocSpan *__restrict__ docs,
    const int32_t *__restrict__ tile_off, int ndocs, int T, float scale_log2,
    uint16_t *__restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint16_t *Ks = (uint16_t *)smem;
    uint16_t *Vt = (uint16_t *)(smem + kKBytes);
    __shared__ int s_id[128];
    __shared__ int s_first[128];
    __shared__ int s_mask[128];
    __shared__ int s_ublk[128];
    __shared__ int s_umask[128];
    __shared__ int s_nu;

    const int tile = blockIdx.x;
    const int g = blockIdx.y;
    if (tile >= tile_off[ndocs]) return;
    const int d = tile_doc(tile_off, ndocs, tile);
    const int nt_doc = tile_off[d + 1] - tile_off[d];
    const int local_tile = nt_doc - 1 - (tile - tile_off[d]);
    const DocSpan doc = docs[d];
    const int p0 = local_tile * kAttnTile;
    const int c = p0 / kBlock;
    const int ntok = min(kAttnTile, doc.len - p0);
    const int p_last = p0 + ntok - 1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hb = lane >> 5;

    // ---- union of the tile's selected blocks (ascending, with token masks)
    if (tid == 0) s_nu = 0;
    if (tid < 128) {
        const int tok = tid >> 4, slot = tid & 15;
        int id = -1;
        if (tok < ntok && slot < topk) id = q2k[(size_t(g) * T + doc.start + p0 + tok) * topk + slot];
        s_id[tid] = (id >= 0 && id <= c) ? id : -1;
    }
    __syncthreads();
    if (tid < 128) {
        const int my = s_id[tid];
        int first = my >= 0, mask = 0;
        for (int j = 0; j < 128; ++j) {
            const int o = s_id[j];
            if (o == my) {
                mask |= 1 << (j >> 4);
                if (j < tid) first = 0;
            }
        }
        s_first[tid] = first;
        s_mask[tid] = mask;
    }
    __syncthreads();
    if (tid < 128 && s_first[tid]) {
        const int my = s_id[tid];
        int pos = 0;
        for (int j = 0; j < 128; ++j) pos += (s_first[j] && s_id[j] < my);
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

    // ---- staging: K rows (8 chunks of 16 B) and V (2 items of 4 keys x 8 d)
    u32x4 kst[8];
    u32x4 vst[2][4];
    auto load_block = [&](int b) {
        const size_t row0 = size_t(doc.start) + size_t(b) * kBlock;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int chunk = tid + 256 * i;
            const int r = chunk >> 4, col = chunk & 15;
            const int kp = b * kBlock + r;
            kst[i] = kp <= p_last ? *(const u32x4 *)(k + ((row0 + r) * kKvHeads + g) * kDim + 8 * col)
                                  : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int item = tid + 256 * j;
            const int dg = item & 15, kg = item >> 4;  // d 8dg..8dg+7, keys 4kg..4kg+3
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int r = 4 * kg + kk;
                const int kp = b * kBlock + r;
                vst[j][kk] = kp <= p_last
                                 ? *(const u32x4 *)(v + ((row0 + r) * kKvHeads + g) * kDim + 8 * dg)
                                 : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_block = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int chunk = tid + 256 * i;
            const int r = chunk >> 4, col = chunk & 15;
            *(u32x4 *)(Ks + r * kKPitch + 8 * col) = kst[i];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int item = tid + 256 * j;
            const int dg = item & 15, kg = item >> 4;
#pragma unroll
            for (int dd = 0; dd < 8; ++dd)
                *(u32x2 *)(Vt + (8 * dg + dd) * kVPitch + 4 * kg) = pick_column(vst[j], dd >> 1, dd & 1);
        }
    };

    f32x16 acc_o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc_o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    if (nu > 0) load_block(s_ublk[0]);
    for (int u = 0; u < nu; ++u) {
        const int b = s_ublk[u];
        const int umask = s_umask[u];
        store_block();
        __syncthreads();
        if (u + 1 < nu) load_block(s_ublk[u + 1]);

        const bool wave_active = ((umask >> (2 * wave)) & 3) != 0;
        if (wave_active) {
            f32x16 acc_s[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc_s[mt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                bf16x8 a[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    a[mt] = __builtin_bit_cast(
                        bf16x8, *(const u32x4 *)(Ks + (32 * mt + n) * kKPitch + 16 * ks + 8 * hb));
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc_s[mt] = mfma_32x32x16(a[mt], qb[ks], acc_s[mt]);
            }

            const bool sel = tok_ok && ((umask >> my_tok) & 1);
            const bool diag = (b == c);
            float mloc = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kp = b * kBlock + 32 * mt + 8 * (r >> 2) + 4 * hb + (r & 3);
                    const bool ok = sel && (!diag || kp <= my_p);
                    const float s = ok ? acc_s[mt][r] * scale_log2 : -INFINITY;
                    acc_s[mt][r] = s;
                    mloc = fmaxf(mloc, s);
                }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const float m_new = fmaxf(m_run, mloc);
            const float base = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - base);
            m_run = m_new;
            float psum = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(acc_s[mt][r] - base);
                    acc_s[mt][r] = p;
                    psum += p;
                }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc_o[dt] *= alpha;

#pragma unroll
            for (int s = 0; s < 8; ++s) {
                bf16x8 pb;
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[i] = (__bf16)acc_s[s >> 1][8 * (s & 1) + i];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const uint16_t *row = Vt + (32 * dt + n) * kVPitch + 16 * s + 4 * hb;
                    const u32x2 lo = *(const u32x2 *)(row);
                    const u32x2 hi = *(const u32x2 *)(row + 8);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                    acc_o[dt] = mfma_32x32x16(a, pb, acc_o[dt]);
                }
            }
        }
        __syncthreads();
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
    const int grid = ceil_div(T, kAttnTile) + ndocs;
    const size_t lds = size_t(kKBytes) + size_t(kVBytes);
    hipLaunchKernelGGL(attend_prefill_kernel, dim3(grid, kKvHeads), dim3(256), lds, stream, q, k, v,
                       q2k, topk, docs, tile_off, ndocs, T, scale * kLog2e, out);
    return hipGetLastError();
}

}  // namespace msa
