// Paged decode: selection and sparse GQA attention for one query token per
// request, over a paged K/V cache plus a side index-K cache that shares its
// slots (TensorRT-LLM "MiniMaxM3SparseAttentionConfig", class description;
// vLLM "vllm.models.minimax_m3.amd.sparse_attention_nvfp4", decode path).
// Request r with context length L is one document evaluated at its last
// position L-1; logical key j lives in slot pt[r, j/128]*128 + j%128.
//
// Kernels (one pass over the caches, HBM-bound):
//   decode_scores_kernel - one wave per (request, page): the page's 128
//       index keys against the 4 index heads on MFMA (bf16 16x16x32, or E4M3
//       16x16x128 with unit scales), slots >= L masked, per-page max.
//   decode_topk_kernel   - one wave per (request, index head): the R-th
//       largest score found by bisection on order-preserving score bits with
//       wave-wide counts, then an ascending ballot-compacted emit (ties go
//       to the lower block id); forced init/local blocks always emitted.
//   decode_attend_kernel - one workgroup per (selected block, KV head,
//       request); 4 waves x 32 keys: S^T = K Q^T and O^T = V^T P^T on MFMA
//       16x16x32 (16 query heads = N), partial softmax merged across waves in
//       LDS, one (O, m, l) partial per selected block written to workspace.
//   decode_combine_kernel - per (request, query head): log-sum-exp merge of
//       the partials in fixed block order, bf16 output.
#include "msa_internal.hpp"

namespace msa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDecPagesPerWg = 4;
}  // namespace

// ---------------------------------------------------------------------------
// G4: per-page index scores
// ---------------------------------------------------------------------------
template <bool kFp8>
__global__ __launch_bounds__(256) void decode_scores_kernel(
    const uint8_t *__restrict__ iq, const uint8_t *__restrict__ ikc, const int32_t *__restrict__ pt,
    int max_pages, const int32_t *__restrict__ ctx, int max_ctx, int nb_max, float *__restrict__ S) {
    const int r = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pi = blockIdx.x * kDecPagesPerWg + wave;
    const int L = min(max(ctx[r], 1), max_ctx);
    const int nb = (L + kBlock - 1) / kBlock;
    if (pi >= nb) return;
    const int n = lane & 15, qd = lane >> 4;
    const size_t slot0 = size_t(pt[size_t(r) * max_pages + pi]) * kBlock;
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
        // lane (m, qd), step ks holds d = 32qd + 8ks .. +7 (64 contiguous bytes per lane).
        bf16x8 qb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[ks] = n < kIdxHeads
                         ? __builtin_bit_cast(bf16x8, *(const u32x4 *)(qrow + 2 * (32 * qd + 8 * ks)))
                         : bf16x8{};
        u32x4 ka[8][4];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                ka[mt][ks] = *(const u32x4 *)(kbase + (16 * mt + n) * kRowBytes + 2 * (32 * qd + 8 * ks));
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
    if (qd == 0 && n < kIdxHeads) S[(size_t(r) * kIdxHeads + n) * nb_max + pi] = mx;
}

hipError_t launch_decode_scores(const void *iq, const void *ikc, bool fp8, const int32_t *pt,
                                int max_pages, const int32_t *ctx, int B, int max_ctx, int nb_max, float *S,
                                hipStream_t stream) {
    const dim3 grid(ceil_div(nb_max, kDecPagesPerWg), B);
    if (fp8)
        hipLaunchKernelGGL(decode_scores_kernel<true>, grid, dim3(256), 0, stream,
                           (const uint8_t *)iq, (const uint8_t *)ikc, pt, max_pages, ctx, max_ctx, nb_max, S);
    else
        hipLaunchKernelGGL(decode_scores_kernel<false>, grid, dim3(256), 0, stream,
                           (const uint8_t *)iq, (const uint8_t *)ikc, pt, max_pages, ctx, max_ctx, nb_max, S);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// G5: top-k per (request, index head), one wave each
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <int kCpl>  // candidates per lane: blocks lane + 64*i
__global__ __launch_bounds__(256) void decode_topk_kernel(const float *__restrict__ S,
                                                          const int32_t *__restrict__ ctx, int B,
                                                          int max_ctx, int nb_max, int topk, int init, int local,
                                                          int32_t *__restrict__ q2k) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + wave;  // (r, h) with h fastest
    if (row >= B * kIdxHeads) return;
    const int r = row / kIdxHeads, h = row % kIdxHeads;
    const int c = (min(max(ctx[r], 1), max_ctx) - 1) / kBlock;
    const int R = topk - forced_count(c, init, local);
    const float *srow = S + (size_t(r) * kIdxHeads + h) * nb_max;
    int32_t *out = q2k + (size_t(h) * B + r) * topk;

    // order bits of each non-forced candidate; 0 marks "not a candidate"
    uint32_t u[kCpl];
#pragma unroll
    for (int i = 0; i < kCpl; ++i) {
        const int b = lane + 64 * i;
        u[i] = (b <= c && !is_forced(b, c, init, local)) ? max(float_order_bits(srow[b]), 1u) : 0u;
    }
    // largest x with #{u >= x} >= R (the R-th largest order value)
    uint32_t thr = 0;
    if (R > 0) {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t trial = thr | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < kCpl; ++i) cnt += u[i] >= trial;
            if (wave_sum(cnt) >= R) thr = trial;
        }
    }
    int n_gt = 0;
    if (R > 0) {
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < kCpl; ++i) cnt += u[i] > thr;
        n_gt = wave_sum(cnt);
    }
    const int ties_wanted = R > 0 ? R - n_gt : 0;  // equal-to-threshold picks, lowest ids first
    int ties_seen = 0, emitted = 0;
    const uint64_t below = (1ull << lane) - 1ull;
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
        if (take && pos < topk) out[pos] = b;
        emitted += __popcll(take_mask);
    }
    for (int i = emitted + lane; i < topk; i += 64) out[i] = -1;
}

hipError_t launch_decode_topk(const float *S, const int32_t *ctx, int B, int max_ctx, int nb_max, int topk,
                              int init, int local, int32_t *q2k, hipStream_t stream) {
    const int cpl = ceil_div(nb_max, 64);
    const dim3 grid(ceil_div(B * kIdxHeads, 4));
#define MSA_TOPK_CASE(N)                                                                         \
    if (cpl <= N) {                                                                              \
        hipLaunchKernelGGL(decode_topk_kernel<N>, grid, dim3(256), 0, stream, S, ctx, B, max_ctx, nb_max, \
                           topk, init, local, q2k);                                              \
        return hipGetLastError();                                                                \
    }
    MSA_TOPK_CASE(1)
    MSA_TOPK_CASE(2)
    MSA_TOPK_CASE(4)
    MSA_TOPK_CASE(8)
    MSA_TOPK_CASE(16)
    MSA_TOPK_CASE(32)
    MSA_TOPK_CASE(64)
    MSA_TOPK_CASE(128)
#undef MSA_TOPK_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// G6: attention over one selected block per workgroup
// ---------------------------------------------------------------------------
namespace {
constexpr int kDVPitch = 32 + 4;  // bf16 per V^T row (32 keys + pad) per wave
constexpr int kDecVtBytes = kDim * kDVPitch * 2;

__device__ __forceinline__ u32x2 pick_col4(const u32x4 (&r)[4], int dd) {
    const int dp = dd >> 1;
    const bool high = dd & 1;
    uint32_t e[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) e[kk] = high ? (r[kk][dp] >> 16) : (r[kk][dp] & 0xFFFFu);
    return u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
}
}  // namespace

__global__ __launch_bounds__(256) void decode_attend_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    const int32_t *__restrict__ pt, int max_pages, const int32_t *__restrict__ ctx, int max_ctx, int B,
    const int32_t *__restrict__ q2k, int topk, float scale_log2, float *__restrict__ part_o,
    float *__restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kDecVtBytes];
    __shared__ float s_m[4][16], s_l[4][16];
    const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, qd = lane >> 4;
    const size_t pidx = (size_t(r) * kKvHeads + g) * topk + s;
    float *po = part_o + pidx * (kGroup * kDim);
    float *pml = part_ml + pidx * (kGroup * 2);

    const int L = min(max(ctx[r], 1), max_ctx);
    const int c = (L - 1) / kBlock;
    const int b = q2k[(size_t(g) * B + r) * topk + s];
    if (b < 0 || b > c) {
        if (tid < kGroup) {
            pml[2 * tid] = -INFINITY;
            pml[2 * tid + 1] = 0.f;
        }
        return;
    }
    const size_t slot0 = size_t(pt[size_t(r) * max_pages + b]) * kBlock;
    const int key0 = 32 * wave;  // this wave's keys within the block

    // Q^T operand: lane (n = head, qd), step ks: d = 32qd + 8ks .. +7
    const uint16_t *qrow = q + (size_t(r) * kHeads + g * kGroup + n) * kDim;
    bf16x8 qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qrow + 32 * qd + 8 * ks));

    // K operand: M-tile mt = keys key0 + 16mt + m, same d order as Q
    u32x4 ka[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const uint16_t *src = kc + ((slot0 + key0 + 16 * mt + n) * kKvHeads + g) * kDim + 32 * qd;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[mt][ks] = *(const u32x4 *)(src + 8 * ks);
    }
    // V: 2 items of 4 keys x 8 d per lane (keys 4kg.., d 8dg..)
    u32x4 vr[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int item = lane + 64 * j;
        const int dg = item & 15, kg = item >> 4;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int key = key0 + 4 * kg + kk;
            const bool ok = b * kBlock + key < L;  // slots past L may hold NaN
            vr[j][kk] = ok ? *(const u32x4 *)(vc + ((slot0 + key) * kKvHeads + g) * kDim + 8 * dg)
                           : u32x4{0, 0, 0, 0};
        }
    }

    f32x4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            sacc[mt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, ka[mt][ks]), qb[ks], sacc[mt]);
    }

    // stage V^T for this wave
    uint16_t *vt = (uint16_t *)(smem + wave * kDecVtBytes);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int item = lane + 64 * j;
        const int dg = item & 15, kg = item >> 4;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) *(u32x2 *)(vt + (8 * dg + dd) * kDVPitch + 4 * kg) = pick_col4(vr[j], dd);
    }

    // softmax over this wave's 32 keys, per head column n
    float mloc = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = b * kBlock + key0 + 16 * mt + 4 * qd + i;
            const float z = j < L ? sacc[mt][i] * scale_log2 : -INFINITY;
            sacc[mt][i] = z;
            mloc = fmaxf(mloc, z);
        }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float base = mloc == -INFINITY ? 0.f : mloc;
    float psum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(sacc[mt][i] - base);
            psum += p;
            pb[4 * mt + i] = (__bf16)p;
        }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    __syncthreads();

    // O^T[d x heads] = V^T . P^T; lane (m = d, qd) reads keys 4qd.. and 16+4qd..
    f32x4 oacc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const uint16_t *row = vt + (16 * dt + n) * kDVPitch + 4 * qd;
        const u32x2 lo = *(const u32x2 *)row;
        const u32x2 hi = *(const u32x2 *)(row + 16);
        oacc[dt] = mfma_16x16x32(__builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, f32x4{});
    }
    __syncthreads();  // V^T no longer needed: reuse LDS for the cross-wave merge

    float *so = (float *)smem;  // [4 waves][16 heads][128 d]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) so[(wave * kGroup + n) * kDim + 16 * dt + 4 * qd + i] = oacc[dt][i];
    if (qd == 0) {
        s_m[wave][n] = mloc;
        s_l[wave][n] = psum;
    }
    __syncthreads();
    // merge: thread -> (head hh, 8 d)
    {
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
        for (int e = 0; e < 8; ++e) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) acc += sc[w] * so[(w * kGroup + hh) * kDim + d0 + e];
            o[e] = acc;
        }
        *(f32x4 *)(po + hh * kDim + d0) = f32x4{o[0], o[1], o[2], o[3]};
        *(f32x4 *)(po + hh * kDim + d0 + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if ((tid & 15) == 0) {
            pml[2 * hh] = M;
            pml[2 * hh + 1] = l;
        }
    }
}

// ---------------------------------------------------------------------------
// G7: combine the per-block partials
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void decode_combine_kernel(const float *__restrict__ part_o,
                                                             const float *__restrict__ part_ml,
                                                             int topk, uint16_t *__restrict__ out) {
    const int h = blockIdx.x, r = blockIdx.y, dd = threadIdx.x;
    const int g = h / kGroup, hh = h % kGroup;
    const size_t base = (size_t(r) * kKvHeads + g) * topk;
    float M = -INFINITY;
    for (int s = 0; s < topk; ++s) M = fmaxf(M, part_ml[(base + s) * (kGroup * 2) + 2 * hh]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < topk; ++s) {
            const float m = part_ml[(base + s) * (kGroup * 2) + 2 * hh];
            if (m == -INFINITY) continue;
            const float w = __builtin_amdgcn_exp2f(m - M);
            den += w * part_ml[(base + s) * (kGroup * 2) + 2 * hh + 1];
            num += w * part_o[(base + s) * (kGroup * kDim) + hh * kDim + dd];
        }
    }
    const float o = den > 0.f ? num / den : 0.f;
    out[(size_t(r) * kHeads + h) * kDim + dd] = __builtin_bit_cast(uint16_t, (__bf16)o);
}

hipError_t launch_decode_attend(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                                const int32_t *pt, int max_pages, const int32_t *ctx, int max_ctx, int B,
                                const int32_t *q2k, int topk, float scale, float *partial,
                                uint16_t *out, hipStream_t stream) {
    float *part_o = partial;
    float *part_ml = partial + size_t(B) * kKvHeads * topk * kGroup * kDim;
    (void)out;
    hipLaunchKernelGGL(decode_attend_kernel, dim3(topk, kKvHeads, B), dim3(256), 0, stream, q, kc, vc,
                       pt, max_pages, ctx, max_ctx, B, q2k, topk, scale * kLog2e, part_o, part_ml);
    return hipGetLastError();
}

hipError_t launch_decode_combine(const float *partial, int B, int topk, uint16_t *out,
                                 hipStream_t stream) {
    const float *part_o = partial;
    const float *part_ml = partial + size_t(B) * kKvHeads * topk * kGroup * kDim;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(kHeads, B), dim3(128), 0, stream, part_o, part_ml,
                       topk, out);
    return hipGetLastError();
}

}  // namespace msa
