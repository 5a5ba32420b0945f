// Device helpers shared by the prefill attention kernels (forward and dQ):
// the global->LDS unit copies and their waits, 4-row reductions over the
// MFMA D layout, and the union of a query tile's selected blocks.
#pragma once

#include "msa_internal.hpp"

namespace msa {

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier that drains this wave's LDS operations but leaves its
// global->LDS prefetch in flight (a plain __syncthreads would also wait for
// every outstanding vector-memory operation).  Callers wait for the unit
// they are about to read with an explicit vmcnt first.
__device__ __forceinline__ void barrier_keep_prefetch() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most n of this wave's copies are outstanding (copies
// complete in issue order).  n > 40 falls back to a full wait.
__device__ __forceinline__ void wait_copies(int n) {
#define MSA_WAIT_CASE(i) \
    case i: asm volatile("s_waitcnt vmcnt(" #i ")" ::: "memory"); break;
    switch (n) {
        MSA_WAIT_CASE(1) MSA_WAIT_CASE(2) MSA_WAIT_CASE(3) MSA_WAIT_CASE(4)
        MSA_WAIT_CASE(5) MSA_WAIT_CASE(6) MSA_WAIT_CASE(7) MSA_WAIT_CASE(8)
        MSA_WAIT_CASE(9) MSA_WAIT_CASE(10) MSA_WAIT_CASE(11) MSA_WAIT_CASE(12)
        MSA_WAIT_CASE(13) MSA_WAIT_CASE(14) MSA_WAIT_CASE(15) MSA_WAIT_CASE(16)
        MSA_WAIT_CASE(17) MSA_WAIT_CASE(18) MSA_WAIT_CASE(19) MSA_WAIT_CASE(20)
        MSA_WAIT_CASE(24) MSA_WAIT_CASE(28) MSA_WAIT_CASE(32) MSA_WAIT_CASE(36)
        MSA_WAIT_CASE(40)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef MSA_WAIT_CASE
}

// HBM -> LDS copy of 16 bytes per lane (lane l writes lds_dst + 16l).  It is
// issued from asm so that the compiler does not hold later LDS reads of
// other ring slots behind it (it cannot tell the slots apart and would wait
// for every copy in flight); completion is awaited with explicit vmcnt.
__device__ __forceinline__ void copy_to_lds(const void *src, uint8_t *lds_dst) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)lds_dst);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The same copy from a wave-uniform base (in SGPRs) plus a 32-bit unsigned
// per-lane byte offset, the instruction's saddr form: the lane's address
// then costs no 64-bit vector arithmetic.
__device__ __forceinline__ void copy_to_lds_s(const void *sbase, uint32_t voff, uint8_t *lds_dst) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)lds_dst);
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Max over the four 16-lane rows of a wave, for each lane position: each
// swap of a register with itself returns, at every lane, the lane's own
// value and that of its partner row (rows r, r^2 for the 32-lane swap;
// r, r^1 for the 16-lane swap).
__device__ __forceinline__ float row_max4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Index d with off[d] <= x < off[d+1] of a prefix-count array off[0..ndocs].
__device__ __forceinline__ int prefix_doc(const int32_t *off, int ndocs, int x) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Union of the selected blocks of a tile of ntok <= 16 consecutive tokens
// (first token tok0, all in query block c of one document) for KV head g:
// ublk[0..nu) ascending, umask[u] bit i set when token i selected ublk[u].
// Ids outside 0..c and -1 are dropped; repeats count once.  Called by every
// thread of the workgroup (>= 256 threads); returns nu to all of them.
__device__ __forceinline__ int tile_union(const int32_t *__restrict__ q2k, int T, int topk, int g,
                                          int tok0, int ntok, int c, int tid, int *s_id,
                                          int *s_first, int *s_mask, int *ublk, int *umask,
                                          int *s_nu) {
    constexpr int kEntries = kAttnTile * kMaxTopk;  // 256 (token, slot) pairs
    if (tid == 0) *s_nu = 0;
    if (tid < kEntries) {
        const int tok = tid >> 4, sl = tid & 15;
        int id = -1;
        if (tok < ntok && sl < topk) id = q2k[(size_t(g) * T + tok0 + tok) * topk + sl];
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
        ublk[pos] = my;
        umask[pos] = s_mask[tid];
        atomicAdd(s_nu, 1);
    }
    __syncthreads();
    return *s_nu;
}

}  // namespace msa
