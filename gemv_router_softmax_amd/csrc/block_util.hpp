// block_util.hpp -- workgroup / wave building blocks shared by the routing,
// permutation and decode kernels (header-only: each kernel file inlines them).
#pragma once

#include "common.hpp"

namespace moe {

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & 63;
    return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Exclusive scan of one int per thread over a 256-thread block.
__device__ inline int block_excl_scan256(int v, int* lds /* >= 4 ints */, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(inc, o, WAVE);
        if (lane >= o) inc += n;
    }
    if (lane == 63) lds[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        int s = lds[w];
        if (w < wave) base += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + inc - v;
}

// Stable scatter of entries [f0, f1).  base[e] (LDS) is the next sorted
// position of expert e and advances as entries are placed; wcnt (LDS,
// 4*256 ints) must be zero on entry and is zero on exit.
__device__ inline void stable_scatter(const int32_t* __restrict__ ids, int f0, int f1, int* base,
                               int* wcnt, int32_t* __restrict__ perm,
                               int32_t* __restrict__ inv, const float* __restrict__ wsrc = nullptr,
                               float* __restrict__ wsorted = nullptr) {
    const int tid = threadIdx.x, wave = tid >> 6;
    for (int c0 = f0; c0 < f1; c0 += 256) {
        const int f = c0 + tid;
        const bool valid = f < f1;
        const int e = valid ? ids[f] : -1;
        const bool ok = valid && e >= 0 && e < E;
        if (valid && !ok) inv[f] = -1;
        const int key = ok ? e : 511;
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            uint64_t m = __ballot((key >> b) & 1);
            peers &= ((key >> b) & 1) ? m : ~m;
        }
        const uint64_t below = peers & lanemask_lt();
        const int rank = __popcll(below);
        if (ok && below == 0) wcnt[wave * 256 + e] = __popcll(peers);
        __syncthreads();
        if (ok) {
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += wcnt[w * 256 + e];
            const int pos = base[e] + pre + rank;
            perm[pos] = f;
            inv[f] = pos;
            if (wsorted) wsorted[pos] = wsrc[f];
        }
        __syncthreads();
        int s = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            s += wcnt[w * 256 + tid];
            wcnt[w * 256 + tid] = 0;
        }
        base[tid] += s;
        __syncthreads();
    }
}

// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t fkey(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);   // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Top-8 of the 256 logits of one token, computed by one wave.  Lane l holds
// experts 4l .. 4l+3.  Writes ids / weights in descending logit order.
__device__ inline void wave_top8(const float* __restrict__ lg, int32_t* __restrict__ ids_out,
                          float* __restrict__ w_out, int32_t* __restrict__ ids_lds) {
    const int lane = threadIdx.x & 63;
    const float4v v4 = reinterpret_cast<const float4v*>(lg)[lane];
    const float v[4] = {v4[0], v4[1], v4[2], v4[3]};
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = fkey(v[i]);
    // largest K with #(key >= K) >= 8  ==  the 8th largest key
    uint32_t prefix = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = prefix | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt += popc64(__ballot(key[i] >= cand));
        if (cnt >= TOPK) prefix = cand;
    }
    const uint32_t k8 = prefix;
    int above = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) above += popc64(__ballot(key[i] > k8));
    // ties at k8: the lowest expert indices fill the remaining places
    const int need = TOPK - above;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
    bool sel[4];
    int eq_before_lane = 0;
    uint64_t eqm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) eqm[i] = __ballot(key[i] == k8);
#pragma unroll
    for (int i = 0; i < 4; ++i) eq_before_lane += popc64(eqm[i] & lt);
    int eq_in_lane = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool eq = key[i] == k8;
        sel[i] = key[i] > k8 || (eq && eq_before_lane + eq_in_lane < need);
        eq_in_lane += eq ? 1 : 0;
    }
    // gather the 8 selected (value, expert) pairs into uniform registers,
    // lowest lane first within each of the four per-lane slots
    uint64_t msk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) msk[i] = __ballot(sel[i]);
    float sv[TOPK];
    int se[TOPK];
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
        const int i = msk[0] ? 0 : (msk[1] ? 1 : (msk[2] ? 2 : 3));
        const uint64_t mi = i == 0 ? msk[0] : (i == 1 ? msk[1] : (i == 2 ? msk[2] : msk[3]));
        const int l = mi ? __builtin_ctzll(mi) : 0;
        const uint64_t clr = mi & (mi - 1);
        if (i == 0) msk[0] = clr; else if (i == 1) msk[1] = clr; else if (i == 2) msk[2] = clr;
        else msk[3] = clr;
        const float vi = i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
        sv[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vi), l));
        se[k] = 4 * l + i;
    }
    // order: rank of element k = #elements before it (larger value, or equal
    // value and lower expert index); ranks are a permutation of 0..7
    int rk[TOPK];
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
        int rnk = 0;
#pragma unroll
        for (int j = 0; j < TOPK; ++j)
            rnk += (sv[j] > sv[k] || (sv[j] == sv[k] && se[j] < se[k])) ? 1 : 0;
        rk[k] = rnk;
    }
    float vmax = sv[0];
#pragma unroll
    for (int k = 1; k < TOPK; ++k) vmax = fmaxf(vmax, sv[k]);
    // softmax over all experts renormalised over the selected eight: the
    // full denominator cancels, leaving exp(l - l_max) / sum_sel exp(l - l_max)
    float ex[TOPK], s = 0.f;
#pragma unroll
    for (int k = 0; k < TOPK; ++k) { ex[k] = expf(sv[k] - vmax); s += ex[k]; }
    const float inv = 1.f / s;
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
        if (lane == rk[k]) {
            ids_out[lane] = se[k];
            w_out[lane] = ex[k] * inv;
            if (ids_lds) ids_lds[lane] = se[k];
        }
    }
}

// Sum eight per-lane values over the 64 lanes of a wave with 10 exchanges:
// three halving steps leave lane l holding the 8-lane partial of value
// ((l>>5)&1)*4 + ((l>>4)&1)*2 + ((l>>3)&1), three more finish the sum.
__device__ __forceinline__ float wave_sum8(float v[8]) {
    const int lane = threadIdx.x & 63;
    const bool h32 = lane & 32, h16 = lane & 16, h8 = lane & 8;
    float a[4], b[2], c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float send = h32 ? v[i] : v[i + 4];
        const float keep = h32 ? v[i + 4] : v[i];
        a[i] = keep + __shfl_xor(send, 32, WAVE);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = h16 ? a[i] : a[i + 2];
        const float keep = h16 ? a[i + 2] : a[i];
        b[i] = keep + __shfl_xor(send, 16, WAVE);
    }
    {
        const float send = h8 ? b[0] : b[1];
        const float keep = h8 ? b[1] : b[0];
        c = keep + __shfl_xor(send, 8, WAVE);
    }
    c += __shfl_xor(c, 4, WAVE);
    c += __shfl_xor(c, 2, WAVE);
    c += __shfl_xor(c, 1, WAVE);
    return c;   // value index: 4*h32 + 2*h16 + h8
}

// s_waitcnt immediate: wait until at most n vector-memory operations of
// this wave are outstanding (they retire in issue order); expcnt and
// lgkmcnt are left at their maximum (no wait).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int LGKM0_IMM = 15 | (3 << 14) | (7 << 4);   // lgkmcnt(0) only

// Workgroup barrier inside a software pipeline.  __syncthreads() also acts
// as a memory fence, which makes every wave wait for ALL of its outstanding
// vector-memory operations -- including the prefetches meant to stay in
// flight.  Here the caller has already waited (s_waitcnt vmcnt) for exactly
// the loads the next stage needs; this drains only the LDS counter and
// synchronises execution.  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void pipe_barrier() {
    __builtin_amdgcn_s_waitcnt(LGKM0_IMM);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace moe
