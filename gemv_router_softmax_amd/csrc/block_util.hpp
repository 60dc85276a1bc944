// block_util.hpp -- workgroup / wave building blocks shared by the routing,
// permutation and decode kernels (header-only: each kernel file inlines them).
#pragma once

#include "common.hpp"

namespace moe {

// Wave index within the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

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

// Maximum of a per-lane key over each row of 16 lanes, left in every lane
// of the row (DPP lane exchanges: pairs, quads, half-row mirror, row mirror).
__device__ __forceinline__ uint32_t row16_max(uint32_t k) {
    k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x141, 0xF, 0xF, false));  // row_half_mirror
    k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x140, 0xF, 0xF, false));  // row_mirror
    return k;
}

// Top-8 of the 256 logits of one token, computed by one wave.  Lane l holds
// experts 4l .. 4l+3 (v4).  Candidates are ordered by (logit descending,
// expert ascending) -- exactly the selection order of the definition, for
// every finite logit: each logit becomes its order-preserving 32-bit key
// (distinct logits give distinct keys; -0 and +0 the same key) and equal keys
// are ordered by expert index.  Each lane first sorts its four (key, expert)
// pairs in that order, so its best remaining candidate is always c[0].  Each
// of the eight rounds takes the wave maximum of the c[0] keys (row maxima by
// DPP, then the four rows through scalar registers); the lowest lane holding
// that key (a ballot) holds the lowest expert among equal logits, since lane
// l's experts are all below lane l+1's, and that lane shifts its list by one.
// The code is branch-free: at one token this wave's instruction count is the
// latency of the routing step.  Lane k < 8 ends with the k-th selection and
// writes its id and weight; the weights are computed from the exact fp32
// logits (fetched once from their lanes at the end) as the softmax over all
// experts renormalised over the eight, i.e. exp(l - l_0) / sum_sel
// exp(l - l_0), with l_0 the first selection's logit (the full denominator
// and the reference logit cancel).  Returns, in lane k < 8, the k-th
// selected expert.
__device__ inline int wave_top8_v(float4v v4, int32_t* __restrict__ ids_out,
                                  float* __restrict__ w_out, int32_t* __restrict__ ids_lds) {
    const int lane = threadIdx.x & 63;
    uint32_t c[4];
    int id[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        c[j] = fkey(v4[j]);
        id[j] = 4 * lane + j;
    }
    // compare-exchange: (c[x], id[x]) ahead of (c[y], id[y]) afterwards
    auto ce = [&](int x, int y) {
        const bool sw = c[y] > c[x] || (c[y] == c[x] && id[y] < id[x]);
        const uint32_t kx = sw ? c[y] : c[x], ky = sw ? c[x] : c[y];
        const int ix = sw ? id[y] : id[x], iy = sw ? id[x] : id[y];
        c[x] = kx; c[y] = ky; id[x] = ix; id[y] = iy;
    };
    ce(0, 1);
    ce(2, 3);
    ce(0, 2);
    ce(1, 3);
    ce(1, 2);
    int emine = 0;
#pragma unroll
    for (int k = 0; k < TOPK; ++k) {
        const uint32_t rm = row16_max(c[0]);
        const uint32_t gm = max(max((uint32_t)__builtin_amdgcn_readlane((int)rm, 0),
                                    (uint32_t)__builtin_amdgcn_readlane((int)rm, 16)),
                                max((uint32_t)__builtin_amdgcn_readlane((int)rm, 32),
                                    (uint32_t)__builtin_amdgcn_readlane((int)rm, 48)));
        const uint64_t holders = __ballot(c[0] == gm);
        const int L = (int)__builtin_ctzll(holders);     // lowest holder: the lowest expert
        const int e = __builtin_amdgcn_readlane(id[0], L);
        const bool me = lane == L;
        c[0] = me ? c[1] : c[0];
        c[1] = me ? c[2] : c[1];
        c[2] = me ? c[3] : c[2];
        c[3] = me ? 0u : c[3];
        id[0] = me ? id[1] : id[0];
        id[1] = me ? id[2] : id[1];
        id[2] = me ? id[3] : id[2];
        emine = lane == k ? e : emine;
    }
    // exact logit of this lane's selection: slot emine & 3 of lane emine >> 2
    const int src = emine >> 2, sl = emine & 3;
    const float s0 = __shfl(v4[0], src, WAVE), s1 = __shfl(v4[1], src, WAVE);
    const float s2 = __shfl(v4[2], src, WAVE), s3 = __shfl(v4[3], src, WAVE);
    const float lv = sl == 0 ? s0 : sl == 1 ? s1 : sl == 2 ? s2 : s3;
    const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), 0));
    const float ex = lane < TOPK ? expf(lv - l0) : 0.f;
    // sum over lanes 0..7 (pairs, quads, then the half-row mirror)
    float s = ex + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                       0, __builtin_bit_cast(int, ex), 0xB1, 0xF, 0xF, false));
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x4E,
                                                               0xF, 0xF, false));
    s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x141,
                                                               0xF, 0xF, false));
    if (lane < TOPK) {
        ids_out[lane] = emine;
        w_out[lane] = ex * (1.f / s);
        if (ids_lds) ids_lds[lane] = emine;
    }
    return emine;
}

// As wave_top8_v, reading the token's 256 logits from lg.
__device__ inline void wave_top8(const float* __restrict__ lg, int32_t* __restrict__ ids_out,
                                 float* __restrict__ w_out, int32_t* __restrict__ ids_lds) {
    const int lane = threadIdx.x & 63;
    wave_top8_v(reinterpret_cast<const float4v*>(lg)[lane], ids_out, w_out, ids_lds);
}

// Sums of eight per-lane values over the 64 lanes of a wave, as
// wave-uniform values (wave_sum on each; the eight DPP chains are
// independent, so they overlap) -- no LDS traffic.
__device__ __forceinline__ void wave_sum8(const float v[8], float out[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = wave_sum(v[i]);
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
