// route.hip -- router of the MoE layer on gfx950.
//
// Routing stays on the GPU ("Perplexity Open-Sources Lily ...", section
// "The optimizations follow the workload"): logits, softmax, top-8 and the
// renormalised weights are produced here and consumed by the permutation
// kernels without any host round trip.
//
//   route_logits_gemv   T <= 32: one wave per expert row of W_r, every lane
//                       streams 64 B of the row (coalesced 16 B loads) and
//                       dots it with the (cached) token rows.
//   route_logits_tile   larger T: the logits as a small GEMM, one workgroup
//                       per 32 tokens x 128 experts, bf16 MFMA 32x32x16 (fp32
//                       accumulation of exact bf16 products) on tiles moved
//                       into LDS by a 7-stage direct-load ring; below a
//                       few thousand tokens K is split over up to 8
//                       workgroup slices to fill the chip.
//   route_topk          one wave per token (summing the K slices, if any):
//                       4 logits per lane, eight arg-max
//                       rounds over the fp32 logits (ties -> lower expert
//                       index), softmax weights renormalised over the
//                       selected eight, and the shared-expert gate
//                       sigmoid(x . w_sg).
#include "block_util.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float dot8_bf16(uint4v a, uint4v b) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s = fmaf(bf16_to_f32(a[i] & 0xFFFFu), bf16_to_f32(b[i] & 0xFFFFu), s);
        s = fmaf(bf16_to_f32(a[i] >> 16), bf16_to_f32(b[i] >> 16), s);
    }
    return s;
}

// grid: E/4 blocks of 4 waves; wave -> expert row; T <= 32.
__global__ __launch_bounds__(256) void route_logits_gemv(const uint16_t* __restrict__ x, int T,
                                                         const uint16_t* __restrict__ wr,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const uint4v* wrow = reinterpret_cast<const uint4v*>(wr + (size_t)e * H) + lane * 4;
    uint4v w0 = wrow[0], w1 = wrow[1], w2 = wrow[2], w3 = wrow[3];
    const float b = bias ? bias[e] : 0.f;
    for (int t = 0; t < T; ++t) {
        const uint4v* xr = reinterpret_cast<const uint4v*>(x + (size_t)t * H) + lane * 4;
        float s = dot8_bf16(xr[0], w0) + dot8_bf16(xr[1], w1) + dot8_bf16(xr[2], w2) +
                  dot8_bf16(xr[3], w3);
        s = wave_sum(s);
        if (lane == 0) logits[(size_t)t * E + e] = s + b;
    }
}

typedef float float16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rt_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Router logits for T > 32.  grid: (ceil(T/TOK), 2) workgroups of 4 waves;
// workgroup (b, h) computes tokens TOK b .. TOK b + TOK-1 against experts
// 128h .. 128h+127, wave w the 32 experts 128h + 32w .. +31, as TOK/32
// 32x32 fp32 accumulators of v_mfma_f32_32x32x16_bf16 (lane l: token /
// expert l%32, k = 8*(l/32)..+7 of each 16-wide step).  K advances in
// supersteps of 64; the x tile (TOK rows) and the W_r tile (128 rows) of a
// superstep move into LDS with coalesced direct loads (1 KB = 8 rows x
// 128 B per instruction) through a ring of 7 stages (6 for 64-token
// tiles), so that many supersteps are in flight while one is multiplied.
// The kernel is bound by that load ring, not by the MFMAs; 64-token tiles
// read the router matrix once per 64 tokens instead of per 32.  Rows are
// stored with their 16-byte pieces XOR-swizzled by (row >> 1) & 7, so a
// 16-lane operand read hits 16 distinct bank groups; MFMA step s reads
// piece 4g + s (g = l/32) of both operands.  Token rows past T load zeros
// (buffer range) and are not stored.
constexpr int RL_EXP = 128;
template <int TOK>
struct RLG {
    static constexpr int STAGES = TOK == 64 ? 6 : 7;
    static constexpr int STAGE = (TOK + RL_EXP) * 128;   // bytes per superstep
    static constexpr int INSTR = STAGE / 1024;           // 1 KB direct loads per superstep
    static constexpr int PER_WAVE = INSTR / 4;
    static constexpr int MT = TOK / 32;                  // 32-token MFMA tiles
    static_assert(TOK == 32 || TOK == 64, "token tile");
    static_assert(INSTR % 4 == 0, "router loads split evenly over the waves");
    static_assert(STAGES * STAGE <= 160 * 1024, "router LDS");
    static_assert((STAGES - 2) * PER_WAVE <= 63, "vmcnt range");
};
// Token tile of the router GEMM at T tokens (the 64-token tile halves the
// router-matrix traffic; below a few thousand tokens the 32-token tile
// keeps twice the workgroups).
#ifndef RL_TOK64_MIN_T
#define RL_TOK64_MIN_T 2048
#endif
static int route_tok(int T) { return T >= RL_TOK64_MIN_T ? 64 : 32; }

typedef __attribute__((address_space(3))) void* rt_lds_t;

// Instruction j = wave + 4i fills stage rows 8j .. 8j+7 (rows 0..TOK-1: x
// tokens, then 128 W_r experts): lane -> row 8j + lane/8, LDS slot lane%8
// holding the row's piece slot ^ ((row >> 1) & 7).
template <int TOK>
__device__ __forceinline__ void rl_issue(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                         int t0, int e0, int wave, int lane, int u,
                                         uint8_t* stage) {
#pragma unroll
    for (int i = 0; i < RLG<TOK>::PER_WAVE; ++i) {
        const int j = wave + 4 * i;
        const int row = 8 * j + (lane >> 3);
        const int p = (lane & 7) ^ ((row >> 1) & 7);
        uint8_t* dst = stage + j * 1024;
        if (j < TOK / 8) {
            const uint32_t off = (uint32_t)(t0 + row) * (H * 2) + (uint32_t)(u * 128 + 16 * p);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (rt_lds_t)dst, 16, off, 0, 0, 0);
        } else {
            const uint32_t off = (uint32_t)(e0 + row - TOK) * (H * 2) + (uint32_t)(u * 128 + 16 * p);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (rt_lds_t)dst, 16, off, 0, 0, 0);
        }
    }
}

// KS > 1 splits K over blockIdx.z: slice z covers supersteps z*NU/KS ..
// (z+1)*NU/KS - 1 and writes its unbiased partial logits to
// logits[(z*T + t)*E + e]; route_topk sums the slices in order and adds the
// bias.  A few hundred tokens make only T/TOK x 2 workgroups, so the split
// is what fills the chip there.
//
// zero / nzero: optional int array the workgroups clear on the way (the
// permutation's chunk histograms, which the top-8 kernel after this one
// accumulates).
template <int KS, int TOK>
__global__ __launch_bounds__(256) void route_logits_tile(const uint16_t* __restrict__ x, int T,
                                                         const uint16_t* __restrict__ wr,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits,
                                                         int32_t* __restrict__ zero, int nzero) {
    using rg = RLG<TOK>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[rg::STAGES * rg::STAGE];
    if (zero) {
        const int nwg = gridDim.x * gridDim.y * gridDim.z;
        const int wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
        for (int i = wg * 256 + (int)threadIdx.x; i < nzero; i += nwg * 256) zero[i] = 0;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int t0 = blockIdx.x * TOK;
    const int e0 = blockIdx.y * RL_EXP;
    const __amdgpu_buffer_rsrc_t rx = rt_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const __amdgpu_buffer_rsrc_t rw = rt_rsrc(wr, (uint32_t)(E * H * 2));
    constexpr int NU = H / 64 / KS;   // supersteps of this K slice (32 in all)
    static_assert((H / 64) % KS == 0, "K slices");
    constexpr int S = rg::STAGES, PW = rg::PER_WAVE;
    const int u0 = blockIdx.z * NU;

    static_assert(TOK % 8 == 0, "x rows must fill whole load instructions");
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
        if (u < NU) rl_issue<TOK>(rx, rw, t0, e0, wave, lane, u0 + u, smem + u * rg::STAGE);

    float16v acc[rg::MT];
#pragma unroll
    for (int m = 0; m < rg::MT; ++m) acc[m] = (float16v)0.f;
    const int rb = TOK + wave * 32 + l32;     // expert operand row in the stage
    for (int u = 0; u < NU; ++u) {
        // superstep u landed (the later ones may stay in flight): each wave
        // has min(NU - 1 - u, S - 2) more supersteps of loads issued
        const int ahead = min(NU - 1 - u, S - 2);
        switch (ahead) {
            case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * PW)); break;
            case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * PW)); break;
            case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PW)); break;
            case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PW)); break;
            case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1 * PW)); break;
            default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
        }
        static_assert(S - 2 <= 5, "wait cases");
        // every wave's part of superstep u is in LDS, and every wave is done
        // with the stage the refill below overwrites (superstep u - 1)
        pipe_barrier();
        if (u + S - 1 < NU)
            rl_issue<TOK>(rx, rw, t0, e0, wave, lane, u0 + u + S - 1,
                          smem + ((u + S - 1) % S) * rg::STAGE);
        const uint8_t* st = smem + (u % S) * rg::STAGE;
        // all operand reads first, then the MFMAs
        uint4v av[rg::MT][4], bv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int pc = 4 * g + s;
#pragma unroll
            for (int m = 0; m < rg::MT; ++m) {
                const int ra = m * 32 + l32;
                av[m][s] = *reinterpret_cast<const uint4v*>(st + ra * 128 + 16 * (pc ^ ((ra >> 1) & 7)));
            }
            bv[s] = *reinterpret_cast<const uint4v*>(st + rb * 128 + 16 * (pc ^ ((rb >> 1) & 7)));
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int m = 0; m < rg::MT; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[m][s]),
                                                                 __builtin_bit_cast(bf16x8, bv[s]), acc[m],
                                                                 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * (rg::MT + 1), 0);    // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * rg::MT, 0);          // MFMAs
    }
    // element i of tile m: token 32m + 8*(i/4) + 4g + i%4, expert e0 + 32w + l32
    const int e = e0 + wave * 32 + l32;
    const float bb = (KS == 1 && bias) ? bias[e] : 0.f;
    float* out = logits + (size_t)blockIdx.z * T * E;
#pragma unroll
    for (int m = 0; m < rg::MT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = t0 + 32 * m + 8 * (i >> 2) + 4 * g + (i & 3);
            const float v = acc[m][i];
            if (t < T) out[(size_t)t * E + e] = v + bb;
        }
}

// K slices of the router GEMM at T tokens: doubled while the grid stays
// within 256 workgroups, at most RL_KS_MAX.
constexpr int RL_KS_MAX = 8;
static int route_ksplit(int T) {
    const int tok = route_tok(T);
    const int tiles = (T + tok - 1) / tok * (E / RL_EXP);
    int ks = 1;
    while (ks < RL_KS_MAX && tiles * ks * 2 <= 256) ks *= 2;
    return ks;
}

// grid: ceil(T/4) blocks of 4 waves; wave -> token: top-8 (wave_top8),
// renormalised weights and the shared-expert gate; optionally (the fused
// layer) also the fp16 copy of the token's row in chunk-slot order that the
// grouped GEMM reads (xh), which saves the conversion kernel.
//
// part / NKS: K-split partial logits [NKS][T][E] of route_logits_tile<KS>
// (NKS > 1; 0: none, the logits are read): summed here in slice order, plus
// the bias (and stored to logits if it is given).  NKS is a template
// argument so that every slice's load is in flight before the sum (a loop
// bounded at run time waited for each load before issuing the next).
//
// chunk_counts: optional; each token's eight experts are added to the
// histogram of its permutation chunk, chunk_counts[8t / PERM_CHUNK][e]
// (integer atomics: the counts do not depend on their order).
template <int NKS>
__global__ __launch_bounds__(256) void route_topk(float* __restrict__ logits,
                                                  const float* __restrict__ part,
                                                  const float* __restrict__ bias,
                                                  const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ wsg, int T,
                                                  int32_t* __restrict__ ids,
                                                  float* __restrict__ wts,
                                                  float* __restrict__ sg,
                                                  uint16_t* __restrict__ xh,
                                                  int32_t* __restrict__ chunk_counts) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int e;
    const uint4v* xr = reinterpret_cast<const uint4v*>(x + (size_t)t * H) + lane * 4;
    const uint4v x0 = xr[0], x1 = xr[1], x2 = xr[2], x3 = xr[3];
    if constexpr (NKS > 0) {
        float4v pv[NKS];
#pragma unroll
        for (int k = 0; k < NKS; ++k)
            pv[k] = reinterpret_cast<const float4v*>(part + ((size_t)k * T + t) * E)[lane];
        float4v v = pv[0];
#pragma unroll
        for (int k = 1; k < NKS; ++k) v += pv[k];
        if (bias) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += bias[lane * 4 + j];
        }
        if (logits) reinterpret_cast<float4v*>(logits + (size_t)t * E)[lane] = v;
        e = wave_top8_v(v, ids + (size_t)t * TOPK, wts + (size_t)t * TOPK, nullptr);
    } else {
        e = wave_top8_v(reinterpret_cast<const float4v*>(logits + (size_t)t * E)[lane],
                        ids + (size_t)t * TOPK, wts + (size_t)t * TOPK, nullptr);
    }
    if (chunk_counts && lane < TOPK)
        atomicAdd(&chunk_counts[(size_t)(t * TOPK / PERM_CHUNK) * E + e], 1);
    const uint4v* gr = reinterpret_cast<const uint4v*>(wsg) + lane * 4;
    float z = dot8_bf16(x0, gr[0]) + dot8_bf16(x1, gr[1]) + dot8_bf16(x2, gr[2]) +
              dot8_bf16(x3, gr[3]);
    z = wave_sum(z);
    if (lane == 0) sg[t] = 1.f / (1.f + expf(-z));
    if (xh) {
        uint4v* xo = reinterpret_cast<uint4v*>(xh + (size_t)t * H) + lane * 4;
        xo[0] = bf16x8_to_f16_slots(x0);
        xo[1] = bf16x8_to_f16_slots(x1);
        xo[2] = bf16x8_to_f16_slots(x2);
        xo[3] = bf16x8_to_f16_slots(x3);
    }
}

void launch_route_logits(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                         float* logits, hipStream_t st, int32_t* zero, int nzero) {
    if (T <= 32) {
        hipLaunchKernelGGL(route_logits_gemv, dim3(E / 4), dim3(256), 0, st, x, T, wr, bias,
                           logits);
    } else {
        // (unsplit: the 32-token tile keeps more workgroups)
        hipLaunchKernelGGL((route_logits_tile<1, 32>), dim3((T + 31) / 32, E / RL_EXP),
                           dim3(256), 0, st, x, T, wr, bias, logits, zero, nzero);
    }
}

// Whether launch_route accumulates the permutation's chunk histograms (when
// given them): every T whose permutation runs in chunks.
bool route_counts_chunks(int T) { return TOPK * T > PERM_SMALL_MAX; }

// xh: optional fp16 activation copy.  part: optional scratch for K-split
// partial logits, RL_KS_MAX * T * E floats, free for the duration of the
// call (without it the router GEMM runs unsplit).  chunk_counts: optional
// permutation chunk histograms (perm_chunks(T) x E ints), cleared by the
// router GEMM and accumulated by the top-8 kernel when
// route_counts_chunks(T).
void launch_route(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                  const uint16_t* wsg, float* logits, int32_t* ids, float* wts, float* sg,
                  hipStream_t st, uint16_t* xh, float* part, int32_t* chunk_counts) {
    if (!route_counts_chunks(T)) chunk_counts = nullptr;
    const int nzero = chunk_counts ? (TOPK * T + PERM_CHUNK - 1) / PERM_CHUNK * E : 0;
    const int ks = (part && T > 32) ? route_ksplit(T) : 1;
    const int tok = route_tok(T);
    if (ks == 1) {
        if (T > 32 && tok == 64)
            hipLaunchKernelGGL((route_logits_tile<1, 64>), dim3((T + 63) / 64, E / RL_EXP), dim3(256), 0,
                               st, x, T, wr, bias, logits, chunk_counts, nzero);
        else
            launch_route_logits(x, T, wr, bias, logits, st, chunk_counts, nzero);
        hipLaunchKernelGGL(route_topk<0>, dim3((T + 3) / 4), dim3(256), 0, st, logits,
                           (const float*)nullptr, (const float*)nullptr, x, wsg, T, ids, wts,
                           sg, xh, chunk_counts);
        return;
    }
    const dim3 grid((T + tok - 1) / tok, E / RL_EXP, ks);
#define RL_LAUNCH(K, TK) \
    hipLaunchKernelGGL((route_logits_tile<K, TK>), grid, dim3(256), 0, st, x, T, wr, bias, part, chunk_counts, nzero)
    if (tok == 64) {
        switch (ks) {
            case 2: RL_LAUNCH(2, 64); break;
            case 4: RL_LAUNCH(4, 64); break;
            default: RL_LAUNCH(8, 64); break;
        }
    } else {
        switch (ks) {
            case 2: RL_LAUNCH(2, 32); break;
            case 4: RL_LAUNCH(4, 32); break;
            default: RL_LAUNCH(8, 32); break;
        }
    }
#undef RL_LAUNCH
    // (nothing reads the summed logits after the top-8: not stored)
#define RT_LAUNCH(K)                                                                        \
    hipLaunchKernelGGL(route_topk<K>, dim3((T + 3) / 4), dim3(256), 0, st, (float*)nullptr,       \
                       (const float*)part, bias, x, wsg, T, ids, wts, sg, xh, chunk_counts)
    switch (ks) {
        case 2: RT_LAUNCH(2); break;
        case 4: RT_LAUNCH(4); break;
        default: RT_LAUNCH(8); break;
    }
#undef RT_LAUNCH
}

}  // namespace moe
