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
//   route_logits_mfma   larger T: bf16 MFMA 16x16x32 tiles, 64 tokens x 16
//                       experts per wave, fp32 accumulation (bf16 products
//                       are exact in fp32).
//   route_topk          one wave per token: 4 logits per lane, radix selection
//                       of the 8th largest fp32 logit with wave ballots (ties ->
//                       lower expert index), softmax weights renormalised over
//                       the selected eight, and the shared-expert gate
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

// grid: (ceil(T/64), E/64); 4 waves, wave w -> experts blockIdx.y*64 + 16w .. +16.
__global__ __launch_bounds__(256) void route_logits_mfma(const uint16_t* __restrict__ x, int T,
                                                         const uint16_t* __restrict__ wr,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, j = lane >> 4;
    const int t0 = blockIdx.x * 64;
    const int e0 = blockIdx.y * 64 + wave * 16;
    const uint4v* wrow = reinterpret_cast<const uint4v*>(wr + (size_t)(e0 + r) * H) + j;
    const uint4v* xrow[4];
    bool tok_ok[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        int t = t0 + mt * 16 + r;
        tok_ok[mt] = t < T;
        xrow[mt] = reinterpret_cast<const uint4v*>(x + (size_t)(tok_ok[mt] ? t : 0) * H) + j;
    }
    float4v acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = (float4v){0.f, 0.f, 0.f, 0.f};
    for (int step = 0; step < H / 32; ++step) {
        uint4v b = wrow[step * 4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            uint4v a = tok_ok[mt] ? xrow[mt][step * 4] : (uint4v){0u, 0u, 0u, 0u};
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, b),
                                                              acc[mt], 0, 0, 0);
        }
    }
    const int e = e0 + r;
    const float bb = bias ? bias[e] : 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int t = t0 + mt * 16 + 4 * j + i;
            if (t < T) logits[(size_t)t * E + e] = acc[mt][i] + bb;
        }
    }
}

// grid: ceil(T/4) blocks of 4 waves; wave -> token: radix-selected top-8,
// renormalised weights and the shared-expert gate.
__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ logits,
                                                  const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ wsg, int T,
                                                  int32_t* __restrict__ ids,
                                                  float* __restrict__ wts,
                                                  float* __restrict__ sg) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    wave_top8(logits + (size_t)t * E, ids + (size_t)t * TOPK, wts + (size_t)t * TOPK, nullptr);
    const uint4v* xr = reinterpret_cast<const uint4v*>(x + (size_t)t * H) + lane * 4;
    const uint4v* gr = reinterpret_cast<const uint4v*>(wsg) + lane * 4;
    float z = dot8_bf16(xr[0], gr[0]) + dot8_bf16(xr[1], gr[1]) + dot8_bf16(xr[2], gr[2]) +
              dot8_bf16(xr[3], gr[3]);
    z = wave_sum(z);
    if (lane == 0) sg[t] = 1.f / (1.f + expf(-z));
}

void launch_route_logits(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                         float* logits, hipStream_t st) {
    if (T <= 32) {
        hipLaunchKernelGGL(route_logits_gemv, dim3(E / 4), dim3(256), 0, st, x, T, wr, bias,
                           logits);
    } else {
        hipLaunchKernelGGL(route_logits_mfma, dim3((T + 63) / 64, E / 64), dim3(256), 0, st, x,
                           T, wr, bias, logits);
    }
}

void launch_route(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                  const uint16_t* wsg, float* logits, int32_t* ids, float* wts, float* sg,
                  hipStream_t st) {
    launch_route_logits(x, T, wr, bias, logits, st);
    hipLaunchKernelGGL(route_topk, dim3((T + 3) / 4), dim3(256), 0, st, logits, x, wsg, T, ids,
                       wts, sg);
}

}  // namespace moe
