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
//   route_fused         larger T: one workgroup per 32 tokens computes all
//                       256 logits with bf16 MFMA 32x32x16 (fp32 accumulation
//                       of exact bf16 products), keeps them in LDS and runs
//                       the top-8 selection and the shared gate there.
//   route_logits_mfma   logits only (kept for the split interface path).
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

typedef float float16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rt_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Router for T > 32.  grid: ceil(T/32) workgroups of 8 waves.
//   Logits: wave w owns experts 32w .. 32w+31 for the block's 32 tokens, a
//   32x32 fp32 accumulator of v_mfma_f32_32x32x16_bf16 (lane l: token /
//   expert l%32, k = 8*(l/32)..+7 of each 16-wide step).  K advances in
//   supersteps of 64: the x tile (32 rows) and the W_r tile (256 rows) of
//   the superstep move into LDS with coalesced direct loads (1 KB = 8 rows x
//   128 B per instruction) through a 3-stage ring; rows are stored with
//   their 16-byte pieces XOR-swizzled by (row >> 1) & 7 so a 16-lane operand
//   read hits 16 distinct bank groups.  MFMA step s reads piece 4g + s
//   (g = l/32) of both operands.  Rows past T load zeros (buffer range).
//   Then the 32 x 256 logits (+ bias) go to LDS and each wave selects the top
//   8 of four tokens (wave_top8) and computes their shared gate.
constexpr int RF_TOK = 32;
constexpr int RF_LDS_STRIDE = E + 4;               // floats per token row of logits (16 B aligned)
constexpr int RF_STAGES = 3;
constexpr int RF_XB = RF_TOK * 128;                // x tile bytes per superstep
constexpr int RF_STAGE = RF_XB + E * 128;          // + W_r tile
constexpr int RF_INSTR = RF_STAGE / 1024;          // 1 KB direct loads per superstep (36)
static_assert(RF_STAGE % 1024 == 0, "router stage in whole load instructions");
static_assert(RF_STAGES * RF_STAGE + RF_TOK * RF_LDS_STRIDE * 4 <= 160 * 1024, "router LDS");

typedef __attribute__((address_space(3))) void* rt_lds_t;

// Loads of wave w: instructions j = w, w+8, ... < RF_INSTR (5 for waves 0-3,
// 4 for waves 4-7).
__device__ __forceinline__ int rf_loads(int wave) { return (RF_INSTR - wave + 7) / 8; }

// Instruction j fills stage rows 8j .. 8j+7 (rows 0..31 are x tokens,
// 32..287 W_r experts): lane -> row 8j + lane/8, LDS slot lane%8 holding
// the row's piece slot ^ ((row >> 1) & 7).
__device__ __forceinline__ void rf_issue(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                                         int t0, int wave, int lane, int u, uint8_t* stage) {
#pragma unroll
    for (int i = 0; i < (RF_INSTR + 7) / 8; ++i) {
        const int j = wave + 8 * i;
        if (j >= RF_INSTR) break;
        const int row = 8 * j + (lane >> 3);
        const int p = (lane & 7) ^ ((row >> 1) & 7);
        uint8_t* dst = stage + j * 1024;
        if (j < RF_TOK / 8) {
            const uint32_t off = (uint32_t)(t0 + row) * (H * 2) + (uint32_t)(u * 128 + 16 * p);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (rt_lds_t)dst, 16, off, 0, 0, 0);
        } else {
            const uint32_t off = (uint32_t)(row - RF_TOK) * (H * 2) + (uint32_t)(u * 128 + 16 * p);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (rt_lds_t)dst, 16, off, 0, 0, 0);
        }
    }
}

__global__ __launch_bounds__(512) void route_fused(const uint16_t* __restrict__ x, int T,
                                                   const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   const uint16_t* __restrict__ wsg,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ wts,
                                                   float* __restrict__ sg) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[RF_STAGES * RF_STAGE + RF_TOK * RF_LDS_STRIDE * 4];
    float* lg = reinterpret_cast<float*>(smem + RF_STAGES * RF_STAGE);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int t0 = blockIdx.x * RF_TOK;
    const __amdgpu_buffer_rsrc_t rx = rt_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const __amdgpu_buffer_rsrc_t rw = rt_rsrc(wr, (uint32_t)(E * H * 2));
    constexpr int NU = H / 64;    // 32 supersteps

    static_assert(RF_TOK % 8 == 0, "x rows must fill whole load instructions");
    for (int u = 0; u < RF_STAGES - 1; ++u) rf_issue(rx, rw, t0, wave, lane, u, smem + u * RF_STAGE);

    float16v acc = (float16v)0.f;
    const int ra = l32, rb = RF_TOK + wave * 32 + l32;     // operand rows in the stage
    for (int u = 0; u < NU; ++u) {
        // superstep u landed (the next one may stay in flight), then every
        // wave is done with the stage the refill overwrites
        if (u + 1 < NU && rf_loads(wave) == 5) __builtin_amdgcn_s_waitcnt(vmcnt_imm(5));
        else if (u + 1 < NU) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        pipe_barrier();
        if (u + RF_STAGES - 1 < NU)
            rf_issue(rx, rw, t0, wave, lane, u + RF_STAGES - 1, smem + ((u + RF_STAGES - 1) % RF_STAGES) * RF_STAGE);
        const uint8_t* st = smem + (u % RF_STAGES) * RF_STAGE;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int pc = 4 * g + s;
            const uint4v av = *reinterpret_cast<const uint4v*>(st + ra * 128 + 16 * (pc ^ ((ra >> 1) & 7)));
            const uint4v bv = *reinterpret_cast<const uint4v*>(st + rb * 128 + 16 * (pc ^ ((rb >> 1) & 7)));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
        }
    }

    // logits (+ bias) into LDS: element i is token 8*(i/4) + 4g + i%4
    const int e = wave * 32 + l32;
    const float bb = bias ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) lg[(8 * (i >> 2) + 4 * g + (i & 3)) * RF_LDS_STRIDE + e] = acc[i] + bb;
    __syncthreads();

    // selection and shared gate: wave w handles tokens 4w .. 4w+3
    for (int q = 0; q < RF_TOK / 8; ++q) {
        const int tl = wave * (RF_TOK / 8) + q;
        const int t = t0 + tl;
        if (t >= T) break;
        wave_top8(lg + tl * RF_LDS_STRIDE, ids + (size_t)t * TOPK, wts + (size_t)t * TOPK, nullptr);
        const uint4v* xr = reinterpret_cast<const uint4v*>(x + (size_t)t * H) + lane * 4;
        const uint4v* gr = reinterpret_cast<const uint4v*>(wsg) + lane * 4;
        float z = dot8_bf16(xr[0], gr[0]) + dot8_bf16(xr[1], gr[1]) + dot8_bf16(xr[2], gr[2]) +
                  dot8_bf16(xr[3], gr[3]);
        z = wave_sum(z);
        if (lane == 0) sg[t] = 1.f / (1.f + expf(-z));
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
    if (T > 32) {
        hipLaunchKernelGGL(route_fused, dim3((T + RF_TOK - 1) / RF_TOK), dim3(512), 0, st, x, T, wr,
                           bias, wsg, ids, wts, sg);
        return;
    }
    launch_route_logits(x, T, wr, bias, logits, st);
    hipLaunchKernelGGL(route_topk, dim3((T + 3) / 4), dim3(256), 0, st, logits, x, wsg, T, ids,
                       wts, sg);
}

}  // namespace moe
