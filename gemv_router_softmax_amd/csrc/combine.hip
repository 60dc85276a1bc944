// combine.hip -- weighted un-permute plus the shared expert, and the
// read/copy probes used to measure the sustained HBM rate.
#include "common.hpp"

namespace moe {

// y[t] = bf16( sum_j w[t][j] out[inv[8t+j]] + sg[t] out[8T+t] ); optionally
// res[t] = bf16( x[t] + y[t] ).  One thread per 4 columns; grid (T, H/1024).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ wts,
                                                      const float* __restrict__ sg, int T,
                                                      uint16_t* __restrict__ y,
                                                      const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ res) {
    const int t = blockIdx.x;
    const int m = (blockIdx.y * 256 + threadIdx.x) * 4;
    float4v acc = (float4v){0.f, 0.f, 0.f, 0.f};
    // (every row's load in flight at once; an entry out of range reads row
    // 0 and adds nothing)
    float4v dv[TOPK];
    float wv[TOPK];
    bool ok[TOPK];
#pragma unroll
    for (int j = 0; j < TOPK; ++j) {
        const int p = inv[(size_t)t * TOPK + j];
        ok[j] = p >= 0 && p < TOPK * T;
        wv[j] = wts[(size_t)t * TOPK + j];
        dv[j] = *reinterpret_cast<const float4v*>(out + (size_t)(ok[j] ? p : 0) * H + m);
    }
#pragma unroll
    for (int j = 0; j < TOPK; ++j)
        if (ok[j]) acc += wv[j] * dv[j];
    {
        const float4v d = *reinterpret_cast<const float4v*>(out + ((size_t)TOPK * T + t) * H + m);
        acc += sg[t] * d;
    }
    uint32_t yb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) yb[i] = f32_to_bf16(acc[i]);
    uint2 yv;
    yv.x = yb[0] | (yb[1] << 16);
    yv.y = yb[2] | (yb[3] << 16);
    *reinterpret_cast<uint2*>(y + (size_t)t * H + m) = yv;
    if (res) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)t * H + m);
        const uint32_t xs[4] = {xv.x & 0xFFFFu, xv.x >> 16, xv.y & 0xFFFFu, xv.y >> 16};
        uint32_t rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = f32_to_bf16(bf16_to_f32(xs[i]) + bf16_to_f32(yb[i]));
        uint2 rv;
        rv.x = rb[0] | (rb[1] << 16);
        rv.y = rb[2] | (rb[3] << 16);
        *reinterpret_cast<uint2*>(res + (size_t)t * H + m) = rv;
    }
}

// Prefill combine: y[t] = bf16( sum_j d16[inv[8t+j]] + d16[8T+t] ), the rows
// already scaled by their routing weight / shared gate (fp16), summed in fp32
// in a fixed order; optionally res = bf16(x + y).  grid (T, H/2048), one
// thread per 8 columns.
__global__ __launch_bounds__(256) void combine_f16_kernel(const uint16_t* __restrict__ d16,
                                                          const int32_t* __restrict__ inv, int T,
                                                          uint16_t* __restrict__ y,
                                                          const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ res) {
    const int t = blockIdx.x;
    const int m = threadIdx.x * 8;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    int rows[TOPK + 1];
#pragma unroll
    for (int jj = 0; jj < TOPK; ++jj) rows[jj] = inv[(size_t)t * TOPK + jj];
    rows[TOPK] = TOPK * T + t;
    // all nine rows in flight at once (a load under a condition was waited
    // for before the next was issued); an entry out of range reads row 0
    // and adds nothing
    uint4v rv[TOPK + 1];
    bool ok[TOPK + 1];
#pragma unroll
    for (int jj = 0; jj <= TOPK; ++jj) {
        ok[jj] = rows[jj] >= 0 && rows[jj] < (TOPK + 1) * T;
        rv[jj] = *reinterpret_cast<const uint4v*>(d16 + (size_t)(ok[jj] ? rows[jj] : 0) * H + m);
    }
#pragma unroll
    for (int jj = 0; jj <= TOPK; ++jj) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t w = rv[jj][k >> 1];
            const uint16_t hb = (uint16_t)((k & 1) ? (w >> 16) : (w & 0xFFFFu));
            if (ok[jj]) acc[k] += (float)__builtin_bit_cast(_Float16, hb);
        }
    }
    uint4v yo, ro;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t y0 = f32_to_bf16(acc[2 * i]), y1 = f32_to_bf16(acc[2 * i + 1]);
        yo[i] = y0 | (y1 << 16);
        if (res) {
            const uint32_t xv = reinterpret_cast<const uint32_t*>(x + (size_t)t * H + m)[i];
            const uint32_t r0 = f32_to_bf16(bf16_to_f32(xv & 0xFFFFu) + bf16_to_f32(y0));
            const uint32_t r1 = f32_to_bf16(bf16_to_f32(xv >> 16) + bf16_to_f32(y1));
            ro[i] = r0 | (r1 << 16);
        }
    }
    *reinterpret_cast<uint4v*>(y + (size_t)t * H + m) = yo;
    if (res) *reinterpret_cast<uint4v*>(res + (size_t)t * H + m) = ro;
}

void launch_combine_f16(const uint16_t* d16, const int32_t* inv, int T, uint16_t* y,
                        const uint16_t* x, uint16_t* res, hipStream_t st) {
    hipLaunchKernelGGL(combine_f16_kernel, dim3(T), dim3(256), 0, st, d16, inv, T, y, x, res);
}

void launch_combine(const float* out, const int32_t* inv, const float* wts, const float* sg, int T,
                    uint16_t* y, const uint16_t* x, uint16_t* res, hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3(T, H / 1024), dim3(256), 0, st, out, inv, wts, sg, T,
                       y, x, res);
}

// ------------------------------------------------------------------ probes

constexpr int PROBE_BLOCKS = 4096;

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4v* __restrict__ src,
                                                         size_t n16, float* __restrict__ sink) {
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * 256) {
        const uint4v v = __builtin_nontemporal_load(src + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // a data-dependent (practically never taken) store keeps the loads alive
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = (float)threadIdx.x;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(uint4v* __restrict__ dst,
                                                         const uint4v* __restrict__ src,
                                                         size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * 256)
        dst[i] = src[i];
}

void launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t st) {
    hipLaunchKernelGGL(probe_read_kernel, dim3(PROBE_BLOCKS), dim3(256), 0, st,
                       reinterpret_cast<const uint4v*>(src), bytes / 16, sink);
}

void launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
    hipLaunchKernelGGL(probe_copy_kernel, dim3(PROBE_BLOCKS), dim3(256), 0, st,
                       reinterpret_cast<uint4v*>(dst), reinterpret_cast<const uint4v*>(src),
                       bytes / 16);
}

}  // namespace moe
