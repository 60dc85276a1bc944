// greedy.hip -- greedy next-token selection after the last layer, kept on
// the GPU for the next decode step ("Perplexity Open-Sources Lily ...",
// section "Generation has a different bottleneck"), and the embedding lookup
// that turns the selected token into the next step's input row.
//
//   head_argmax_part   output-head GEMV (bf16 [V][2048] head, fp32
//                      accumulation of exact bf16 products) with a running
//                      maximum per token: every workgroup reduces its rows
//                      to one 64-bit key per token, (order-preserving key of
//                      the fp32 logit) << 32 | (0xFFFFFFFF - v), so the
//                      largest key is the largest logit and, among equal
//                      logits, the lowest token -- and a maximum does not
//                      depend on the order it is taken in (deterministic)
//   head_argmax_final  one workgroup: the maximum of the workgroups' keys
//   embed_rows         x[t] = emb[token[t]] (zeros for a token outside the
//                      table)
//
// The head GEMV reads V x 4 KB once: it is bound by HBM bandwidth.  Each
// wave takes one row at a time (four 16-byte loads per lane, each covering
// 1 KB of the row over the wave), four rows in flight, all tokens'
// activations in registers.
#include "block_util.hpp"

namespace moe {

constexpr int HD_WG = 1024;       // head workgroups (4 waves each)
constexpr int HD_ROWS = 4;        // rows per wave in flight

__device__ __forceinline__ unsigned long long head_key(float logit, int v) {
    return ((unsigned long long)fkey(logit) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)v);
}

// grid HD_WG x 256 threads.  Workgroup b takes the contiguous block of rows
// [b R, (b+1) R), R = ceil(V / HD_WG), so its reads stay within one or two
// pages of the table; wave w the rows b R + w + 4 i.  part[b][t] = its key
// for token t.
template <int TT>
__global__ __launch_bounds__(256) void head_argmax_part(const uint16_t* __restrict__ x, int T,
                                                        const uint16_t* __restrict__ w, int V,
                                                        unsigned long long* __restrict__ part) {
    __shared__ unsigned long long best_w[4][TT];
    const int lane = threadIdx.x & 63, wave = wave_id();
    // this lane's 32 activations of every token, as fp32: elements
    // 512 c + 8 lane .. 512 c + 8 lane + 7, c = 0..3 (each of a row's four
    // 16-byte loads then covers 1 KB of the row contiguously over the wave)
    float xv[TT][32];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const uint4v* xr = reinterpret_cast<const uint4v*>(x + (size_t)min(t, T - 1) * H) + lane;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4v a = xr[64 * c];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xv[t][8 * c + 2 * i] = bf16_to_f32(a[i] & 0xFFFFu);
                xv[t][8 * c + 2 * i + 1] = bf16_to_f32(a[i] >> 16);
            }
        }
    }
    unsigned long long best[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) best[t] = 0ull;
    const int R = (V + HD_WG - 1) / HD_WG;
    const int rb = blockIdx.x * R, re = min(rb + R, V);
    const int stride = 4;                               // rows per round over the waves
    for (int r0 = rb + wave; r0 < re; r0 += stride * HD_ROWS) {
        uint4v wv[HD_ROWS][4];
#pragma unroll
        for (int j = 0; j < HD_ROWS; ++j) {
            const int r = min(r0 + j * stride, V - 1);
            const uint4v* wr = reinterpret_cast<const uint4v*>(w + (size_t)r * H) + lane;
#pragma unroll
            for (int c = 0; c < 4; ++c) wv[j][c] = __builtin_nontemporal_load(wr + 64 * c);
        }
#pragma unroll
        for (int j = 0; j < HD_ROWS; ++j) {
            const int r = r0 + j * stride;
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if (t >= T) continue;
                float s = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t b = wv[j][c][i];
                        s = fmaf(xv[t][8 * c + 2 * i], __builtin_bit_cast(float, b << 16), s);
                        s = fmaf(xv[t][8 * c + 2 * i + 1], __builtin_bit_cast(float, b & 0xFFFF0000u), s);
                    }
                s = wave_sum(s);
                if (r < re) {
                    const unsigned long long k = head_key(s, r);
                    best[t] = k > best[t] ? k : best[t];
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
        if (lane == 0) best_w[wave][t] = best[t];
    __syncthreads();
    if ((int)threadIdx.x < T) {
        unsigned long long k = best_w[0][threadIdx.x];
#pragma unroll
        for (int q = 1; q < 4; ++q) k = best_w[q][threadIdx.x] > k ? best_w[q][threadIdx.x] : k;
        part[(size_t)blockIdx.x * TT + threadIdx.x] = k;
    }
}

// one workgroup of 256 threads: token[t] from the HD_WG keys of token t.
template <int TT>
__global__ __launch_bounds__(256) void head_argmax_final(const unsigned long long* __restrict__ part,
                                                         int T, int32_t* __restrict__ token) {
    __shared__ unsigned long long red[256];
    for (int t = 0; t < T; ++t) {
        unsigned long long k = 0ull;
        for (int b = threadIdx.x; b < HD_WG; b += 256) {
            const unsigned long long v = part[(size_t)b * TT + t];
            k = v > k ? v : k;
        }
        red[threadIdx.x] = k;
        __syncthreads();
        for (int s = 128; s > 0; s >>= 1) {
            if ((int)threadIdx.x < s) {
                const unsigned long long o = red[threadIdx.x + s];
                red[threadIdx.x] = o > red[threadIdx.x] ? o : red[threadIdx.x];
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) token[t] = (int32_t)(0xFFFFFFFFu - (uint32_t)(red[0] & 0xFFFFFFFFull));
        __syncthreads();
    }
}

// grid T x 256 threads: row token[t] of the table (16 bytes per thread).
__global__ __launch_bounds__(256) void embed_rows(const int32_t* __restrict__ token,
                                                  const uint16_t* __restrict__ emb, int V,
                                                  uint16_t* __restrict__ x) {
    const int t = blockIdx.x;
    const int v = token[t];
    uint4v r = {0u, 0u, 0u, 0u};
    if (v >= 0 && v < V) r = reinterpret_cast<const uint4v*>(emb + (size_t)v * H)[threadIdx.x];
    reinterpret_cast<uint4v*>(x + (size_t)t * H)[threadIdx.x] = r;
}

size_t head_part_bytes() { return (size_t)HD_WG * MOE_DECODE_T * sizeof(unsigned long long); }

void launch_head_argmax(const uint16_t* x, int T, const uint16_t* w, int V, int32_t* token,
                        unsigned long long* part, hipStream_t st) {
    if (T == 1) {
        hipLaunchKernelGGL(head_argmax_part<1>, dim3(HD_WG), dim3(256), 0, st, x, T, w, V, part);
        hipLaunchKernelGGL(head_argmax_final<1>, dim3(1), dim3(256), 0, st, part, T, token);
    } else {
        hipLaunchKernelGGL(head_argmax_part<MOE_DECODE_T>, dim3(HD_WG), dim3(256), 0, st, x, T, w, V,
                           part);
        hipLaunchKernelGGL(head_argmax_final<MOE_DECODE_T>, dim3(1), dim3(256), 0, st, part, T,
                           token);
    }
}

void launch_embed(const int32_t* token, int T, const uint16_t* emb, int V, uint16_t* x,
                  hipStream_t st) {
    hipLaunchKernelGGL(embed_rows, dim3(T), dim3(256), 0, st, token, emb, V, x);
}

}  // namespace moe
