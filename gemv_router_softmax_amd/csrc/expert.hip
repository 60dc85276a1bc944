// expert.hip -- SwiGLU expert FFNs with 4-bit weights dequantised inside the
// kernels (the weights are never expanded in memory: "Perplexity Open-Sources
// Lily ...", section "The optimizations follow the workload"; "A Rust + Metal
// Inference Engine for Qwen3.6-35B-A3B on Apple Silicon", paragraph 4).
//
// Work is described by the row-tile list built on the device (plan_tiles):
// tile = (expert or shared group, first row, row count <= 128).
//
// Decode (few tokens; the gate/up GEMV and the fused down+combine kernel
// live in decode.hip):
//   decode_down    16 lanes per output row (16 B of codes each), 4 rows per
//                  wave; exact codes through v_dot2_f32_bf16 (dot8_codes),
//                  group scale/bias applied once per lane; writes the fp32
//                  expert rows of the split expert-FFN call.
//
// Prefill (grouped GEMM on MFMA):
//   expert_mfma<2048, true>   gate/up: tile rows x 128 columns of gate and up
//   expert_mfma<512, false>   down:    tile rows x 256 output columns
//   A (activations) is staged in LDS per 128-wide K chunk, already fp16 and
//   in the chunk-slot order the dequantiser produces.  Each wave owns 64
//   weight columns for all tile rows; its lanes load 16 B of codes per
//   column per K chunk straight into registers, rebuild fp16 weights
//   w = q*s + b with packed half arithmetic (one rounding), and feed
//   v_mfma_f32_16x16x32_f16 with fp32 accumulation.  SwiGLU and the bf16
//   rounding of h are fused into the gate/up epilogue.
#include "common.hpp"

namespace moe {

constexpr int AST = 136;   // LDS row stride of the A tile, in halves (128 + 8)

__device__ __forceinline__ int row_token(int row, int T, const int32_t* __restrict__ perm) {
    if (row < TOPK * T) {
        int t = perm[row] >> 3;
        return min(max(t, 0), T - 1);
    }
    return row - TOPK * T;
}

// ------------------------------------------------------------------ decode

__global__ __launch_bounds__(256) void decode_down(const uint16_t* __restrict__ hin, int T,
                                                   const Tile* __restrict__ tiles,
                                                   const int* __restrict__ tile_count,
                                                   moe_qffn routed, moe_qffn shared,
                                                   float* __restrict__ out) {
    if ((int)blockIdx.x >= *tile_count) return;
    const Tile tl = tiles[blockIdx.x];
    const bool sh = tl.group >= E;
    const int e = sh ? 0 : tl.group;
    const moe_qffn q = sh ? shared : routed;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int m = blockIdx.y * 16 + (threadIdx.x >> 6) * 4 + (lane >> 4);
    const size_t row = (size_t)e * H + m;
    const uint4v dw = reinterpret_cast<const uint4v*>(q.down_q + row * (I / 8))[c];
    const float s = fp16_to_f32(q.down_s[row * (I / G) + (c >> 1)]);
    const float b = fp16_to_f32(q.down_b[row * (I / G) + (c >> 1)]);
    for (int rr = 0; rr < tl.nrows; ++rr) {
        // h rows are fp16 in chunk-slot order (decode_gateup)
        const uint4v* hr = reinterpret_cast<const uint4v*>(hin + (size_t)(tl.row0 + rr) * I) + c * 4;
        float sh_ = 0.f, dot = 0.f;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const uint4v hv = hr[cc];
            sh_ = sum8_h(hv, sh_);
            dot = dot8_codes(dw[cc], hv, dot);
        }
        float p = fmaf(s, dot, b * sh_);
        p += __shfl_xor(p, 8, WAVE);
        p += __shfl_xor(p, 4, WAVE);
        p += __shfl_xor(p, 2, WAVE);
        p += __shfl_xor(p, 1, WAVE);
        if (c == 0) out[(size_t)(tl.row0 + rr) * H + m] = p;
    }
}

// ----------------------------------------------------------------- prefill

__device__ __forceinline__ half2v splat_h(uint16_t bits) {
    const _Float16 h = __builtin_bit_cast(_Float16, bits);
    return (half2v){h, h};
}

// Eight codes of one word -> fp16 weights w = q*s + b, in chunk-slot order
// (k = 0,4,1,5,2,6,3,7).  (0x6400 | q) is the fp16 value 1024 + q, so one
// packed subtraction recovers q exactly and one packed FMA applies the
// group's scale and bias with a single rounding.
__device__ __forceinline__ half8 dequant8(uint32_t w, half2v s2, half2v b2) {
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
        half2v h = __builtin_bit_cast(half2v, p) - (half2v){(_Float16)1024.f, (_Float16)1024.f};
        h = __builtin_elementwise_fma(h, s2, b2);
        r[2 * i] = h[0];
        r[2 * i + 1] = h[1];
    }
    return r;
}

template <int KDIM, bool GATEUP>
__global__ __launch_bounds__(256, 1) void expert_mfma(const uint16_t* __restrict__ ain, int T,
                                                      const int32_t* __restrict__ perm,
                                                      const Tile* __restrict__ tiles,
                                                      const int* __restrict__ tile_count,
                                                      moe_qffn routed, moe_qffn shared,
                                                      uint16_t* __restrict__ hout,
                                                      float* __restrict__ dout) {
    constexpr int NCH = KDIM / 128;              // K chunks
    constexpr int WPR = KDIM / 8;                // code words per weight row
    constexpr int SPR = KDIM / G;                // groups per weight row
    constexpr int ROWS_W = GATEUP ? I : H;       // weight rows per expert
    __shared__ __attribute__((aligned(16))) uint16_t As[MT_ROWS * AST];

    if ((int)blockIdx.x >= *tile_count) return;
    const Tile tl = tiles[blockIdx.x];
    const bool sh = tl.group >= E;
    const int e = sh ? 0 : tl.group;
    const moe_qffn q = sh ? shared : routed;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, j = lane >> 4;
    const int nr = tl.nrows, n_mt = (nr + 15) >> 4;

    // This lane's weight row in each of the wave's four 16-column tiles.
    const uint32_t* wq[4];
    const uint16_t* wsc[4];
    const uint16_t* wbi[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        int n;
        const uint32_t* qb;
        const uint16_t *sb, *bb;
        if (GATEUP) {
            n = blockIdx.y * 128 + wave * 32 + (nt & 1) * 16 + r;
            qb = nt < 2 ? q.gate_q : q.up_q;
            sb = nt < 2 ? q.gate_s : q.up_s;
            bb = nt < 2 ? q.gate_b : q.up_b;
        } else {
            n = blockIdx.y * 256 + wave * 64 + nt * 16 + r;
            qb = q.down_q;
            sb = q.down_s;
            bb = q.down_b;
        }
        const size_t row = (size_t)e * ROWS_W + n;
        wq[nt] = qb + row * WPR + 4 * j;
        wsc[nt] = sb + row * SPR + (j >> 1);
        wbi[nt] = bb + row * SPR + (j >> 1);
    }

    // A rows this thread stages: row (tid>>4) + 16 i, 16-byte column tid&15.
    const uint16_t* asrc[8];
    bool aok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 4) + 16 * i;
        aok[i] = row < nr;
        const int rr = aok[i] ? row : 0;
        if (GATEUP)
            asrc[i] = ain + (size_t)row_token(tl.row0 + rr, T, perm) * H + (tid & 15) * 8;
        else
            asrc[i] = ain + (size_t)(tl.row0 + rr) * I + (tid & 15) * 8;
    }

    float4v acc[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (float4v){0.f, 0.f, 0.f, 0.f};

    uint4v bw[4];
    half2v bs[4], bb[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        bw[nt] = *reinterpret_cast<const uint4v*>(wq[nt]);
        bs[nt] = splat_h(wsc[nt][0]);
        bb[nt] = splat_h(wbi[nt][0]);
    }

    for (int kc = 0; kc < NCH; ++kc) {
        uint4v cw[4];
        half2v cs[4], cb[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) { cw[nt] = bw[nt]; cs[nt] = bs[nt]; cb[nt] = bb[nt]; }
        if (kc + 1 < NCH) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                bw[nt] = *reinterpret_cast<const uint4v*>(wq[nt] + (kc + 1) * 16);
                bs[nt] = splat_h(wsc[nt][(kc + 1) * 2]);
                bb[nt] = splat_h(wbi[nt][(kc + 1) * 2]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint4v v = (uint4v){0u, 0u, 0u, 0u};
            if (aok[i]) v = *reinterpret_cast<const uint4v*>(asrc[i] + kc * 128);
            *reinterpret_cast<uint4v*>(&As[((tid >> 4) + 16 * i) * AST + (tid & 15) * 8]) = v;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8 bf[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) bf[nt] = dequant8(cw[nt][s], cs[nt], cb[nt]);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                if (mt < n_mt) {
                    const half8 a =
                        *reinterpret_cast<const half8*>(&As[(mt * 16 + r) * AST + 32 * j + 8 * s]);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[mt][nt] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[nt], acc[mt][nt], 0, 0, 0);
                }
            }
        }
    }

    if (GATEUP) {
        // h = bf16(silu(g) * u), stored as fp16 (exact) in chunk-slot order so
        // the down kernel can stage it without conversion.
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            if (mt < n_mt) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = mt * 16 + 4 * j + i;
                        const int col = wave * 32 + nt * 16 + r;
                        const float g = acc[mt][nt][i], u = acc[mt][nt + 2][i];
                        const float hv = (g / (1.f + expf(-g))) * u;
                        const _Float16 hh = (_Float16)bf16_to_f32(f32_to_bf16(hv));
                        As[row * AST + (col & ~7) + chunk_slot(col & 7)] =
                            __builtin_bit_cast(uint16_t, hh);
                    }
                }
            }
        }
        __syncthreads();
        for (int c = tid; c < nr * 16; c += 256) {
            const int row = c >> 4, col = (c & 15) * 8;
            *reinterpret_cast<uint4v*>(hout + (size_t)(tl.row0 + row) * I + blockIdx.y * 128 + col) =
                *reinterpret_cast<const uint4v*>(&As[row * AST + col]);
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            if (mt < n_mt) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = mt * 16 + 4 * j + i;
                        if (row < nr)
                            dout[(size_t)(tl.row0 + row) * H + blockIdx.y * 256 + wave * 64 +
                                 nt * 16 + r] = acc[mt][nt][i];
                    }
                }
            }
        }
    }
}

// x (bf16) -> fp16 in chunk-slot order, the activation layout of the expert kernels.
__global__ __launch_bounds__(256) void prep_x_f16(const uint16_t* __restrict__ x, int T,
                                                  uint16_t* __restrict__ xh) {
    const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;   // 8-element chunk index
    if (c >= (size_t)T * (H / 8)) return;
    reinterpret_cast<uint4v*>(xh)[c] = bf16x8_to_f16_slots(reinterpret_cast<const uint4v*>(x)[c]);
}

void launch_decode_gateup(const uint16_t* xh, int T, const int32_t* perm, const Tile* tiles,
                          const int* tile_count, int max_tiles, const moe_qffn& routed,
                          const moe_qffn& shared, uint16_t* hbuf, hipStream_t st);

void launch_expert_decode(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                          const int* tile_count, int max_tiles, const moe_qffn& routed,
                          const moe_qffn& shared, uint16_t* xh, uint16_t* hbuf, float* dout,
                          hipStream_t st) {
    const size_t chunks = (size_t)T * (H / 8);
    hipLaunchKernelGGL(prep_x_f16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, x, T,
                       xh);
    launch_decode_gateup(xh, T, perm, tiles, tile_count, max_tiles, routed, shared, hbuf, st);
    hipLaunchKernelGGL(decode_down, dim3(max_tiles, H / 16), dim3(256), 0, st, hbuf, T, tiles,
                       tile_count, routed, shared, dout);
}

void launch_expert_prefill(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                           const int* tile_count, int max_tiles, const moe_qffn& routed,
                           const moe_qffn& shared, uint16_t* xh, uint16_t* hbuf, float* dout,
                           hipStream_t st) {
    const size_t chunks = (size_t)T * (H / 8);
    hipLaunchKernelGGL(prep_x_f16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, x, T,
                       xh);
    hipLaunchKernelGGL((expert_mfma<H, true>), dim3(max_tiles, I / 128), dim3(256), 0, st, xh, T,
                       perm, tiles, tile_count, routed, shared, hbuf, (float*)nullptr);
    hipLaunchKernelGGL((expert_mfma<I, false>), dim3(max_tiles, H / 256), dim3(256), 0, st, hbuf,
                       T, perm, tiles, tile_count, routed, shared, (uint16_t*)nullptr, dout);
}

}  // namespace moe
