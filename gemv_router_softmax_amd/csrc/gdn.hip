// gdn.hip -- chunked scan of the gated delta rule (the recurrent layers of
// the model the pages describe), on fp16 MFMA with the state in registers.
//
// The pages say the engine holds the recurrent scan of the model's Gated
// DeltaNet layers in registers ("leslieli.dev note on the Perplexity Lily
// engine", paragraph 3; "Perplexity Open-Sources Lily ...", section "A
// runtime shaped around one model") but do not define the recurrence.
// This file computes the published gated delta rule (Yang, Kautz,
// Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule"),
// per value head h with key head h / (hv / hk), S (128 x 128) the state:
//
//   S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
//
// Over a chunk of n <= 64 tokens with cumulative log decay gam_i and b_i =
// e^{gam_i}, unrolling the recurrence from the state S0 entering the chunk
// gives the chunk's corrected values U (n x 128) as the solution of
//   (I + L) U = diag(beta) V - diag(beta b) K S0^T,
//   L_ij = beta_i e^{gam_i - gam_j} k_i . k_j   (j < i),
// so with T = (I + L)^{-1}, Ut = T diag(beta) V and W = T diag(beta b) K:
//   U  = Ut - W S0^T
//   O  = diag(b) Q S0^T + A U,      A_ij = e^{gam_i - gam_j} q_i . k_j  (j <= i)
//   S1 = b_n S0 + U^T diag(e^{gam_n - gam}) K.
// Everything that does not involve S0 is independent across chunks:
//
//   gdn_prep  grid (chunks, hv): per chunk and head, K K^T and Q K^T on
//             MFMA, the masks and decays, T by forward substitution (fp32,
//             one quad of lanes per column), Ut and W on MFMA; writes Ut
//             (fp32), W and A (fp16) and gam to the workspace.
//   gdn_scan  grid (hv, 4): one workgroup per head and 32-row slice of the
//             state (rows are value channels, independent of one another).
//             The slice (32 x 128 fp32) stays in the four waves' MFMA
//             accumulators for the whole sequence; per chunk it is staged
//             once to LDS as fp16 for the products S0^T, the chunk's inputs
//             having been fetched into registers during the previous chunk.
//
// Precision: products on v_mfma_f32_32x32x16_f16 (fp32 accumulation);
// q, k, v are bf16 inputs converted to fp16 (exact within fp16's range);
// beta v, beta b k, T, W, A, U and the staged state are rounded to fp16 as
// MFMA operands; the state, Ut and every accumulation stay fp32.
#include "common.hpp"

namespace moe {

constexpr int GD = MOE_GDN_DIM;       // 128: key and value head dimension
constexpr int GC = MOE_GDN_CHUNK;     // 64 tokens per chunk
constexpr int LD_D = GD + 8;          // LDS row stride (halves) of 128-wide fp16 rows
constexpr int LD_C = GC + 8;          // LDS row stride (halves) of 64-wide fp16 rows
// workspace block of one (chunk, head): Ut fp32 [64][128], W fp16 [64][128],
// A fp16 [64][64], gam fp32 [64]
constexpr size_t GW_UT = 0, GW_W = GW_UT + GC * GD * 4, GW_A = GW_W + GC * GD * 2,
                 GW_GAM = GW_A + GC * GC * 2, GW_BLK = GW_GAM + GC * 4;
static_assert(GW_BLK % 256 == 0, "workspace blocks stay 256-byte aligned");

typedef float float16v __attribute__((ext_vector_type(16)));

// acc += A x B^T for a 32 x 32 tile: A = 32 rows at a, B = 32 rows at b,
// both fp16 row-major in LDS (row strides lda, ldb halves), K a multiple
// of 16.  v_mfma_f32_32x32x16_f16: lane l supplies row l%32 of each
// operand, k = 8 (l/32) .. +7 of every 16-wide step; accumulator element e
// of lane l is row 8 (e/4) + 4 (l/32) + e%4, column l%32.
template <int K>
__device__ __forceinline__ void mma_rows(const _Float16* a, int lda, const _Float16* b, int ldb,
                                         float16v& acc) {
    const int l = threadIdx.x & 63, r = l & 31, kh = (l >> 5) * 8;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        const half8 av = *reinterpret_cast<const half8*>(a + r * lda + k0 + kh);
        const half8 bv = *reinterpret_cast<const half8*>(b + r * ldb + k0 + kh);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ int acc_row(int e, int l) { return 8 * (e >> 2) + 4 * (l >> 5) + (e & 3); }

// eight bf16 -> eight fp16 (through fp32; exact within fp16's normal range)
__device__ __forceinline__ half8 bf16x8_to_h8(uint4v w) {
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = (_Float16)bf16_to_f32(w[i] & 0xFFFFu);
        r[2 * i + 1] = (_Float16)bf16_to_f32(w[i] >> 16);
    }
    return r;
}

struct GdnArgs {
    const uint16_t *q, *k, *v;   // bf16 [T][hk][128], [T][hk][128], [T][hv][128]
    const float *g, *beta;       // fp32 [T][hv]
    const float* s0;             // fp32 [hv][128][128] or null
    uint16_t* o;                 // bf16 [T][hv][128]
    float* s_out;                // fp32 [hv][128][128] or null
    uint8_t* ws;                 // chunks x hv blocks of GW_BLK bytes
    int T, hk, hv;
};

// ------------------------------------------------------------------ prep

__global__ __launch_bounds__(256) void gdn_prep(GdnArgs p) {
    __shared__ __attribute__((aligned(16))) _Float16 Ks[GC * LD_D], Qs[GC * LD_D];
    __shared__ __attribute__((aligned(16))) _Float16 VbT[GD * LD_C], KbT[GD * LD_C], Ts[GC * LD_C];
    __shared__ __attribute__((aligned(16))) float Lp[GC * GC];   // row i: L[i][4q+s] at s*16+q
    __shared__ float gam[GC], bet[GC];
    const int c = blockIdx.x, h = blockIdx.y;
    const int kh = h / (p.hv / p.hk);
    const int t0 = c * GC, n = min(GC, p.T - t0);
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    uint8_t* blk = p.ws + ((size_t)c * p.hv + h) * GW_BLK;

    // cumulative log decay over the chunk (tokens past n: g = 0, beta = 0)
    if (w == 0) {
        float x = l < n ? p.g[(size_t)(t0 + l) * p.hv + h] : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(x, o, 64);
            if (l >= o) x += y;
        }
        gam[l] = x;
        bet[l] = l < n ? p.beta[(size_t)(t0 + l) * p.hv + h] : 0.f;
        reinterpret_cast<float*>(blk + GW_GAM)[l] = x;
    }
    __syncthreads();
    // K, Q rows as fp16; beta v and beta b k transposed ([channel][token])
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) {
        const int idx = pi * 256 + tid, i = idx >> 4, c8 = (idx & 15) * 8;
        uint4v kw = {0, 0, 0, 0}, qw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
        if (i < n) {
            kw = *reinterpret_cast<const uint4v*>(p.k + ((size_t)(t0 + i) * p.hk + kh) * GD + c8);
            qw = *reinterpret_cast<const uint4v*>(p.q + ((size_t)(t0 + i) * p.hk + kh) * GD + c8);
            vw = *reinterpret_cast<const uint4v*>(p.v + ((size_t)(t0 + i) * p.hv + h) * GD + c8);
        }
        const half8 kv = bf16x8_to_h8(kw);
        *reinterpret_cast<half8*>(Ks + i * LD_D + c8) = kv;
        *reinterpret_cast<half8*>(Qs + i * LD_D + c8) = bf16x8_to_h8(qw);
        const float bv = bet[i], bk = bet[i] * __expf(gam[i]);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            VbT[(c8 + 2 * x) * LD_C + i] = (_Float16)(bv * bf16_to_f32(vw[x] & 0xFFFFu));
            VbT[(c8 + 2 * x + 1) * LD_C + i] = (_Float16)(bv * bf16_to_f32(vw[x] >> 16));
            KbT[(c8 + 2 * x) * LD_C + i] = (_Float16)(bk * bf16_to_f32(kw[x] & 0xFFFFu));
            KbT[(c8 + 2 * x + 1) * LD_C + i] = (_Float16)(bk * bf16_to_f32(kw[x] >> 16));
        }
    }
    __syncthreads();
    // K K^T and Q K^T: wave w owns the 32 x 32 tile (w/2, w%2)
    {
        const int ti = w >> 1, tj = w & 1;
        float16v aG = (float16v)0.f, aQ = (float16v)0.f;
        mma_rows<GD>(Ks + 32 * ti * LD_D, LD_D, Ks + 32 * tj * LD_D, LD_D, aG);
        mma_rows<GD>(Qs + 32 * ti * LD_D, LD_D, Ks + 32 * tj * LD_D, LD_D, aQ);
        _Float16* Aw = reinterpret_cast<_Float16*>(blk + GW_A);
        const int j = 32 * tj + (l & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = 32 * ti + acc_row(e, l);
            const float d = j <= i ? __expf(gam[i] - gam[j]) : 0.f;
            Lp[i * GC + (j & 3) * 16 + (j >> 2)] = j < i ? bet[i] * d * aG[e] : 0.f;
            Aw[i * GC + j] = (_Float16)(d * aQ[e]);
        }
    }
    __syncthreads();
    // T = (I + L)^{-1}, L strictly lower: column m by the quad of lanes
    // 4m .. 4m+3, lane s holding rows 4q + s (q = 0..15) in registers;
    // row i: T[i][m] = [i == m] - sum_{j<i} L[i][j] T[j][m] (the rows j >= i
    // are still zero, as are L's entries there)
    {
        const int m = tid >> 2, s = tid & 3;
        float tq[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) tq[q] = 0.f;
#pragma unroll
        for (int i = 0; i < GC; ++i) {
            const float4v* lr = reinterpret_cast<const float4v*>(Lp + i * GC + s * 16);
            float part = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float4v lv = lr[b];
#pragma unroll
                for (int x = 0; x < 4; ++x) part = fmaf(lv[x], tq[4 * b + x], part);
            }
            part += dpp_f<DPP_XOR1>(part);
            part += dpp_f<DPP_XOR2>(part);
            const float tim = (i == m ? 1.f : 0.f) - part;
            if (s == (i & 3)) tq[i >> 2] = tim;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) Ts[(4 * q + s) * LD_C + m] = (_Float16)tq[q];
    }
    __syncthreads();
    // Ut = T (beta V) and W = T (beta b K): wave w owns row tile w/2 and
    // column tiles 2 (w%2), 2 (w%2) + 1 of both
    {
        const int ti = w >> 1;
        float* Ut = reinterpret_cast<float*>(blk + GW_UT);
        _Float16* Ww = reinterpret_cast<_Float16*>(blk + GW_W);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tc = 2 * (w & 1) + u;
            float16v aU = (float16v)0.f, aW = (float16v)0.f;
            mma_rows<GC>(Ts + 32 * ti * LD_C, LD_C, VbT + 32 * tc * LD_C, LD_C, aU);
            mma_rows<GC>(Ts + 32 * ti * LD_C, LD_C, KbT + 32 * tc * LD_C, LD_C, aW);
            const int col = 32 * tc + (l & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = 32 * ti + acc_row(e, l);
                Ut[i * GD + col] = aU[e];
                Ww[i * GD + col] = (_Float16)aW[e];
            }
        }
    }
}

// ------------------------------------------------------------------ scan

// One chunk's inputs for one workgroup, in registers while the previous
// chunk is computed: W rows (fp16), Q and K rows (bf16), A (fp16), this
// slice's 32 columns of Ut (fp32) and gam.
struct ChunkRegs {
    uint4v w[4], q[4], k[4], a[2], u[2];
    float gam;
};

__device__ __forceinline__ void fetch_chunk(const GdnArgs& p, int c, int h, int kh, int r0,
                                            ChunkRegs& R) {
    const int tid = threadIdx.x, t0 = c * GC, n = min(GC, p.T - t0);
    const uint8_t* blk = p.ws + ((size_t)c * p.hv + h) * GW_BLK;
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) {
        const int idx = pi * 256 + tid, i = idx >> 4, c8 = (idx & 15) * 8;
        R.w[pi] = *reinterpret_cast<const uint4v*>(blk + GW_W + (size_t)(i * GD + c8) * 2);
        R.q[pi] = R.k[pi] = (uint4v){0, 0, 0, 0};
        if (i < n) {
            R.q[pi] = *reinterpret_cast<const uint4v*>(p.q + ((size_t)(t0 + i) * p.hk + kh) * GD + c8);
            R.k[pi] = *reinterpret_cast<const uint4v*>(p.k + ((size_t)(t0 + i) * p.hk + kh) * GD + c8);
        }
    }
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
        const int idx = pi * 256 + tid;
        R.a[pi] = *reinterpret_cast<const uint4v*>(blk + GW_A + (size_t)idx * 16);
        const int i = idx >> 3, c4 = (idx & 7) * 4;
        R.u[pi] = *reinterpret_cast<const uint4v*>(blk + GW_UT + (size_t)(i * GD + r0 + c4) * 4);
    }
    R.gam = tid < GC ? reinterpret_cast<const float*>(blk + GW_GAM)[tid] : 0.f;
}

__global__ __launch_bounds__(256) void gdn_scan(GdnArgs p) {
    __shared__ __attribute__((aligned(16))) _Float16 S16[32 * LD_D], Ws[GC * LD_D], Qs[GC * LD_D];
    __shared__ __attribute__((aligned(16))) _Float16 As[GC * LD_C], KT[GD * LD_C];
    __shared__ __attribute__((aligned(16))) _Float16 UT[32 * LD_C], UdT[32 * LD_C];
    __shared__ __attribute__((aligned(16))) float Us[GC * 32];
    __shared__ float gam[GC];
    const int h = blockIdx.x, r0 = blockIdx.y * 32;
    const int kh = h / (p.hv / p.hk);
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int nch = (p.T + GC - 1) / GC;

    // the state slice: wave w holds S[r0 + row][32 w + l % 32] (accumulator layout)
    float16v S;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        S[e] = p.s0 ? p.s0[((size_t)h * GD + r0 + acc_row(e, l)) * GD + 32 * w + (l & 31)] : 0.f;

    ChunkRegs R;
    if (nch > 0) fetch_chunk(p, 0, h, kh, r0, R);
    for (int c = 0; c < nch; ++c) {
        const int t0 = c * GC, n = min(GC, p.T - t0);
        // chunk c's inputs and the state (fp16) into LDS
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) {
            const int idx = pi * 256 + tid, i = idx >> 4, c8 = (idx & 15) * 8;
            *reinterpret_cast<uint4v*>(Ws + i * LD_D + c8) = R.w[pi];
            *reinterpret_cast<half8*>(Qs + i * LD_D + c8) = bf16x8_to_h8(R.q[pi]);
            const half8 kv = bf16x8_to_h8(R.k[pi]);
#pragma unroll
            for (int x = 0; x < 8; ++x) KT[(c8 + x) * LD_C + i] = kv[x];
        }
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) {
            const int idx = pi * 256 + tid;
            *reinterpret_cast<uint4v*>(As + (idx >> 3) * LD_C + (idx & 7) * 8) = R.a[pi];
            *reinterpret_cast<uint4v*>(Us + idx * 4) = R.u[pi];
        }
        if (tid < GC) gam[tid] = R.gam;
#pragma unroll
        for (int e = 0; e < 16; ++e) S16[acc_row(e, l) * LD_D + 32 * w + (l & 31)] = (_Float16)S[e];
        __syncthreads();
        // the next chunk's inputs travel while this one is computed
        if (c + 1 < nch) fetch_chunk(p, c + 1, h, kh, r0, R);

        // waves 0, 1: X = W S0^T (rows 32 w ..); waves 2, 3: Y = Q S0^T (rows 32 (w - 2) ..)
        const int ti = w & 1;
        float16v XY = (float16v)0.f;
        mma_rows<GD>((w < 2 ? Ws : Qs) + 32 * ti * LD_D, LD_D, S16, LD_D, XY);
        const float bn = __expf(gam[n - 1]);
        if (w < 2) {
            // U = Ut - W S0^T (zero past the chunk's last token), as U^T and
            // as U^T scaled by e^{gam_n - gam_j} for the state update
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = 32 * ti + acc_row(e, l), r = l & 31;
                const float u = i < n ? Us[i * 32 + r] - XY[e] : 0.f;
                UT[r * LD_C + i] = (_Float16)u;
                UdT[r * LD_C + i] = (_Float16)(u * __expf(gam[n - 1] - gam[i]));
            }
        }
        __syncthreads();
        if (w >= 2) {
            // O = diag(b) Q S0^T + A U for rows 32 (w - 2) ..
            float16v Z = (float16v)0.f;
            mma_rows<GC>(As + 32 * ti * LD_C, LD_C, UT, LD_C, Z);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = 32 * ti + acc_row(e, l), r = l & 31;
                if (i < n) {
                    const float ov = __expf(gam[i]) * XY[e] + Z[e];
                    p.o[((size_t)(t0 + i) * p.hv + h) * GD + r0 + r] = (uint16_t)f32_to_bf16(ov);
                }
            }
        }
        // S1 = b_n S0 + U^T diag(e^{gam_n - gam}) K, tile w
#pragma unroll
        for (int e = 0; e < 16; ++e) S[e] *= bn;
        mma_rows<GC>(UdT, LD_C, KT + 32 * w * LD_C, LD_C, S);
        __syncthreads();
    }
    if (p.s_out) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            p.s_out[((size_t)h * GD + r0 + acc_row(e, l)) * GD + 32 * w + (l & 31)] = S[e];
    }
}

}  // namespace moe

extern "C" size_t moe_gdn_workspace_bytes(int T, int hv) {
    if (T < 0 || T > MOE_T_MAX || hv < 1 || hv > MOE_GDN_HEADS_MAX) return 0;
    return (size_t)((T + moe::GC - 1) / moe::GC) * hv * moe::GW_BLK;
}

extern "C" int moe_gdn_scan(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                            const float* beta, int T, int hk, int hv, const float* s0, uint16_t* o,
                            float* s_out, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || T > MOE_T_MAX || hk < 1 || hv < 1 || hv > MOE_GDN_HEADS_MAX || hv % hk)
        return MOE_ERR_INVALID_ARG;
    if (T == 0 && !s_out) return MOE_OK;
    auto al = [](const void* x, uintptr_t a) { return ((uintptr_t)x & (a - 1)) == 0; };
    if (T > 0 && (!q || !k || !v || !g || !beta || !o || !ws)) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!al(q, 16) || !al(k, 16) || !al(v, 16) || !al(ws, 256) || !al(g, 4) ||
                  !al(beta, 4) || !al(o, 2)))
        return MOE_ERR_ALIGN;
    if ((s0 && !al(s0, 4)) || (s_out && !al(s_out, 4))) return MOE_ERR_ALIGN;
    if (T > 0 && ws_bytes < moe_gdn_workspace_bytes(T, hv)) return MOE_ERR_WORKSPACE;
    moe::GdnArgs p{q, k, v, g, beta, s0, o, s_out, (uint8_t*)ws, T, hk, hv};
    const hipStream_t st = (hipStream_t)stream;
    const int nch = (T + moe::GC - 1) / moe::GC;
    if (nch > 0) hipLaunchKernelGGL(moe::gdn_prep, dim3(nch, hv), dim3(256), 0, st, p);
    // (with no tokens the scan kernel only passes the state through)
    hipLaunchKernelGGL(moe::gdn_scan, dim3(hv, moe::GD / 32), dim3(256), 0, st, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
