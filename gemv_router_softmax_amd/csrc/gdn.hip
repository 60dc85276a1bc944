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
//             one quad of lanes per column), Ut and W on MFMA; writes W, A,
//             Ut, the decayed K^T (fp16), gam and -- once per key head -- Q
//             (fp16) to the workspace.
//   gdn_scan  grid (hv, 4): one workgroup per head and 32-row slice of the
//             state (rows are value channels, independent of one another).
//             The slice (32 x 128 fp32) stays in four compute waves' MFMA
//             accumulators for the whole sequence; per chunk it is staged
//             once to LDS as fp16 for the products S0^T.  gdn_prep leaves
//             each chunk's operands in the workspace as an LDS image, which
//             three more waves move in with direct-to-LDS loads (a two-stage
//             ring) while the previous chunk is computed.
//
// Precision: products on v_mfma_f32_32x32x16_f16 (fp32 accumulation);
// q, k, v are bf16 inputs converted to fp16 (exact within fp16's range);
// beta v, beta b k, T, W, A, U and the staged state are rounded to fp16 as
// MFMA operands; the state, Ut and every accumulation stay fp32.
//
// Calls of up to MOE_GDN_STEP_T_MAX tokens (decode) skip all of this:
//   gdn_step  grid (hv, 8): the recurrence itself, token by token, in fp32,
//             each workgroup holding 16 rows of a head's state in registers
//             (see the kernel).
#include "common.hpp"

namespace moe {

constexpr int GD = MOE_GDN_DIM;       // 128: key and value head dimension
constexpr int GC = MOE_GDN_CHUNK;     // 64 tokens per chunk
constexpr int LD_D = GD + 8;          // LDS row stride (halves) of 128-wide fp16 rows
constexpr int LD_C = GC + 8;          // LDS row stride (halves) of 64-wide fp16 rows
// Workspace block of one (chunk, head): the chunk's operands exactly as
// gdn_scan holds them in LDS (padded rows included), so that the scan
// moves them with direct-to-LDS loads -- a part common to the head's four
// state slices, then the four slices' columns of Ut.
constexpr int IMG_Q = 0;                          // fp16 Q [64][136]
constexpr int IMG_W = IMG_Q + GC * LD_D * 2;      // fp16 W [64][136]
constexpr int IMG_KD = IMG_W + GC * LD_D * 2;     // fp16 (e^{gam_n - gam_j} k_j)^T [128][72]
constexpr int IMG_A = IMG_KD + GD * LD_C * 2;     // fp16 A [64][72]
constexpr int IMG_GAM = IMG_A + GC * LD_C * 2;    // fp32 gam [64], then e^{gam} [64] (a 1 KB slot)
constexpr int IMG_COMMON = IMG_GAM + 1024;        // 62 KB
constexpr int UT_SLICE = GC * 32 * 2;             // fp16 Ut[:, 32 z .. 32 z + 31] as [64][32]
constexpr int GW_BLK = IMG_COMMON + 4 * UT_SLICE;
constexpr int STAGE_IMG = IMG_COMMON + UT_SLICE;  // 66 KB moved per chunk and slice
constexpr int STAGE = STAGE_IMG;                  // one LDS stage holds one image
static_assert(IMG_COMMON % 1024 == 0 && IMG_W % 1024 == 0 && STAGE_IMG % 1024 == 0 && STAGE >= STAGE_IMG,
              "1 KB slots");
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

// LDS of gdn_prep, one region reused across the phases (byte offsets):
//   K K^T, Q K^T          Ks [0, 17408)       Qs [17408, 34816)
//   masks, decays         Lp [0, 16384)       A staged [17408, 26624) (Qs read before)
//   triangular solve      Lp read, T written to Ts [26624, 35840)
//   Ut, then W            beta V, then beta b K (transposed) [0, 18432); Ts
//   (Ut, W staged)        [0, 16384) and [16384, 33792)
// 35 KB, so that four workgroups fit on a compute unit: 1024 of them (the
// 32 chunks x 32 heads of 2048 tokens) run in one round.  The Q and
// decayed-K images go from registers straight to the workspace.
constexpr int PR_QS = GC * LD_D * 2, PR_A = PR_QS, PR_LP = 0, PR_TS = PR_QS + GC * LD_C * 2;
constexpr int PR_BT = 0;                          // beta V / beta b K, transposed
constexpr int PR_BYTES = PR_TS + GC * LD_C * 2;
static_assert(PR_LP + GC * GC * 4 <= PR_QS && PR_BT + GD * LD_C * 2 <= PR_TS &&
              4 * UT_SLICE + GC * LD_D * 2 <= PR_BYTES && 2 * PR_QS <= PR_BYTES &&
              4 * (PR_BYTES + 512) <= 160 * 1024, "prep LDS");

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void gdn_prep(GdnArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[PR_BYTES];
    __shared__ float gam[GC], bet[GC];
    _Float16* Ks = reinterpret_cast<_Float16*>(lds);
    _Float16* Qs = reinterpret_cast<_Float16*>(lds + PR_QS);
    float* Lp = reinterpret_cast<float*>(lds + PR_LP);          // row i: L[i][4q+s] at s*16+q
    _Float16* Ts = reinterpret_cast<_Float16*>(lds + PR_TS);
    _Float16* BT = reinterpret_cast<_Float16*>(lds + PR_BT);
    const int c = blockIdx.x, h = blockIdx.y;
    const int kh = h / (p.hv / p.hk);
    const int t0 = c * GC, n = min(GC, p.T - t0);
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    uint8_t* blk = p.ws + ((size_t)c * p.hv + h) * GW_BLK;

    // this thread's rows: token i = tid % 64, channels 32 (tid / 64) .. +31
    // (so that a wave's transposed writes cover 64 consecutive tokens of a
    // channel); loaded first, while the decays are summed
    const int ti_ = tid & 63, cg = tid >> 6;
    uint4v kw[4], qw[4], vw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kw[u] = qw[u] = vw[u] = (uint4v){0, 0, 0, 0};
    if (ti_ < n) {
        const uint4v* kr = reinterpret_cast<const uint4v*>(p.k + ((size_t)(t0 + ti_) * p.hk + kh) * GD + 32 * cg);
        const uint4v* qr = reinterpret_cast<const uint4v*>(p.q + ((size_t)(t0 + ti_) * p.hk + kh) * GD + 32 * cg);
        const uint4v* vr = reinterpret_cast<const uint4v*>(p.v + ((size_t)(t0 + ti_) * p.hv + h) * GD + 32 * cg);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            kw[u] = kr[u];
            qw[u] = qr[u];
            vw[u] = vr[u];
        }
    }
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
        reinterpret_cast<float*>(blk + IMG_GAM)[l] = x;
        reinterpret_cast<float*>(blk + IMG_GAM)[GC + l] = __expf(x);
    }
    __syncthreads();
    const float gn = gam[GC - 1];     // = gam[n - 1]: g is zero past n
    // K, Q rows as fp16 to LDS; Q also to its image; e^{gam_n - gam} k
    // transposed ([channel][token]) to its image, a wave's 64 tokens of a
    // channel in one 128-byte store
    {
        const float dk = __expf(gn - gam[ti_]);
        _Float16* kd_img = reinterpret_cast<_Float16*>(blk + IMG_KD);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c8 = 32 * cg + 8 * u;
            const half8 qh = bf16x8_to_h8(qw[u]);
            *reinterpret_cast<half8*>(Ks + ti_ * LD_D + c8) = bf16x8_to_h8(kw[u]);
            *reinterpret_cast<half8*>(Qs + ti_ * LD_D + c8) = qh;
            if (h % (p.hv / p.hk) == 0)   // (one copy per key head)
                *reinterpret_cast<half8*>(blk + IMG_Q + (ti_ * LD_D + c8) * 2) = qh;
#pragma unroll
            for (int x = 0; x < 8; ++x)
                kd_img[(c8 + x) * LD_C + ti_] =
                    (_Float16)(dk * bf16_to_f32(x & 1 ? kw[u][x >> 1] >> 16 : kw[u][x >> 1] & 0xFFFFu));
        }
    }
    __syncthreads();
    // K K^T and Q K^T: wave w owns the 32 x 32 tile (w/2, w%2)
    const int ti = w >> 1, tj = w & 1;
    float16v aG = (float16v)0.f, aQ = (float16v)0.f;
    mma_rows<GD>(Ks + 32 * ti * LD_D, LD_D, Ks + 32 * tj * LD_D, LD_D, aG);
    mma_rows<GD>(Qs + 32 * ti * LD_D, LD_D, Ks + 32 * tj * LD_D, LD_D, aQ);
    __syncthreads();                  // Ks and Qs read: Lp and A may overwrite them
    {
        // A is staged in its image layout, then stored
        _Float16* As = reinterpret_cast<_Float16*>(lds + PR_A);
        const int j = 32 * tj + (l & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = 32 * ti + acc_row(e, l);
            const float d = j <= i ? __expf(gam[i] - gam[j]) : 0.f;
            Lp[i * GC + (j & 3) * 16 + (j >> 2)] = j < i ? bet[i] * d * aG[e] : 0.f;
            As[i * LD_C + j] = (_Float16)(d * aQ[e]);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < GC * LD_C / 8; idx += 256)
        reinterpret_cast<uint4v*>(blk + IMG_A)[idx] = reinterpret_cast<const uint4v*>(lds + PR_A)[idx];
    // T = (I + L)^{-1}, L strictly lower: column m by the quad of lanes
    // 4m .. 4m+3, lane s holding rows 4q + s (q = 0..15) in registers;
    // row i: T[i][m] = [i == m] - sum_{j<i} L[i][j] T[j][m] (the rows j >= i
    // are still zero, as are L's entries there); four partial sums per lane
    {
        const int m = tid >> 2, s = tid & 3;
        // the column starts as the identity's: row m's 1 is final (the sum
        // of row m is over rows j < m, where the column is zero), and rows
        // not yet solved are multiplied only by L's zeros on and above the
        // diagonal, so step i just subtracts its sum from the row's entry
        float tq[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) tq[q] = 4 * q + s == m ? 1.f : 0.f;
        bool mine[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) mine[x] = s == x;
        // row i + 1 of L is read while row i is reduced.  Only rows j < i
        // contribute (the rest of T's column is still zero), i.e. q <
        // ceil(i / 4): with i a constant after unrolling, the other terms
        // and their reads are left out (up to the sign of a zero, the sums
        // are the same)
        float4v lcur[4], lnxt[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) lcur[b] = lnxt[b] = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < GC; ++i) {
            const int nq = (i + 3) / 4, nqn = (i + 4) / 4;   // active q of rows i and i + 1
            if (i + 1 < GC) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (4 * b < nqn) lnxt[b] = reinterpret_cast<const float4v*>(Lp + (i + 1) * GC + s * 16)[b];
            }
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if (4 * b >= nq) continue;
                const float4v lv = lcur[b];
                part[b] = lv[0] * tq[4 * b];
#pragma unroll
                for (int x = 1; x < 4; ++x)
                    if (4 * b + x < nq) part[b] = fmaf(lv[x], tq[4 * b + x], part[b]);
            }
            float sum = (part[0] + part[1]) + (part[2] + part[3]);
            sum += dpp_f<DPP_XOR1>(sum);
            sum += dpp_f<DPP_XOR2>(sum);
            const float tim = tq[i >> 2] - sum;
            tq[i >> 2] = mine[i & 3] ? tim : tq[i >> 2];
#pragma unroll
            for (int b = 0; b < 4; ++b) lcur[b] = lnxt[b];
        }
        // (Ts lies past Lp and the A staging, which other threads may still read)
#pragma unroll
        for (int q = 0; q < 16; ++q) Ts[(4 * q + s) * LD_C + m] = (_Float16)tq[q];
    }
    __syncthreads();                  // Lp read: beta V may overwrite it
    // Ut = T (beta V), then W = T (beta b K), through one transposed
    // ([channel][token]) region: wave w owns row tile w/2 and column tiles
    // 2 (w%2), 2 (w%2) + 1 of both (column tile = state slice)
    float16v aU[2], aW[2];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const float sc = pass == 0 ? bet[ti_] : bet[ti_] * __expf(gam[ti_]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c8 = 32 * cg + 8 * u;
            const uint4v src = pass == 0 ? vw[u] : kw[u];
#pragma unroll
            for (int x = 0; x < 8; ++x)
                BT[(c8 + x) * LD_C + ti_] =
                    (_Float16)(sc * bf16_to_f32(x & 1 ? src[x >> 1] >> 16 : src[x >> 1] & 0xFFFFu));
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tc = 2 * (w & 1) + u;
            float16v a = (float16v)0.f;
            mma_rows<GC>(Ts + 32 * ti * LD_C, LD_C, BT + 32 * tc * LD_C, LD_C, a);
            if (pass == 0) aU[u] = a;
            else aW[u] = a;
        }
        __syncthreads();              // BT (and after the second pass Ts) read
    }
    // staged in their image layouts (Ut: 4 slices of [64][32] fp16, then W
    // [64][136] fp16), then stored with 16-byte writes
    {
        _Float16* Us = reinterpret_cast<_Float16*>(lds);
        _Float16* Wst = reinterpret_cast<_Float16*>(lds + 4 * UT_SLICE);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tc = 2 * (w & 1) + u;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = 32 * ti + acc_row(e, l);
                Us[tc * (UT_SLICE / 2) + i * 32 + (l & 31)] = (_Float16)aU[u][e];
                Wst[i * LD_D + 32 * tc + (l & 31)] = (_Float16)aW[u][e];
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < 4 * UT_SLICE / 16; idx += 256)
        reinterpret_cast<uint4v*>(blk + IMG_COMMON)[idx] = reinterpret_cast<const uint4v*>(lds)[idx];
    for (int idx = tid; idx < GC * LD_D / 8; idx += 256)
        reinterpret_cast<uint4v*>(blk + IMG_W)[idx] =
            reinterpret_cast<const uint4v*>(lds + 4 * UT_SLICE)[idx];
}

// ------------------------------------------------------------------ scan

typedef __attribute__((address_space(3))) void* gdn_lds_t;

// A wave-uniform 64-bit pointer as scalar values (for buffer resources).
template <typename P>
__device__ __forceinline__ P* gdn_uniform(P* q) {
    const uint64_t v = reinterpret_cast<uint64_t>(q);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gdn_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Mover m's share of chunk c's image for state slice z into one LDS stage:
// slots 22 m .. 22 m + 21, where 1 KB slot j comes from byte j K of the
// block's common part (j < 62) or of the slice's Ut columns (j = 62 .. 65).
constexpr int MV_SLOTS = 22;
static_assert(3 * MV_SLOTS * 1024 == STAGE_IMG, "three movers cover an image");
// The Q image depends only on the key head: the first value head of each
// key head's group holds it for the group, so the range starts at that
// head's block.
__device__ __forceinline__ void gdn_issue(const GdnArgs& p, int c, int h, int z, int m,
                                          uint8_t* __restrict__ stage) {
    const int grp = p.hv / p.hk, hq = h - h % grp;
    const uint8_t* blk = gdn_uniform(p.ws + ((size_t)c * p.hv + hq) * GW_BLK);
    const __amdgpu_buffer_rsrc_t r = gdn_rsrc(blk, (uint32_t)grp * GW_BLK);
    const uint32_t own = (uint32_t)(h - hq) * GW_BLK;
    const uint32_t lane16 = (threadIdx.x & 63) * 16;
#pragma unroll
    for (int i = 0; i < MV_SLOTS; ++i) {
        const int j = m * MV_SLOTS + i;
        const uint32_t src = j < IMG_W / 1024 ? (uint32_t)j * 1024
                             : j < IMG_COMMON / 1024
                                 ? own + (uint32_t)j * 1024
                                 : own + (uint32_t)(IMG_COMMON + z * UT_SLICE + (j - IMG_COMMON / 1024) * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (gdn_lds_t)(stage + j * 1024), 16, lane16, src, 0, 0);
    }
}

__device__ __forceinline__ constexpr int gdn_vmcnt(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);   // vmcnt(n), other counters free
}

// A workgroup barrier without a memory fence: this wave's LDS operations
// are complete before it (lgkmcnt(0)), so LDS written before it is visible
// after it, while global memory operations in flight -- the image loads --
// stay in flight (__syncthreads would wait for them).  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void gdn_barrier() {
    __builtin_amdgcn_s_waitcnt((3 << 14) | (7 << 4) | 15);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The image movers (waves 4, 5, 6): chunk c + 1 into nxt while the compute
// waves work on chunk c.  They read no LDS and the compute waves issue no
// image loads, so no wait for the loads ever lands in the compute waves'
// code.  The 66 loads of an image are split so that no mover holds up a
// barrier: mover 0 issues slots 0..21 after barrier (1) (the compute waves
// then multiply for a while), movers 1 and 2 slots 22..43 and 44..65 after
// barrier (2).  Two barriers per chunk, matched one for one by gdn_chunk.
__device__ __forceinline__ void gdn_mover_chunk(const GdnArgs& p, int c, int nch, int h, int z,
                                                int m, uint8_t* __restrict__ nxt) {
    __builtin_amdgcn_s_waitcnt(gdn_vmcnt(0));       // this mover's part of chunk c landed
    gdn_barrier();                                // (1) chunk c ready, S16 staged
    // (every compute wave read nxt, chunk c - 1's image, before it staged
    // S16 for chunk c and reached barrier (1))
    if (m == 0 && c + 1 < nch) gdn_issue(p, c + 1, h, z, m, nxt);
    gdn_barrier();                                // (2)
    if (m != 0 && c + 1 < nch) gdn_issue(p, c + 1, h, z, m, nxt);
}

// Output rows of one chunk (waves 2, 3: rows 32 (w - 2) .. of the chunk
// starting at token t0), packed as bf16 pairs in accumulator order.  The
// per-lane offset is computed once; each element adds a wave-uniform step
// (the scalar offset operand).  Rows past T lie past the buffer's range,
// so their stores write nothing; every offset stays below 2^32 (at most
// 65599 token rows of at most 64 heads x 256 bytes).
__device__ __forceinline__ void gdn_store_out(const GdnArgs& p, int t0, int h, int r0, int ti,
                                              const uint32_t (&pk)[8], __amdgpu_buffer_rsrc_t ro) {
    const int l = threadIdx.x & 63;
    const uint32_t rs = (uint32_t)p.hv * GD * 2;      // bytes per token of o
    const uint32_t voff = (uint32_t)(((size_t)t0 * p.hv + h) * GD + r0 + (l & 31)) * 2 + 4u * (l >> 5) * rs;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t soff = (uint32_t)(32 * ti + 8 * (e >> 2) + (e & 3)) * rs;
        const uint32_t v = (e & 1) ? pk[e >> 1] >> 16 : pk[e >> 1];
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, ro, voff, soff, 0);
    }
}

// One chunk of the scan for the state slice held in S (compute waves 0-3).
// cur holds chunk c's image.  Waves 2, 3 form this chunk's outputs but
// store them during the next chunk's U phase (pend, from token pend_t0;
// -1: none), where they would otherwise wait for waves 0, 1.
__device__ __forceinline__ void gdn_chunk(const GdnArgs& p, int c, int h, int z, int w,
                                          const uint8_t* __restrict__ cur,
                                          _Float16* __restrict__ S16, _Float16* __restrict__ UT,
                                          __amdgpu_buffer_rsrc_t ro, float16v& S, uint32_t (&pend)[8],
                                          int& pend_t0) {
    const int l = threadIdx.x & 63, r0 = z * 32;
    const int t0 = c * GC, n = min(GC, p.T - t0);
#pragma unroll
    for (int e = 0; e < 16; ++e) S16[acc_row(e, l) * LD_D + 32 * w + (l & 31)] = (_Float16)S[e];
    gdn_barrier();                                // (1)
    const _Float16* Qs = reinterpret_cast<const _Float16*>(cur + IMG_Q);
    const _Float16* Ws = reinterpret_cast<const _Float16*>(cur + IMG_W);
    const _Float16* KdT = reinterpret_cast<const _Float16*>(cur + IMG_KD);
    const _Float16* As = reinterpret_cast<const _Float16*>(cur + IMG_A);
    const float* bexp = reinterpret_cast<const float*>(cur + IMG_GAM) + GC;   // e^{gam}
    const _Float16* Us = reinterpret_cast<const _Float16*>(cur + IMG_COMMON);

    // waves 0, 1: X = W S0^T (rows 32 w ..); waves 2, 3: Y = Q S0^T (rows 32 (w - 2) ..)
    const int ti = w & 1;
    float16v XY = (float16v)0.f;
    mma_rows<GD>((w < 2 ? Ws : Qs) + 32 * ti * LD_D, LD_D, S16, LD_D, XY);
    if (w < 2) {
        // U = Ut - W S0^T, as U^T (rows past the chunk's tokens are zero in
        // both terms)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = 32 * ti + acc_row(e, l), r = l & 31;
            UT[r * LD_C + i] = (_Float16)((float)Us[i * 32 + r] - XY[e]);
        }
    } else if (pend_t0 >= 0) {
        gdn_store_out(p, pend_t0, h, r0, ti, pend, ro);
    }
    gdn_barrier();                                // (2)
    // S1 = b_n S0 + U^T (e^{gam_n - gam} K), tile w; waves 2, 3 also
    // O = diag(b) Q S0^T + A U for rows 32 (w - 2) .. (two independent MFMA
    // chains in one block)
    const float bn = bexp[n - 1];
#pragma unroll
    for (int e = 0; e < 16; ++e) S[e] *= bn;
    if (w >= 2) {
        float16v Zo = (float16v)0.f;
        mma_rows<GC>(As + 32 * ti * LD_C, LD_C, UT, LD_C, Zo);
        mma_rows<GC>(UT, LD_C, KdT + 32 * w * LD_C, LD_C, S);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i0 = 32 * ti + acc_row(2 * j, l), i1 = 32 * ti + acc_row(2 * j + 1, l);
            const float o0 = bexp[i0] * XY[2 * j] + Zo[2 * j];
            const float o1 = bexp[i1] * XY[2 * j + 1] + Zo[2 * j + 1];
            pend[j] = f32_to_bf16(o0) | (f32_to_bf16(o1) << 16);
        }
        pend_t0 = t0;
    } else {
        mma_rows<GC>(UT, LD_C, KdT + 32 * w * LD_C, LD_C, S);
    }
    // No barrier here: the next chunk's S16 writes follow this chunk's S16
    // reads across barrier (2), its U^T writes follow every wave's U^T reads
    // across its barrier (1), and the movers refill this chunk's image only
    // after that barrier too.
}

// grid (hv, 4) workgroups of 7 waves: waves 0-3 compute (wave w holds the
// state tile of key channels 32 w ..), waves 4-6 move the chunk images.
__global__ __launch_bounds__(448) void gdn_scan(GdnArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t stage0[STAGE], stage1[STAGE];
    __shared__ __attribute__((aligned(16))) _Float16 S16[32 * LD_D], UT[32 * LD_C];
    const int h = blockIdx.x, z = blockIdx.y, r0 = z * 32;
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = (p.T + GC - 1) / GC;

    if (w >= 4) {
        const int m = w - 4;
        if (nch > 0) gdn_issue(p, 0, h, z, m, stage0);
        for (int c = 0; c < nch; c += 2) {
            gdn_mover_chunk(p, c, nch, h, z, m, stage1);
            if (c + 1 < nch) gdn_mover_chunk(p, c + 1, nch, h, z, m, stage0);
        }
        return;
    }
    // output rows through a buffer range: rows past T are not written
    const __amdgpu_buffer_rsrc_t ro = gdn_rsrc(p.o, (uint32_t)((size_t)p.T * p.hv * GD * 2));
    // the state slice: wave w holds S[r0 + row][32 w + l % 32] (accumulator layout)
    float16v S;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        S[e] = p.s0 ? p.s0[((size_t)h * GD + r0 + acc_row(e, l)) * GD + 32 * w + (l & 31)] : 0.f;
    uint32_t pend[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int pend_t0 = -1;
    for (int c = 0; c < nch; c += 2) {
        gdn_chunk(p, c, h, z, w, stage0, S16, UT, ro, S, pend, pend_t0);
        if (c + 1 < nch) gdn_chunk(p, c + 1, h, z, w, stage1, S16, UT, ro, S, pend, pend_t0);
    }
    if (w >= 2 && pend_t0 >= 0) gdn_store_out(p, pend_t0, h, r0, w & 1, pend, ro);
    if (p.s_out) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            p.s_out[((size_t)h * GD + r0 + acc_row(e, l)) * GD + 32 * w + (l & 31)] = S[e];
    }
}

// ------------------------------------------------------------------ step

// Token by token, for short calls (decode: a few tokens per call), where
// the chunked form's two kernels and per-chunk preparation cost more than
// the state's own traffic.  grid (hv, 8) workgroups of 256 threads, each
// holding 16 value rows of one head's state in registers, in fp32: thread
// tid has row 16 blockIdx.y + tid / 16 and key channels 8 (tid % 16) .. +7,
// so a row's 16 threads are one 16-lane DPP row.  Per token, with a = e^g:
//   Sk_r = sum_c S[r][c] k[c]                      (row all-reduce)
//   S[r][c] = a S[r][c] + beta (v_r - a Sk_r) k[c]  (= a S (I - beta k k^T) + beta v k^T)
//   o_r = sum_c S[r][c] q[c]
// The operands of the next four tokens are in flight while one is processed.
constexpr int GS_ROWS = 16, GS_PF = 4;

__device__ __forceinline__ void bf16x8_to_f32(uint4v w, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
}

__global__ __launch_bounds__(256) void gdn_step(GdnArgs p) {
    const int h = blockIdx.x, r = blockIdx.y * GS_ROWS + (threadIdx.x >> 4), cg = threadIdx.x & 15;
    const int kh = h / (p.hv / p.hk);
    // (16-byte accesses where the state arrays allow them; they need only
    // be 4-byte aligned)
    const size_t soff = ((size_t)h * GD + r) * GD + 8 * cg;
    float S[8];
    if (p.s0 && ((uintptr_t)p.s0 & 15) == 0) {
        const float4v* sp = reinterpret_cast<const float4v*>(p.s0 + soff);
        const float4v s0 = sp[0], s1 = sp[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S[i] = s0[i];
            S[4 + i] = s1[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = p.s0 ? p.s0[soff + i] : 0.f;
    }
    // operands of tokens t .. t + GS_PF - 1 in flight (slot t % GS_PF; the
    // loop is unrolled by GS_PF so that the slots are registers)
    uint4v kn[GS_PF], qn[GS_PF];
    uint32_t vn[GS_PF];
    float gn[GS_PF], bn[GS_PF];
    auto fetch = [&](int t, int u) {
        if (t < p.T) {
            kn[u] = *reinterpret_cast<const uint4v*>(p.k + ((size_t)t * p.hk + kh) * GD + 8 * cg);
            qn[u] = *reinterpret_cast<const uint4v*>(p.q + ((size_t)t * p.hk + kh) * GD + 8 * cg);
            vn[u] = p.v[((size_t)t * p.hv + h) * GD + r];
            gn[u] = p.g[(size_t)t * p.hv + h];
            bn[u] = p.beta[(size_t)t * p.hv + h];
        }
    };
#pragma unroll
    for (int u = 0; u < GS_PF; ++u) fetch(u, u);
    for (int t0 = 0; t0 < p.T; t0 += GS_PF) {
#pragma unroll
        for (int u = 0; u < GS_PF; ++u) {
            const int t = t0 + u;
            if (t >= p.T) break;
            float kk[8], qq[8];
            bf16x8_to_f32(kn[u], kk);
            bf16x8_to_f32(qn[u], qq);
            const float vr = bf16_to_f32(vn[u]), a = __expf(gn[u]), bt = bn[u];
            fetch(t + GS_PF, u);
            float sk = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) sk = fmaf(S[c], kk[c], sk);
            sk = row16_sum(sk);
            const float coef = bt * (vr - a * sk);
            float ov = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                S[c] = fmaf(coef, kk[c], a * S[c]);
                ov = fmaf(S[c], qq[c], ov);
            }
            ov = row16_sum(ov);
            if (cg == 0) p.o[((size_t)t * p.hv + h) * GD + r] = (uint16_t)f32_to_bf16(ov);
        }
    }
    if (p.s_out && ((uintptr_t)p.s_out & 15) == 0) {
        float4v* sp = reinterpret_cast<float4v*>(p.s_out + soff);
        sp[0] = (float4v){S[0], S[1], S[2], S[3]};
        sp[1] = (float4v){S[4], S[5], S[6], S[7]};
    } else if (p.s_out) {
#pragma unroll
        for (int i = 0; i < 8; ++i) p.s_out[soff + i] = S[i];
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
    if (T <= MOE_GDN_STEP_T_MAX) {
        // (with no tokens the state only passes through)
        hipLaunchKernelGGL(moe::gdn_step, dim3(hv, moe::GD / moe::GS_ROWS), dim3(256), 0, st, p);
    } else {
        const int nch = (T + moe::GC - 1) / moe::GC;
        hipLaunchKernelGGL(moe::gdn_prep, dim3(nch, hv), dim3(256), 0, st, p);
        hipLaunchKernelGGL(moe::gdn_scan, dim3(hv, moe::GD / 32), dim3(448), 0, st, p);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
