// decode.hip -- the decode (dequantising GEMV) paths of the MoE layer.
//
// Decode is memory bound (leslieli.dev note on the Lily engine, paragraph 5:
// the sparse GEMV barely changes when its arithmetic is removed) and, at a
// few tokens, dominated by latency.  Two paths, neither with host
// involvement:
//
// Few tokens (T <= MOE_DECODE_T, the default there), further below: a layer
// on its own is three kernels (router logits | gate/up with the top-8 inside
// | down with the combine and the residual add); inside a chain every layer
// after the first is two, because the down kernel also forms the next
// layer's router logits.
//
// Up to MOE_DECODE_T_MAX tokens when the decode path is forced, four
// kernels:
//
//   route_logits_gemv   (route.hip) logits of the 256 experts
//   route_select        ONE workgroup: top-8 per token (ties to the lower
//                       expert index), renormalised softmax weights, the
//                       shared-expert gate, the stable permutation, the
//                       row-tile list and the fp16 copy of x the GEMV reads
//   decode_gateup       16 gate rows + 16 up rows of one active expert per
//                       workgroup; every lane streams 16 B of each row
//                       (coalesced 128-bit loads, all issued up front) and
//                       applies the group scale/bias once per lane on exact
//                       codes (v_dot2_f32_f16 on fp16 code pairs); eight dot
//                       products are reduced together with a transposing
//                       butterfly; h = bf16(silu(g) u)
//   decode_down_combine 4 output rows per workgroup for ALL active experts:
//                       down GEMV on exact codes, then the weighted combine
//                       with the shared expert and the residual add, so the
//                       expert outputs never go to memory
//
// Fusing the chain follows "A Rust + Metal Inference Engine for
// Qwen3.6-35B-A3B on Apple Silicon", paragraph 5 (decode fuses kernel
// chains).
#include "block_util.hpp"

namespace moe {

// One workgroup (256 threads), T <= MOE_DECODE_T_MAX.  logits [T][256] from
// route_logits_gemv; writes ids, weights, shared gate, counts, offsets,
// perm, inv and the row tiles.
__global__ __launch_bounds__(256) void route_select(const float* __restrict__ logits,
                                                    const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wsg, int T,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts,
                                                    float* __restrict__ sg,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ inv,
                                                    Tile* __restrict__ tiles,
                                                    int* __restrict__ tile_count,
                                                    uint16_t* __restrict__ xh) {
    __shared__ int ids_l[MOE_DECODE_T_MAX * TOPK];
    __shared__ int hist[256];
    __shared__ int base[256];
    __shared__ int offs_l[257];
    __shared__ int wcnt[4 * 256];
    __shared__ int scr[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    hist[tid] = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w * 256 + tid] = 0;
    for (int t = wave; t < T; t += 4) {
        wave_top8(logits + (size_t)t * E, ids + (size_t)t * TOPK, wts + (size_t)t * TOPK,
                  ids_l + t * TOPK);
        const uint4v* xr = reinterpret_cast<const uint4v*>(x + (size_t)t * H) + lane * 4;
        const uint4v* gr = reinterpret_cast<const uint4v*>(wsg) + lane * 4;
        float z = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4v a = xr[c], b = gr[c];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z = fmaf(bf16_to_f32(a[i] & 0xFFFFu), bf16_to_f32(b[i] & 0xFFFFu), z);
                z = fmaf(bf16_to_f32(a[i] >> 16), bf16_to_f32(b[i] >> 16), z);
            }
        }
        z = wave_sum(z);
        if (lane == 0) sg[t] = 1.f / (1.f + expf(-z));
    }
    // fp16 activations in chunk-slot order for the gate/up GEMV
    for (int ci = tid; ci < T * (H / 8); ci += 256)
        reinterpret_cast<uint4v*>(xh)[ci] =
            bf16x8_to_f16_slots(reinterpret_cast<const uint4v*>(x)[ci]);
    __syncthreads();
    const int n = TOPK * T;
    for (int f = tid; f < n; f += 256) atomicAdd(&hist[ids_l[f]], 1);
    __syncthreads();
    const int c = hist[tid];
    int total;
    const int off = block_excl_scan256(c, scr, &total);
    counts[tid] = c;
    offsets[tid] = off;
    offs_l[tid] = off;
    if (tid == 0) { offsets[E] = total; offs_l[E] = total; }
    base[tid] = off;
    __syncthreads();
    stable_scatter(ids_l, 0, n, base, wcnt, perm, inv);
    // row tiles: one per active expert (T <= 32 rows each), then the shared expert
    const int active = c > 0 ? 1 : 0;
    int na;
    const int slot = block_excl_scan256(active, scr, &na);
    if (active) {
        Tile tl;
        tl.group = tid;
        tl.row0 = off;
        tl.nrows = c;
        tl.pad = 0;
        tiles[slot] = tl;
    }
    if (tid == 0) {
        Tile tl;
        tl.group = E;
        tl.row0 = n;
        tl.nrows = T;
        tl.pad = 0;
        tiles[na] = tl;
        *tile_count = na + 1;
    }
}

// grid (max tiles, I / 16); 4 waves x 4 rows (gate and up) each.  Lane l
// covers K = 32l .. 32l+31 (one 16-byte code load per row, half of one
// 64-wide group).  xh: fp16 activations in chunk-slot order.  h = bf16(silu(g)
// u) is stored as fp16 (exact) in chunk-slot order, the layout every expert
// kernel reads.
__global__ __launch_bounds__(256) void decode_gateup(const uint16_t* __restrict__ xh, int T,
                                                     const int32_t* __restrict__ perm,
                                                     const Tile* __restrict__ tiles,
                                                     const int* __restrict__ tile_count,
                                                     QFFN routed, QFFN shared,
                                                     uint16_t* __restrict__ hout) {
    if ((int)blockIdx.x >= *tile_count) return;
    const Tile tl = tiles[blockIdx.x];
    const bool sh = tl.group >= E;
    const int e = sh ? 0 : tl.group;
    const QFFN q = sh ? shared : routed;
    const int lane = threadIdx.x & 63;
    const int n0 = blockIdx.y * 16 + (threadIdx.x >> 6) * 4;
    // value index i < 4: gate row n0+i, i >= 4: up row n0+i-4
    uint4v wq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const size_t row = n0 + (i & 3);
        const uint32_t* qb = expert_at(i < 4 ? q.gate_q : q.up_q, e, q.sq);
        wq[i] = reinterpret_cast<const uint4v*>(qb + row * (H / 8))[lane];
    }
    float s[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const size_t row = n0 + (i & 3);
        const uint16_t* sb = expert_at(i < 4 ? q.gate_s : q.up_s, e, q.ss);
        const uint16_t* bb = expert_at(i < 4 ? q.gate_b : q.up_b, e, q.ss);
        s[i] = fp16_to_f32(sb[row * (H / G) + (lane >> 1)]);
        b[i] = fp16_to_f32(bb[row * (H / G) + (lane >> 1)]);
    }
    for (int rr = 0; rr < tl.nrows; ++rr) {
        const int p = tl.row0 + rr;
        int t;
        if (p < TOPK * T) t = min(max(perm[p] >> 3, 0), T - 1);
        else t = p - TOPK * T;
        const uint4v* xr = reinterpret_cast<const uint4v*>(xh + (size_t)t * H) + lane * 4;
        uint4v xp[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) xp[cc] = xr[cc];
        float sx = 0.f;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) sx = sum8_h(xp[cc], sx);
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float d = 0.f;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) d = dot8_codes(wq[i][cc], xp[cc], d);
            acc[i] = fmaf(s[i], d, b[i] * sx);
        }
        float tot[8];                                   // gate rows n0.., then up rows n0..
        wave_sum8(acc, tot);
        if (lane < 4) {
            const int vi = lane;
            const float g = vi == 0 ? tot[0] : vi == 1 ? tot[1] : vi == 2 ? tot[2] : tot[3];
            const float u = vi == 0 ? tot[4] : vi == 1 ? tot[5] : vi == 2 ? tot[6] : tot[7];
            const float a = g / (1.f + expf(-g));
            const int n = n0 + vi;
            const float hb = bf16_to_f32(f32_to_bf16(a * u));
            hout[(size_t)p * I + (n & ~7) + chunk_slot(n & 7)] =
                __builtin_bit_cast(uint16_t, (_Float16)hb);
        }
    }
}

// grid (H / 4): 4 output rows per workgroup; wave w takes tiles w, w+4, ...;
// 16 lanes per row (16 B of codes each, K = 32c .. 32c+31).
// y[t] = bf16(sum over the token's experts of coef * d + sg * d_shared),
// optionally res = bf16(x + y).
__global__ __launch_bounds__(256) void decode_down_combine(
    const uint16_t* __restrict__ hin, int T, const int32_t* __restrict__ perm,
    const Tile* __restrict__ tiles, const int* __restrict__ tile_count,
    const float* __restrict__ wts, const float* __restrict__ sg, QFFN routed,
    QFFN shared, uint16_t* __restrict__ y, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ res) {
    __shared__ float yacc[4][MOE_DECODE_T_MAX][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane >> 4, c = lane & 15;
    const int m = blockIdx.x * 4 + r;
    const int ntiles = *tile_count;
    float acc[MOE_DECODE_T_MAX];
#pragma unroll
    for (int t = 0; t < MOE_DECODE_T_MAX; ++t) acc[t] = 0.f;
    for (int ti0 = wave; ti0 < ntiles; ti0 += 16) {
        // up to four tiles per pass, loads issued before any arithmetic
        uint4v dw[4];
        float ds[4], db[4];
        Tile tl[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int ti = ti0 + 4 * k;
            tl[k] = tiles[ti < ntiles ? ti : ti0];
            const bool sh = tl[k].group >= E;
            const int e = sh ? 0 : tl[k].group;
            const QFFN& q = sh ? shared : routed;
            const size_t row = m;
            dw[k] = reinterpret_cast<const uint4v*>(expert_at(q.down_q, e, q.sq) + row * (I / 8))[c];
            ds[k] = fp16_to_f32(expert_at(q.down_s, e, q.ss)[row * (I / G) + (c >> 1)]);
            db[k] = fp16_to_f32(expert_at(q.down_b, e, q.ss)[row * (I / G) + (c >> 1)]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (ti0 + 4 * k >= ntiles) break;
            const float bk = db[k];
            for (int rr = 0; rr < tl[k].nrows; ++rr) {
                const int p = tl[k].row0 + rr;
                int t;
                float coef;
                if (p < TOPK * T) {
                    const int f = perm[p];
                    t = min(max(f >> 3, 0), T - 1);
                    coef = wts[f];
                } else {
                    t = p - TOPK * T;
                    coef = sg[t];
                }
                const uint4v* hr = reinterpret_cast<const uint4v*>(hin + (size_t)p * I) + c * 4;
                float sh_ = 0.f, dot = 0.f;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const uint4v hv = hr[cc];
                    sh_ = sum8_h(hv, sh_);
                    dot = dot8_codes(dw[k][cc], hv, dot);
                }
                const float part = coef * fmaf(ds[k], dot, bk * sh_);
#pragma unroll
                for (int tt = 0; tt < MOE_DECODE_T_MAX; ++tt)
                    if (tt == t) acc[tt] += part;
            }
        }
    }
    // reduce the 16 lanes of each row, then the four waves in a fixed order
#pragma unroll
    for (int t = 0; t < MOE_DECODE_T_MAX; ++t) {
        if (t < T) {
            float v = acc[t];
            v += __shfl_xor(v, 8, WAVE);
            v += __shfl_xor(v, 4, WAVE);
            v += __shfl_xor(v, 2, WAVE);
            v += __shfl_xor(v, 1, WAVE);
            if (c == 0) yacc[wave][t][r] = v;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * 4; i += 256) {
        const int t = i >> 2, rr = i & 3;
        const float v = ((yacc[0][t][rr] + yacc[1][t][rr]) + yacc[2][t][rr]) + yacc[3][t][rr];
        const uint32_t yb = f32_to_bf16(v);
        const size_t o = (size_t)t * H + blockIdx.x * 4 + rr;
        y[o] = (uint16_t)yb;
        if (res) res[o] = (uint16_t)f32_to_bf16(bf16_to_f32(x[o]) + bf16_to_f32(yb));
    }
}

// ---------------------------------------------------------------------
// Few-token layer (T <= MOE_DECODE_T).
//
// A layer that follows another layer of a chain is two kernels; a layer on
// its own (or the first of a chain) adds the router kernel in front:
//
//   route_logits_dec   the 256 expert logits and the shared-gate logit of
//                      each token (one wave per router row), stored as 64-bit
//                      fixed point (below), and the fp16 copy of x in
//                      chunk-slot order;
//   decode_gateup_dec  slot 0 = the shared expert (needs no routing); one
//                      token: slot a >= 1 = the a-th active routed expert,
//                      which every routed workgroup finds by running the
//                      top-8 selection itself on the logits (block_route),
//                      and workgroup (0, 0) publishes the down record; more
//                      tokens: slot 1 + 8t + j = token t's j-th expert, from
//                      token t's logits alone.  h rows are compact: the T
//                      shared rows, then one row per routed (slot, token),
//                      9T rows in all;
//   decode_down_dec    DN_ROWS output rows per workgroup over every slot
//                      (each wave a row group x a slot group), h rows read
//                      straight from global memory; combine with the routing
//                      weights and the shared gate, residual add.  Inside a
//                      chain it also writes the next layer's fp16
//                      activations and adds its share of the next layer's
//                      router logits.
//
// Router logits in 64-bit fixed point: a down workgroup of a chain holds
// DN_ROWS entries of the next layer's input, so it can form its partial
// router sums for all 257 logits itself (fp32, in a fixed order) and add
// round(p * 2^32) to the next layer's accumulators with integer atomics.
// Integer addition is associative, so the sum does not depend on the order
// in which the DN_WG workgroups' atomics land: the routing stays
// deterministic.  This takes the router kernel and one kernel boundary off
// every chained layer -- the decode chain fused across layers ("A Rust +
// Metal Inference Engine for Qwen3.6-35B-A3B on Apple Silicon", paragraph 5).
//
// Ids read back from the record are clamped, so a corrupted record cannot
// send a load outside the weights.

// Fixed-point logit accumulators: a set is ACC_COPIES copies of [T]
// [ACC_STRIDE] int64 words (words 0..255 of a token: the expert logits
// without the router bias, word 256: the shared-gate logit); a logit is the
// sum over the copies.
//
// The down kernel's shape (decode_down_dec): DN_RG row groups of four rows x
// DN_SG slot groups of waves per workgroup, DN_WG workgroups.  Its
// workgroups add their partial router sums to ACC_COPIES copies of the
// accumulators (DN_WG / ACC_COPIES workgroups meet on one address), which
// the gate/up kernel adds up.  Measured on the 40-layer T = 1 chain, us per
// layer (rows per workgroup / workgroups / copies): 8 / 256 / 8: 14.75;
// 8 / 256 / 4: 15.02; 8 / 256 / 2: 15.80; 4 / 512 / 8: 15.00; 4 / 512 / 4:
// 15.93; 4 / 512 / 1: 23.4; 16 / 128 / 4: 16.56; 16 / 128 / 1: 17.76.  More
// atomics on one address cost the down kernel more than reading more copies
// costs the gate/up kernel, down to 32 workgroups per address.  (The
// compile-time knobs exist for such sweeps.)
#ifndef MOE_DN_RG
#define MOE_DN_RG 2
#endif
#ifndef MOE_DN_SG
#define MOE_DN_SG 4
#endif
#ifndef MOE_ACC_COPIES
#define MOE_ACC_COPIES 8
#endif
constexpr int DN_RG = MOE_DN_RG;
constexpr int DN_SG = MOE_DN_SG;
constexpr int DN_WAVES = DN_RG * DN_SG;
constexpr int DN_ROWS = 4 * DN_RG;
constexpr int DN_WG = H / DN_ROWS;
constexpr int DN_SPW = (1 + TOPK + DN_SG - 1) / DN_SG;   // slots per wave per pass
constexpr int ACC_COPIES = MOE_ACC_COPIES;
static_assert(DN_WG % ACC_COPIES == 0, "accumulator copies");
static_assert(64 * DN_WAVES <= 1024, "workgroup size");

constexpr int ACC_N = E + 1;
constexpr int ACC_STRIDE = 264;                 // 32-byte aligned per token
constexpr double ACC_ONE = 4294967296.0;        // 2^32
static_assert(ACC_STRIDE >= ACC_N && ACC_STRIDE % 4 == 0, "accumulator layout");

__device__ __forceinline__ long long acc_fix(float v) {
    // |v| < 2^30 keeps 257 tokens' worth of sums far from the int64 range;
    // larger (never finite-sensible) values are clamped
    const double d = fmin(fmax((double)v * ACC_ONE, -0x1p62), 0x1p62);
    return (long long)__builtin_elementwise_rint(d);
}
__device__ __forceinline__ float acc_val(long long q) { return (float)((double)q * (1.0 / ACC_ONE)); }

// Logits of experts 4l .. 4l+3 of token t for lane l (the sum over the
// ACC_COPIES accumulator copies of T tokens each, all loads issued
// together), plus the router bias.
__device__ __forceinline__ float4v load_logits4(const long long* __restrict__ acc, int T,
                                                const float* __restrict__ bias, int t, int lane) {
    typedef long long ll2 __attribute__((ext_vector_type(2)));
    // the bias first, with no branch around the load (a missing bias is an
    // empty buffer range, which reads as zeros): behind a branch the load
    // would go out only after the logits had arrived
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(bias), 0, bias ? (uint32_t)(E * sizeof(float)) : 0u, 0x00020000);
    const float4v bv = __builtin_bit_cast(
        float4v, __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)(16 * lane), 0, 0));
    ll2 pa[ACC_COPIES], pb[ACC_COPIES];
#pragma unroll
    for (int c = 0; c < ACC_COPIES; ++c) {
        const ll2* p = reinterpret_cast<const ll2*>(acc + ((size_t)c * T + t) * ACC_STRIDE + 4 * lane);
        pa[c] = p[0];
        pb[c] = p[1];
    }
    ll2 a = pa[0], b = pb[0];
#pragma unroll
    for (int c = 1; c < ACC_COPIES; ++c) {
        a += pa[c];
        b += pb[c];
    }
    float4v v = {acc_val(a[0]), acc_val(a[1]), acc_val(b[0]), acc_val(b[1])};
    return v + bv;
}

// The routing of up to MOE_DECODE_T tokens, in LDS of the gate/up kernel.
struct RouteRec {
    int ids[MOE_DECODE_T][TOPK];
    float w[MOE_DECODE_T][TOPK];
    float sg[MOE_DECODE_T];
    int active[MOE_DECODE_T * TOPK];     // active experts, ascending id
    uint32_t tmask[MOE_DECODE_T * TOPK]; // tokens that selected active[a]
    int nact;
};

// What the down kernel needs, in global memory: slot 0 is the shared
// expert, slot a >= 1 the a-th active routed expert (ascending id).  Every
// array is read with one 8-byte load per lane (lane l: slots 2l, 2l+1), all
// issued together, and picked apart with lane reads -- one memory round
// trip for the whole record.
constexpr int DEC_SLOTS = 1 + MOE_DECODE_T * TOPK;
struct DownRec {
    int slot_e[128];                   // expert of each slot; [127]: the slot count
    uint32_t slot_m[128];              // tokens of each slot (bit t)
    int slot_h[128];                   // first h row of each slot (its tokens' rows
                                       // follow in ascending token order)
    float coef[MOE_DECODE_T][128];     // token t's weight for slot a (the shared gate for
                                       // slot 0; 0 where the token did not pick the expert)
};
static_assert(DEC_SLOTS < 127, "slot count word");

// Weight pointers of one expert stack as opaque scalar values, taken from
// the kernel arguments at entry.  Choosing between the routed and the
// shared stack by a condition on the argument structs themselves makes the
// compiler select the structs' addresses and re-read the pointers with
// vector-memory loads just before the weight loads -- one more memory round
// trip on the critical path.  A choice between these values is a scalar
// select.
// (Global address space: behind the opaque copy the compiler could not
// otherwise tell the pointers from generic ones and would use flat loads.)
#define GLOBAL_AS __attribute__((address_space(1)))
struct GUPtrs {
    const GLOBAL_AS uint32_t *gq, *uq;
    const GLOBAL_AS uint16_t *gs, *gb, *us, *ub;
    uint32_t sq, ss;
};
struct DnPtrs {
    const GLOBAL_AS uint32_t* q;
    const GLOBAL_AS uint16_t *s, *b;
    uint32_t sq, ss;
};
__device__ __forceinline__ GUPtrs gu_ptrs(const QFFN& f) {
    GUPtrs p{(const GLOBAL_AS uint32_t*)f.gate_q, (const GLOBAL_AS uint32_t*)f.up_q,
             (const GLOBAL_AS uint16_t*)f.gate_s, (const GLOBAL_AS uint16_t*)f.gate_b,
             (const GLOBAL_AS uint16_t*)f.up_s,   (const GLOBAL_AS uint16_t*)f.up_b,
             f.sq, f.ss};
    asm volatile("" : "+s"(p.gq), "+s"(p.uq), "+s"(p.gs), "+s"(p.gb), "+s"(p.us), "+s"(p.ub));
    return p;
}
__device__ __forceinline__ DnPtrs dn_ptrs(const QFFN& f) {
    DnPtrs p{(const GLOBAL_AS uint32_t*)f.down_q, (const GLOBAL_AS uint16_t*)f.down_s,
             (const GLOBAL_AS uint16_t*)f.down_b, f.sq, f.ss};
    asm volatile("" : "+s"(p.q), "+s"(p.s), "+s"(p.b));
    return p;
}
__device__ __forceinline__ GUPtrs pick(bool c, const GUPtrs& a, const GUPtrs& b) {
    return GUPtrs{c ? a.gq : b.gq, c ? a.uq : b.uq, c ? a.gs : b.gs, c ? a.gb : b.gb,
                  c ? a.us : b.us, c ? a.ub : b.ub, c ? a.sq : b.sq, c ? a.ss : b.ss};
}
__device__ __forceinline__ DnPtrs pick(bool c, const DnPtrs& a, const DnPtrs& b) {
    return DnPtrs{c ? a.q : b.q, c ? a.s : b.s, c ? a.b : b.b, c ? a.sq : b.sq, c ? a.ss : b.ss};
}
// Expert e's block of a global-memory array with byte stride `stride`.
template <typename T>
__device__ __forceinline__ const GLOBAL_AS T* gexpert(const GLOBAL_AS T* p, int e, uint32_t stride) {
    return (const GLOBAL_AS T*)((const GLOBAL_AS char*)p + (size_t)e * stride);
}

// The shared-gate logit of token t: the ACC_COPIES accumulator words, loads
// issued here and summed by acc_zsum where the logit is needed, so that the
// loads travel with the router logits' loads instead of before them.
struct ZLoads {
    long long q[ACC_COPIES];
};
__device__ __forceinline__ ZLoads acc_zload(const long long* __restrict__ acc, int T, int t) {
    ZLoads z;
#pragma unroll
    for (int c = 0; c < ACC_COPIES; ++c) z.q[c] = acc[((size_t)c * T + t) * ACC_STRIDE + E];
    return z;
}
__device__ __forceinline__ float acc_zsum(const ZLoads& z) {
    long long s = z.q[0];
#pragma unroll
    for (int c = 1; c < ACC_COPIES; ++c) s += z.q[c];
    return acc_val(s);
}

// Top-8 of every token (one wave per token) and the active-expert list, by
// one workgroup, into R (LDS), with the shared gate of every token.  The
// waves exchange only LDS, so the barriers here leave the caller's
// outstanding global loads in flight.
static_assert(MOE_DECODE_T <= 8, "block_route: at most two tokens per wave");
__device__ void block_route(const long long* __restrict__ acc, const float* __restrict__ bias,
                            int T, RouteRec& R, int* mark) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (T == 1) {
        // one token: its 8 experts are the active list; wave 0 sorts them by
        // id (rank = number of selected ids below its own) and writes the
        // list directly -- no marks, one barrier
        if (wave == 0) {
            const ZLoads z = acc_zload(acc, T, 0);
            const float4v v = load_logits4(acc, T, bias, 0, lane);
            const int e = wave_top8_v(v, R.ids[0], R.w[0], nullptr);
            int rank = 0;
#pragma unroll
            for (int j = 0; j < TOPK; ++j) rank += __builtin_amdgcn_readlane(e, j) < e ? 1 : 0;
            if (lane < TOPK) {
                R.active[rank] = e;
                R.tmask[rank] = 1u;
            }
            if (lane == 0) {
                R.nact = TOPK;
                R.sg[0] = 1.f / (1.f + expf(-acc_zsum(z)));
            }
        }
        pipe_barrier();
        return;
    }
    const int t0 = wave, t1 = wave + 4;
    const ZLoads z = acc_zload(acc, T, min(tid, T - 1));
    float4v v0 = {}, v1 = {};
    if (t0 < T) v0 = load_logits4(acc, T, bias, t0, lane);
    if (t1 < T) v1 = load_logits4(acc, T, bias, t1, lane);
    mark[tid] = 0;
    pipe_barrier();
    if (t0 < T) {
        const int e = wave_top8_v(v0, R.ids[t0], R.w[t0], nullptr);
        if (lane < TOPK) atomicOr((unsigned*)&mark[e], 1u << t0);
    }
    if (t1 < T) {
        const int e = wave_top8_v(v1, R.ids[t1], R.w[t1], nullptr);
        if (lane < TOPK) atomicOr((unsigned*)&mark[e], 1u << t1);
    }
    if (tid < T) R.sg[tid] = 1.f / (1.f + expf(-acc_zsum(z)));
    pipe_barrier();
    if (wave == 0) {
        // active experts in ascending id: lane l owns experts 4l .. 4l+3
        int mk[4];
        uint32_t nbelow = 0, nact = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mk[j] = mark[4 * lane + j];
            const uint64_t bj = __ballot(mk[j] != 0);
            nbelow += (uint32_t)popc64(bj & lanemask_lt());
            nact += (uint32_t)popc64(bj);
        }
        int slot = (int)nbelow;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (mk[j]) {
                R.active[slot] = 4 * lane + j;
                R.tmask[slot] = (uint32_t)mk[j];
                ++slot;
            }
        }
        if (lane == 0) R.nact = (int)nact;
    }
    pipe_barrier();
}

// First h row of slot a >= 1 (the shared slot 0 has rows 0 .. T-1): T plus
// the token counts of the active experts before it.  One wave, wave-uniform.
__device__ __forceinline__ int slot_hrow(const RouteRec& R, int a, int T) {
    if (T == 1) return a;
    const int lane = threadIdx.x & 63;
    const int n = lane < a - 1 ? __builtin_popcount(R.tmask[lane]) : 0;
    return T + (int)wave_sum((float)n);      // at most 64 small integers: exact
}

constexpr int NRB = 64;   // router workgroups (4 experts each, one per wave)

// grid (NRB + 1 + T): blocks < NRB: logits of 4 experts each (one expert
// row per wave); block NRB: shared-gate logits z[t] = x[t] . w_sg; the last
// T blocks: fp16 copy of x in chunk-slot order.  The selection itself runs
// in every routed workgroup of decode_gateup_dec (all in parallel), so this
// kernel ends as soon as its dot products are written.
__global__ __launch_bounds__(256) void route_logits_dec(const uint16_t* __restrict__ x, int T,
                                                        const uint16_t* __restrict__ wr,
                                                        const uint16_t* __restrict__ wsg,
                                                        long long* __restrict__ acc,
                                                        uint16_t* __restrict__ xh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b = blockIdx.x;
    if (b > NRB) {                        // x -> fp16, token b - NRB - 1
        const int t = b - NRB - 1;
        const size_t ci = (size_t)t * (H / 8) + threadIdx.x;
        reinterpret_cast<uint4v*>(xh)[ci] =
            bf16x8_to_f16_slots(reinterpret_cast<const uint4v*>(x)[ci]);
        return;
    }
    if (b < NRB || wave == 0) {
        uint4v xv[MOE_DECODE_T][4];
#pragma unroll
        for (int t = 0; t < MOE_DECODE_T; ++t) {
            if (t < T) {
                const uint4v* xr = reinterpret_cast<const uint4v*>(x + (size_t)t * H) + lane * 4;
#pragma unroll
                for (int c = 0; c < 4; ++c) xv[t][c] = xr[c];
            }
        }
        const int nrows = b < NRB ? E / NRB / 4 : 1;    // rows per wave
        uint4v wv[E / NRB / 4][4];
#pragma unroll
        for (int k = 0; k < E / NRB / 4; ++k) {
            if (k < nrows) {
                const uint16_t* row =
                    b < NRB ? wr + (size_t)(b * (E / NRB) + wave * (E / NRB / 4) + k) * H : wsg;
                const uint4v* wrow = reinterpret_cast<const uint4v*>(row) + lane * 4;
#pragma unroll
                for (int c = 0; c < 4; ++c) wv[k][c] = wrow[c];
            }
        }
#pragma unroll
        for (int k = 0; k < E / NRB / 4; ++k) {
            if (k >= nrows) break;
#pragma unroll
            for (int t = 0; t < MOE_DECODE_T; ++t) {
                if (t < T) {
                    float s = 0.f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t a = xv[t][c][i], bb = wv[k][c][i];
                            s = fmaf(bf16_to_f32(a & 0xFFFFu), bf16_to_f32(bb & 0xFFFFu), s);
                            s = fmaf(bf16_to_f32(a >> 16), bf16_to_f32(bb >> 16), s);
                        }
                    }
                    s = wave_sum(s);
                    if (lane < ACC_COPIES) {    // copy 0 holds the logit, the others zero
                        const int e = b < NRB ? b * (E / NRB) + wave * (E / NRB / 4) + k : E;
                        acc[((size_t)lane * T + t) * ACC_STRIDE + e] = lane == 0 ? acc_fix(s) : 0;
                    }
                }
            }
        }
    }
}

// grid (1 + 8T, I/16).  Slot 0 is the shared expert.  One token: slot s > 0
// is the s-th active routed expert (ascending id), which each routed
// workgroup finds by running the selection itself on the logits
// (block_route); the workgroup (0, 0) publishes the route record for
// decode_down_dec (and, if asked, the routing itself: ids, weights and
// shared gates).  Two or more tokens: slot 1 + 8t + j is the j-th expert of
// token t alone, found from token t's logits only; each routed workgroup of
// row chunk 0 publishes its slot's record entry (and token t's routing),
// workgroup (0, 0) the shared slot's.  Workgroup (0, 1) clears the next
// layer's logit accumulators (acc_next, if any), which the down kernel then
// adds to.  h rows (fp16, chunk-slot order) are compact: the T shared rows,
// then one row per (slot, token) -- see slot_hrow for one token.
__global__ __launch_bounds__(256) void decode_gateup_dec(const uint16_t* __restrict__ xh, int T,
                                                         const long long* __restrict__ acc,
                                                         const float* __restrict__ bias,
                                                         long long* __restrict__ acc_next,
                                                         DownRec* __restrict__ rec,
                                                         QFFN routed, QFFN shared,
                                                         uint16_t* __restrict__ hout,
                                                         int32_t* __restrict__ ids_out,
                                                         float* __restrict__ w_out,
                                                         float* __restrict__ sg_out) {
    __shared__ RouteRec R;
    __shared__ int mark[E];
    const int slot = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const GUPtrs pr = gu_ptrs(routed), ps = gu_ptrs(shared);
    int e = 0;
    const uint32_t tall = (1u << T) - 1u;
    uint32_t mask = tall;
    // two or more tokens: one slot per (token, rank) pair (slot 1 + 8t + j:
    // the j-th expert of token t, for token t alone), so a workgroup needs
    // only its own token's logits and top-8 -- not every token's, which the
    // active-expert list of the single-token path would need in every
    // workgroup.  Two tokens sharing an expert then read its weights twice.
    const bool pairs = T >= 2;
    const int town = pairs && slot > 0 ? (slot - 1) >> 3 : 0;     // this slot's token
    // loads that do not depend on the routing go out before it: the
    // activations of this slot's (first) token
    uint4v x0[4];
    {
        const uint4v* xr = reinterpret_cast<const uint4v*>(xh + (size_t)town * H) + lane * 4;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) x0[cc] = xr[cc];
    }
    if (acc_next && slot == 0 && blockIdx.y == 1)
        for (int i = threadIdx.x; i < ACC_COPIES * T * ACC_STRIDE; i += 256) acc_next[i] = 0;
    int hrow = 0;
    if (pairs) {
        const int tid = threadIdx.x;
        if (slot > 0) {
            const int j = (slot - 1) & 7;
            if (wave_id() == 0) {
                const ZLoads z = acc_zload(acc, T, town);
                const float4v v = load_logits4(acc, T, bias, town, lane);
                wave_top8_v(v, R.ids[town], R.w[town], nullptr);
                if (lane == 0) R.sg[town] = 1.f / (1.f + expf(-acc_zsum(z)));
            }
            pipe_barrier();
            e = min(max(R.ids[town][j], 0), E - 1);
            mask = 1u << town;
            hrow = T + slot - 1;
            if (blockIdx.y == 0) {
                if (tid == 0) {
                    rec->slot_e[slot] = e;
                    rec->slot_m[slot] = mask;
                    rec->slot_h[slot] = hrow;
                    rec->coef[town][slot] = R.w[town][j];
                }
                if (j == 0 && tid < TOPK) {        // the routing of token `town`
                    if (ids_out) {
                        ids_out[town * TOPK + tid] = R.ids[town][tid];
                        w_out[town * TOPK + tid] = R.w[town][tid];
                    }
                    if (sg_out && tid == 0) sg_out[town] = R.sg[town];
                }
            }
        } else if (blockIdx.y == 0) {
            // the shared slot: every token, weighted by its gate; and the
            // slot count
            if (tid < T) {
                const ZLoads z = acc_zload(acc, T, tid);
                rec->coef[tid][0] = 1.f / (1.f + expf(-acc_zsum(z)));
            }
            if (tid == 0) {
                rec->slot_e[0] = 0;
                rec->slot_m[0] = tall;
                rec->slot_h[0] = 0;
                rec->slot_e[127] = 1 + TOPK * T;
            }
        }
    } else if (slot > 0 || blockIdx.y == 0) {
        block_route(acc, bias, T, R, mark);
    }
    if (!pairs && slot == 0 && blockIdx.y == 0) {
        const int nact = min(max(R.nact, 0), TOPK * T);
        const int a = threadIdx.x;
        if (a <= nact) {
            rec->slot_e[a] = a == 0 ? 0 : R.active[a - 1];
            rec->slot_m[a] = a == 0 ? tall : R.tmask[a - 1];
            for (int t = 0; t < T; ++t) {
                float cf = R.sg[t];
                if (a > 0) {
                    cf = 0.f;
#pragma unroll
                    for (int j = 0; j < TOPK; ++j)
                        if (R.ids[t][j] == R.active[a - 1]) cf = R.w[t][j];
                }
                rec->coef[t][a] = cf;
            }
        }
        // first h rows: a per-thread serial sum (one workgroup, off the
        // other workgroups' critical path)
        if (a <= nact) {
            int hb = a == 0 ? 0 : T;
            for (int s = 0; s + 1 < a; ++s) hb += __builtin_popcount(R.tmask[s]);
            rec->slot_h[a] = hb;
        }
        if (a == 127) rec->slot_e[127] = nact + 1;
        if (ids_out && a < T * TOPK) {
            ids_out[a] = R.ids[a / TOPK][a % TOPK];
            w_out[a] = R.w[a / TOPK][a % TOPK];
        }
        if (sg_out && a < T) sg_out[a] = R.sg[a];
    }
    if (!pairs && slot > 0) {
        const int nact = min(max(R.nact, 0), TOPK * T);
        if (slot - 1 >= nact) return;
        e = min(max(R.active[slot - 1], 0), E - 1);
        mask = R.tmask[slot - 1] & tall;
        hrow = slot_hrow(R, slot, T);
    }
    const GUPtrs q = pick(slot == 0, ps, pr);
    e = __builtin_amdgcn_readfirstlane(e);
    const int n0 = blockIdx.y * 16 + wave_id() * 4;
    uint4v wq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const size_t row = n0 + (i & 3);
        const GLOBAL_AS uint32_t* qb = gexpert(i < 4 ? q.gq : q.uq, e, q.sq);
        wq[i] = ((const GLOBAL_AS uint4v*)(qb + row * (H / 8)))[lane];
    }
    float s[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const size_t row = n0 + (i & 3);
        const GLOBAL_AS uint16_t* sb = gexpert(i < 4 ? q.gs : q.us, e, q.ss);
        const GLOBAL_AS uint16_t* bb = gexpert(i < 4 ? q.gb : q.ub, e, q.ss);
        s[i] = fp16_to_f32(sb[row * (H / G) + (lane >> 1)]);
        b[i] = fp16_to_f32(bb[row * (H / G) + (lane >> 1)]);
    }
    // every weight load is in flight before the first use of one
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t mag = fp16_1024_pair();
    for (int t = 0; t < T; ++t) {
        if (!((mask >> t) & 1u)) continue;
        uint4v xp[4];
        if (t == town) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) xp[cc] = x0[cc];
        } else {
            const uint4v* xr = reinterpret_cast<const uint4v*>(xh + (size_t)t * H) + lane * 4;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) xp[cc] = xr[cc];
        }
        float sx = 0.f, off = 0.f;
        uint4v xs[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            sx = sum8_h(xp[cc], sx);
            xs[cc] = prescale_pairs(xp[cc]);
            off = pair_offset(xs[cc], off);
        }
        float acc8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float dd = 0.f;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) dd = dot8_biased(wq[i][cc], xs[cc], dd, mag);
            acc8[i] = fmaf(s[i], dd - off, b[i] * sx);
        }
        float tot[8];                                   // value i: gate row n0+i (i < 4),
        wave_sum8(acc8, tot);                           // up row n0+i-4 (i >= 4)
        if (lane < 4) {
            const int vi = lane;
            const float g = vi == 0 ? tot[0] : vi == 1 ? tot[1] : vi == 2 ? tot[2] : tot[3];
            const float u = vi == 0 ? tot[4] : vi == 1 ? tot[5] : vi == 2 ? tot[6] : tot[7];
            const float a = g / (1.f + expf(-g));
            const float hb = bf16_to_f32(f32_to_bf16(a * u));
            const int n = n0 + vi;
            hout[(size_t)hrow * I + (n & ~7) + chunk_slot(n & 7)] =
                __builtin_bit_cast(uint16_t, (_Float16)hb);
        }
        ++hrow;
    }
}

// grid (DN_WG) workgroups of DN_RG x DN_SG waves.  Wave w owns the output
// rows m0 + 4 (w % DN_RG) .. +3 (row group) and the slots a == w / DN_RG
// (mod DN_SG) (slot group); lane l covers the K range 8l .. 8l+7 of each of
// its rows, so a wave reads every row as one coalesced 256-byte segment (one
// code dword per lane) and every h row as one coalesced 1 KB piece that
// serves all four rows.  A pass issues all loads of up to DN_SPW of its
// slots before any arithmetic (one pass covers a token's nine slots).  Each
// wave sums its rows over its 64 lanes; the slot groups' partial rows are
// then added in LDS in a fixed order (deterministic).  Writes y (optional),
// res = bf16(x + y) (optional) and, for the next layer of a chain
// (wrt_next != NULL: its transposed router): its fp16 input in chunk-slot
// order (xh_next) and this
// workgroup's share of its router and shared-gate logits, added to
// accumulator copy blockIdx.x % ACC_COPIES of acc_next.  TT: 1 when T == 1,
// else MOE_DECODE_T (a bound on T).
template <int TT>
__global__ __launch_bounds__(64 * DN_WAVES) void decode_down_dec(
    const uint16_t* __restrict__ hin, int T, const DownRec* __restrict__ rec, QFFN routed,
    QFFN shared, uint16_t* __restrict__ y, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ res, uint16_t* __restrict__ xh_next,
    const uint16_t* __restrict__ wrt_next, const uint16_t* __restrict__ wsg_next,
    long long* __restrict__ acc_next) {
    __shared__ float yp[DN_SG][MOE_DECODE_T][DN_ROWS];     // partial rows of each slot group
    __shared__ float xs[MOE_DECODE_T][DN_ROWS];             // the next layer's input rows
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int rg = wave % DN_RG, sg = wave / DN_RG;
    const int m0 = blockIdx.x * DN_ROWS;
    const int mw = m0 + 4 * rg;
    const DnPtrs pr = dn_ptrs(routed), ps = dn_ptrs(shared);
    const uint32_t mag = fp16_1024_pair();
    const uint32_t tall = (1u << T) - 1u;
    const bool chained = wrt_next != nullptr;
    // the record first: one load per array and lane, all issued together,
    // then picked apart with lane reads
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 re = reinterpret_cast<const u32x2*>(rec->slot_e)[lane];
    const u32x2 rm = reinterpret_cast<const u32x2*>(rec->slot_m)[lane];
    const u32x2 rh = reinterpret_cast<const u32x2*>(rec->slot_h)[lane];
    u32x2 rc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) rc[t] = reinterpret_cast<const u32x2*>(rec->coef[t])[lane];
    // then the loads that need no routing, needed only at the very end: the
    // next layer's transposed router rows m0 .. m0 + DN_ROWS - 1 (thread e:
    // entry e of each, coalesced 512-byte rows) and the same entries of its
    // shared-gate vector (buffer loads with no branch around them: a missing
    // next layer is an empty range, so the wait counts of the loads issued
    // before stay exact)
    static_assert(64 * DN_WAVES >= E, "one thread per expert for the router partials");
    const __amdgpu_buffer_rsrc_t rwt = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(wrt_next), 0, chained ? (uint32_t)(H * E * 2) : 0u, 0x00020000);
    const __amdgpu_buffer_rsrc_t rwg = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(wsg_next), 0, chained ? (uint32_t)(H * 2) : 0u, 0x00020000);
    uint16_t wt[DN_ROWS], wg[DN_ROWS];
#pragma unroll
    for (int k = 0; k < DN_ROWS; ++k) {
        const uint32_t ot = tid < E ? (uint32_t)(((m0 + k) * E + tid) * 2) : 0x80000000u;
        wt[k] = __builtin_amdgcn_raw_buffer_load_b16(rwt, ot, 0, 0);
        wg[k] = __builtin_amdgcn_raw_buffer_load_b16(rwg, (uint32_t)((m0 + k) * 2), 0, 0);
    }
    // the whole record is needed next (without this the compiler issues the
    // later record loads only after waiting for the first one)
    asm volatile("" ::"v"(re), "v"(rm), "v"(rh));
#pragma unroll
    for (int t = 0; t < TT; ++t) asm volatile("" ::"v"(rc[t]));
    auto slot_word = [](u32x2 v, int a) -> uint32_t {
        const uint32_t lo = __builtin_amdgcn_readlane(v[0], a >> 1);
        const uint32_t hi = __builtin_amdgcn_readlane(v[1], a >> 1);
        return (a & 1) ? hi : lo;
    };
    const int nslots = min(max((int)__builtin_amdgcn_readlane(re[1], 63), 1), TOPK * T + 1);
    const int hmax = (TOPK + 1) * T - 1;
    float acc[4][TT];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[r][t] = 0.f;
    // the residual input, for the output lanes (no branch around the load)
    const int xi = min(lane, T * 4 - 1);
    const uint16_t xin = x[(size_t)(xi >> 2) * H + mw + (xi & 3)];
    // one pass: this wave's slots a0 + sg + DN_SG * k, k < DN_SPW
    auto pass = [&](const int a0) {
        uint32_t cw[DN_SPW][4];
        uint16_t sb[DN_SPW][8];
        uint4v h1[DN_SPW];
#pragma unroll
        for (int k = 0; k < DN_SPW; ++k) {
            // slots past the last one repeat a valid slot's loads (unused)
            const int a = min(a0 + sg + DN_SG * k, nslots - 1);
            const int e = min(max((int)slot_word(re, a), 0), E - 1);
            const DnPtrs q = pick(a == 0, ps, pr);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const size_t row = mw + r;
                cw[k][r] = (gexpert(q.q, e, q.sq) + row * (I / 8))[lane];
                sb[k][r] = gexpert(q.s, e, q.ss)[row * (I / G) + (lane >> 3)];
                sb[k][4 + r] = gexpert(q.b, e, q.ss)[row * (I / G) + (lane >> 3)];
            }
            const int hr = min(max((int)slot_word(rh, a), 0), hmax);
            h1[k] = reinterpret_cast<const uint4v*>(hin + (size_t)hr * I)[lane];
        }
#pragma unroll
        for (int k = 0; k < DN_SPW; ++k) {
            const int a = a0 + sg + DN_SG * k;
            if (a >= nslots) continue;     // (a guard, not a break: the loop unrolls fully)
            const uint32_t mk = slot_word(rm, a) & tall;
            int hrow = min(max((int)slot_word(rh, a), 0), hmax);
            bool firsttok = true;
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if (t >= T || !((mk >> t) & 1u)) continue;
                const float coef = __builtin_bit_cast(float, slot_word(rc[t], a));
                uint4v hv = h1[k];
                if (!firsttok)
                    hv = reinterpret_cast<const uint4v*>(hin + (size_t)min(hrow, hmax) * I)[lane];
                firsttok = false;
                ++hrow;
                const float sx = sum8_h(hv, 0.f);
                const uint4v hs = prescale_pairs(hv);
                const float off = pair_offset(hs, 0.f);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dd = dot8_biased(cw[k][r], hs, 0.f, mag);
                    acc[r][t] += coef * fmaf(fp16_to_f32(sb[k][r]), dd - off,
                                             fp16_to_f32(sb[k][4 + r]) * sx);
                }
            }
        }
    };
    // one token has at most 9 slots, which one pass covers: no loop whose
    // head would make the wait counts of the loads above conservative
    static_assert(DN_SG * DN_SPW >= 1 + TOPK, "one pass covers a token's slots");
    if constexpr (TT == 1) {
        pass(0);
    } else {
        for (int a0 = 0; a0 < nslots; a0 += DN_SG * DN_SPW) pass(a0);
    }
    // this wave's partial rows over its 64 lanes, then the slot groups' sums
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if (t >= T) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = wave_sum(acc[r][t]);
            if (lane == 0) yp[sg][t][4 * rg + r] = v;
        }
    }
    __syncthreads();
    if (sg == 0 && lane < T * 4) {
        // lane r + 4t of each row group's first wave: row mw + r of token t
        const int t = lane >> 2, r = lane & 3, rr = 4 * rg + r;
        float v = yp[0][t][rr];
#pragma unroll
        for (int g = 1; g < DN_SG; ++g) v += yp[g][t][rr];
        const uint32_t yb = f32_to_bf16(v);
        const size_t o = (size_t)t * H + mw + r;
        if (y) y[o] = (uint16_t)yb;
        const uint32_t xb = f32_to_bf16(bf16_to_f32(xin) + bf16_to_f32(yb));
        if (res) res[o] = (uint16_t)xb;
        xs[t][rr] = bf16_to_f32(xb);
        if (chained) {
            const int m = mw + r;
            xh_next[(size_t)t * H + (m & ~7) + chunk_slot(m & 7)] =
                __builtin_bit_cast(uint16_t, (_Float16)bf16_to_f32(xb));
        }
    }
    if (!chained) return;
    __syncthreads();
    // this workgroup's partial router and shared-gate logits of the next
    // layer (thread e < 256: logit e, thread 256 - 256 = the shared gate is
    // done by thread 0 as a second sum): DN_ROWS exact bf16 products summed
    // in fp32 in order
    long long* cp = acc_next + (size_t)(blockIdx.x % ACC_COPIES) * T * ACC_STRIDE;
    if (tid < E) {
        for (int t = 0; t < T; ++t) {
            float p = 0.f, z = 0.f;
#pragma unroll
            for (int k = 0; k < DN_ROWS; ++k) {
                p = fmaf(bf16_to_f32(wt[k]), xs[t][k], p);
                z = fmaf(bf16_to_f32(wg[k]), xs[t][k], z);
            }
            atomicAdd(reinterpret_cast<unsigned long long*>(cp + (size_t)t * ACC_STRIDE + tid),
                      (unsigned long long)acc_fix(p));
            if (tid == 0)
                atomicAdd(reinterpret_cast<unsigned long long*>(cp + (size_t)t * ACC_STRIDE + E),
                          (unsigned long long)acc_fix(z));
        }
    }
}

// w_router bf16 [256][2048] -> w_router_t bf16 [2048][256], through a 64 x
// 64 tile in LDS (grid (2048 / 64, 256 / 64), 256 threads).
__global__ __launch_bounds__(256) void router_transpose(const uint16_t* __restrict__ wr,
                                                        uint16_t* __restrict__ wrt) {
    __shared__ uint16_t tile[64][66];
    const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        tile[r][c] = wr[(size_t)(e0 + r) * H + k0 + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        wrt[(size_t)(k0 + r) * E + e0 + c] = tile[c][r];
    }
}

void launch_router_transpose(const uint16_t* wr, uint16_t* wrt, hipStream_t st) {
    hipLaunchKernelGGL(router_transpose, dim3(H / 64, E / 64), dim3(256), 0, st, wr, wrt);
}

size_t route_rec_bytes() { return sizeof(DownRec); }
size_t route_acc_bytes(int T) { return (size_t)2 * ACC_COPIES * T * ACC_STRIDE * sizeof(long long); }

// One few-token layer.  first: the layer computes its own router logits
// (route_logits_dec) into acc_cur; otherwise a previous chained layer left
// them there.  next (optional): the following layer of a chain, whose
// router logits go to acc_next and whose fp16 input goes to xh.
void launch_layer_decode_small(const uint16_t* x, int T, const moe_layer& L, bool first,
                               long long* acc_cur, long long* acc_next, const moe_layer* next,
                               uint16_t* xh, uint16_t* hbuf, void* rec, uint16_t* y,
                               uint16_t* res, int32_t* ids_out, float* w_out, float* sg_out,
                               hipStream_t st) {
    const QFFN routed = qffn_view(L.routed), shared = qffn_view(L.shared);
    DownRec* R = static_cast<DownRec*>(rec);
    if (first)
        hipLaunchKernelGGL(route_logits_dec, dim3(NRB + 1 + T), dim3(256), 0, st, x, T, L.w_router,
                           L.w_shared_gate, acc_cur, xh);
    hipLaunchKernelGGL(decode_gateup_dec, dim3(1 + TOPK * T, I / 16), dim3(256), 0, st, xh, T,
                       acc_cur, L.router_bias, next ? acc_next : nullptr, R, routed, shared, hbuf,
                       ids_out, w_out, sg_out);
    const dim3 g(DN_WG), b(64 * DN_WAVES);
    if (T == 1)
        hipLaunchKernelGGL(decode_down_dec<1>, g, b, 0, st, hbuf, T, R, routed, shared, y, x, res,
                           next ? xh : nullptr, next ? next->w_router_t : nullptr,
                           next ? next->w_shared_gate : nullptr, next ? acc_next : nullptr);
    else
        hipLaunchKernelGGL(decode_down_dec<MOE_DECODE_T>, g, b, 0, st, hbuf, T, R, routed, shared, y,
                           x, res, next ? xh : nullptr, next ? next->w_router_t : nullptr,
                           next ? next->w_shared_gate : nullptr, next ? acc_next : nullptr);
}

void launch_route_select(const float* logits, const uint16_t* x, const uint16_t* wsg, int T,
                         int32_t* ids, float* wts, float* sg, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv, Tile* tiles, int* tile_count,
                         uint16_t* xh, hipStream_t st) {
    hipLaunchKernelGGL(route_select, dim3(1), dim3(256), 0, st, logits, x, wsg, T, ids, wts, sg,
                       counts, offsets, perm, inv, tiles, tile_count, xh);
}

void launch_decode_gateup(const uint16_t* xh, int T, const int32_t* perm, const Tile* tiles,
                          const int* tile_count, int max_tiles, const QFFN& routed,
                          const QFFN& shared, uint16_t* hbuf, hipStream_t st) {
    hipLaunchKernelGGL(decode_gateup, dim3(max_tiles, I / 16), dim3(256), 0, st, xh, T, perm, tiles,
                       tile_count, routed, shared, hbuf);
}

void launch_decode_down_combine(const uint16_t* hbuf, int T, const int32_t* perm,
                                const Tile* tiles, const int* tile_count, const float* wts,
                                const float* sg, const QFFN& routed, const QFFN& shared,
                                uint16_t* y, const uint16_t* x, uint16_t* res, hipStream_t st) {
    hipLaunchKernelGGL(decode_down_combine, dim3(H / 4), dim3(256), 0, st, hbuf, T, perm, tiles,
                       tile_count, wts, sg, routed, shared, y, x, res);
}

}  // namespace moe
