// common.hpp -- shared device-side definitions of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int H = MOE_HIDDEN;     // 2048
constexpr int I = MOE_INTER;      // 512
constexpr int E = MOE_EXPERTS;    // 256
constexpr int TOPK = MOE_TOPK;    // 8
constexpr int G = MOE_GROUP;      // 64
constexpr int WAVE = 64;

// Row tiles of the grouped expert work: at most MT_ROWS rows of one expert
// (group 256 = the shared expert) per tile at large T, MT_MIN_ROWS at small
// T; a group is split into equal tiles (160 covers the busiest expert of a
// uniformly routed 4096-token batch in one tile).
constexpr int MT_ROWS = 160;
constexpr int MT_MIN_ROWS = 32;

// Permutation of 8T (token, rank) entries: one workgroup sorts up to
// PERM_SMALL_MAX entries alone; above that the entries are histogrammed,
// scanned and scattered in chunks of PERM_CHUNK (the layer call's top-8
// kernel adds each token's eight picks to its chunk's histogram).
constexpr int PERM_CHUNK = 512;
constexpr int PERM_SMALL_MAX = 1024;

// Device view of one expert stack: the nine arrays and the byte distance
// between consecutive experts in the code arrays (sq) and in the
// scale/bias arrays (ss) -- the dense sizes, or the caller's expert stride.
struct QFFN {
    const uint32_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b, *down_s, *down_b;
    uint32_t sq, ss;
};

constexpr uint32_t DENSE_SQ = I * H / 2;         // one expert's codes: 524288 B (any matrix)
constexpr uint32_t DENSE_SS = I * (H / G) * 2;   // one expert's scales: 32768 B (any matrix)
static_assert(DENSE_SQ == H * I / 2 && DENSE_SS == H * (I / G) * 2, "square per-expert blocks");

inline QFFN qffn_view(const moe_qffn& q) {
    const bool dense = q.expert_stride == 0;
    return QFFN{q.gate_q, q.up_q, q.down_q, q.gate_s, q.gate_b, q.up_s, q.up_b, q.down_s, q.down_b,
                dense ? DENSE_SQ : (uint32_t)q.expert_stride,
                dense ? DENSE_SS : (uint32_t)q.expert_stride};
}

// Base of expert e's block in an array with byte stride `stride`.
template <typename P>
__device__ __forceinline__ P expert_at(P p, int e, uint32_t stride) {
    typedef const char* CP;
    return (P)((CP)p + (size_t)e * stride);
}

// The tile count's workspace slot also holds the grouped GEMMs' work
// counters, one per XCD and GEMM (gate/up: words 8..15, down: 16..23),
// zeroed by the tile planner before each use.
constexpr int GEMM_CTR_GATEUP = 8, GEMM_CTR_DOWN = 16, TILE_COUNT_WORDS = 24;

struct Tile {
    int group;     // 0..255 routed expert, 256 shared expert
    int row0;      // first row in the permuted row space (shared rows start at 8T)
    int nrows;     // 1..MT_ROWS (1..MT_MIN_ROWS for small-T plans)
    int pad;
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef uint16_t ushort8v __attribute__((ext_vector_type(8)));

// Position of element k (0..7) inside an 8-element chunk of the fp16
// operand layout used by every expert kernel.  The dequantiser produces the
// eight codes of a word in the order k = 0,4,1,5,2,6,3,7 (two nibbles per
// packed half2), so activations are stored in that same order.
__device__ __forceinline__ int chunk_slot(int k) { return ((k & 3) << 1) | (k >> 2); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// float -> bf16 bits, round to nearest even (one v_cvt_pk_bf16_f32 on this
// chip; it agrees bit for bit with the integer rounding sequence on ties,
// subnormals and large values); NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float fp16_to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
}

// Exact-code dot products for the decode GEMVs.  A code word holds eight
// 4-bit codes q0..q7 (q_k in bits 4k..4k+3).  ((w >> 4i) & 0x000F000F) |
// 0x64006400 is the fp16 pair (1024 + q_i, 1024 + q_{i+4}); one packed
// subtraction leaves (q_i, q_{i+4}) exactly, and v_dot2_f32_f16 against the
// activation pair (a_i, a_{i+4}) -- activations stored as fp16 in chunk-slot
// order -- adds a_i q_i + a_{i+4} q_{i+4} to an fp32 accumulator (exact
// products).  The bf16 variant of the dot instruction is not used: it drops
// addends far below the accumulator instead of keeping fp32 precision.
__device__ __forceinline__ float dot8_codes(uint32_t w, uint4v apairs, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
        const half2v qh = __builtin_bit_cast(half2v, p) - (half2v){(_Float16)1024.f, (_Float16)1024.f};
        // (copy the element to a scalar first: bit-casting an ext-vector element
        // directly reads element 0 with this compiler)
        const uint32_t ai = apairs[i];
        acc = __builtin_amdgcn_fdot2(qh, __builtin_bit_cast(half2v, ai), acc, false);
    }
    return acc;
}

// Sum of the eight fp16 activations of a pair vector.
__device__ __forceinline__ float sum8_h(uint4v apairs, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ai = apairs[i];
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, 0x3C003C00u),
                                     __builtin_bit_cast(half2v, ai), acc, false);
    }
    return acc;
}

// The same dot product in 9 instructions per code word instead of 15, for
// the latency-bound decode kernels.  OR-ing 0x6400 into each half of
//   w & 0x000F000F, w & 0x00F000F0, (w >> 8) & 0x000F000F, (w >> 8) & 0x00F000F0
// gives the exact fp16 pairs 1024 + (q0, q4), 1024 + 16 (q1, q5),
// 1024 + (q2, q6), 1024 + 16 (q3, q7) without any shift of the odd nibbles
// and without the subtraction.  Against activation pairs whose second and
// fourth pair are pre-scaled by 1/16 (prescale_pairs) the dot products add
// up to sum_k q_k x_k plus a constant part, pair_offset() of the same
// pre-scaled pairs, which the caller subtracts once per row.
__device__ __forceinline__ uint4v prescale_pairs(uint4v a) {
    const half2v k = {(_Float16)0.0625f, (_Float16)0.0625f};
    uint4v r = a;
    const uint32_t a1 = a[1], a3 = a[3];
    r[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a1) * k);
    r[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a3) * k);
    return r;
}

// 0x64006400 in a vector register the compiler cannot see through: with the
// mask in a scalar register, each nibble pair is then one v_and_or_b32 (a
// VOP3 instruction takes no literal operand, and two literals would split
// it into an AND and an OR).
__device__ __forceinline__ uint32_t fp16_1024_pair() {
    uint32_t v;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(v));
    return v;
}

// mag: fp16_1024_pair(), taken once per kernel.
__device__ __forceinline__ float dot8_biased(uint32_t w, uint4v xs, float acc, uint32_t mag) {
    const uint32_t w8 = w >> 8;
    const uint32_t p[4] = {(w & 0x000F000Fu) | mag, (w & 0x00F000F0u) | mag,
                           (w8 & 0x000F000Fu) | mag, (w8 & 0x00F000F0u) | mag};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t xi = xs[i];
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, p[i]),
                                     __builtin_bit_cast(half2v, xi), acc, false);
    }
    return acc;
}

// The part of dot8_biased that does not depend on the codes: 1024 times the
// sum of the pre-scaled pairs (exact products, fp32 accumulation).
__device__ __forceinline__ float pair_offset(uint4v xs, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t xi = xs[i];
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, 0x64006400u),
                                     __builtin_bit_cast(half2v, xi), acc, false);
    }
    return acc;
}

// Eight natural-order bf16 values -> fp16 in chunk-slot order (k = 0,4,1,5,
// 2,6,3,7), the activation layout of every expert kernel.  bf16 -> fp16 is
// exact for magnitudes in [2^-14, 65504]; smaller values keep fp16's
// subnormal spacing 2^-24.
__device__ __forceinline__ uint4v bf16x8_to_f16_slots(uint4v v) {
    uint16_t o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float f = bf16_to_f32((v[k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
        o[chunk_slot(k)] = __builtin_bit_cast(uint16_t, (_Float16)f);
    }
    uint4v w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)o[2 * i] | ((uint32_t)o[2 * i + 1] << 16);
    return w;
}

// Lane exchanges that stay in the vector ALU (no LDS round trip).
// dpp_f<CTL>: v of another lane of the same 16-lane row -- quad_perm
// 1,0,3,2 (lane ^ 1), quad_perm 2,3,0,1 (lane ^ 2), row_half_mirror (lane
// i <-> 7 - i within 8), row_mirror (lane i <-> 15 - i within 16).
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int CTL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTL,
                                                                 0xF, 0xF, false));
}

// Sum of v over each 16-lane row, in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    v += dpp_f<DPP_MIRROR>(v);
    return v;
}

// Sum of v over the wave, as a wave-uniform value: row sums by DPP, then
// row_bcast:15 adds row 0 into row 1 and row 2 into row 3 (rows 0 and 2 add
// the 0 of their masked-off lanes), row_bcast:31 adds rows 0-1 into rows
// 2-3, and lane 63 holds the total.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142,
                                                               0xA, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143,
                                                               0xC, 0xF, false));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}


}  // namespace moe
