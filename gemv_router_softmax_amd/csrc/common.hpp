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
// (group 256 = the shared expert) per tile.
constexpr int MT_ROWS = 128;

struct Tile {
    int group;     // 0..255 routed expert, 256 shared expert
    int row0;      // first row in the permuted row space (shared rows start at 8T)
    int nrows;     // 1..MT_ROWS
    int pad;
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef uint16_t ushort8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float fp16_to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Exact-code dot products for the decode GEMVs.  A code word holds eight
// 4-bit codes q0..q7 (q_k in bits 4k..4k+3).  ((w >> 4i) & 0x000F000F) |
// 0x43004300 is the bf16 pair (128 + q_i, 128 + q_{i+4}) -- exact, since bf16
// spacing at 128 is 1 -- so v_dot2_f32_bf16 against the activation pair
// (a_i, a_{i+4}) accumulates sum_k a_k (128 + q_k).  With sa = sum_k a_k the
// group's contribution is  s * (dot - 128 sa) + b * sa = s * dot + (b - 128 s) sa.
__device__ __forceinline__ float dot8_codes(uint32_t w, uint4v apairs, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = ((w >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, p),
                                              __builtin_bit_cast(bf16x2v, apairs[i]), acc, false);
    }
    return acc;
}

// Sum of the eight bf16 activations of a pair vector.
__device__ __forceinline__ float sum8_bf16(uint4v apairs, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, 0x3F803F80u),
                                              __builtin_bit_cast(bf16x2v, apairs[i]), acc, false);
    return acc;
}

// Eight natural-order bf16 values (a0,a1),(a2,a3),(a4,a5),(a6,a7) -> the
// code-pair order (a0,a4),(a1,a5),(a2,a6),(a3,a7).
__device__ __forceinline__ uint4v pair_i_i4(uint4v v) {
    uint4v r;
    r[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
    return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Position of element k (0..7) inside an 8-element chunk of the fp16
// operand layout used by the MFMA kernels.  The dequantiser produces the
// eight codes of a word in the order k = 0,4,1,5,2,6,3,7 (two nibbles per
// packed half2), so activations are stored in that same order.
__device__ __forceinline__ int chunk_slot(int k) { return ((k & 3) << 1) | (k >> 2); }

}  // namespace moe
