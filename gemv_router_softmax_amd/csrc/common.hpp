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
