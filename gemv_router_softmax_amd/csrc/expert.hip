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
// Prefill (grouped GEMM on MFMA): expert_gemm below.
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

// (x & m) | o in one instruction.  A VOP3 instruction on this chip may read
// only one scalar operand, so the mask is an SGPR and o stays in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
    return r;
}

// Eight codes of one word -> fp16 weights w = q*s + b, in chunk-slot order
// (k = 0,4,1,5,2,6,3,7).  (0x6400 | q) is the fp16 value 1024 + q, so one
// packed subtraction recovers q exactly and one packed FMA applies the
// group's scale and bias with a single rounding.
__device__ __forceinline__ half8 dequant8(uint32_t w, half2v s2, half2v b2) {
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = and_or(w >> (4 * i), 0x000F000Fu, 0x64006400u);
        half2v h = __builtin_bit_cast(half2v, p) - (half2v){(_Float16)1024.f, (_Float16)1024.f};
        h = __builtin_elementwise_fma(h, s2, b2);
        r[2 * i] = h[0];
        r[2 * i + 1] = h[1];
    }
    return r;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum GemmMode { GM_GATEUP = 0, GM_DOWN_F32 = 1, GM_DOWN_F16W = 2 };

// Raw buffer resource over [p, p + bytes): loads beyond the range return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

struct GemmArgs {
    const uint16_t* ain;
    uint32_t ain_bytes;
    int T;
    const int32_t* perm;
    uint16_t* hout;
    float* dout32;
    uint16_t* dout16;
    const float* wts;
    const float* sg;
};

constexpr int GW = 8;                 // waves per GEMM workgroup
constexpr int GSTAGES = 3;            // A pipeline depth (LDS buffers)
constexpr int CHB = 128 * 2;          // bytes per A row per 128-wide K chunk
constexpr int BUFB = MT_ROWS * CHB;   // bytes per A buffer (32 KB)

// s_waitcnt immediate: wait until at most n vector-memory operations of
// this wave are outstanding (loads retire in issue order); expcnt and
// lgkmcnt are left at their maximum (no wait).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int LGKM0_IMM = 15 | (3 << 14) | (7 << 4);   // lgkmcnt(0) only

// Workgroup barrier inside a software pipeline.  __syncthreads() also acts
// as a memory fence, which makes every wave wait for ALL of its outstanding
// vector-memory loads -- including the prefetches meant to stay in flight.
// Here the caller has already waited (s_waitcnt vmcnt) for exactly the loads
// the next stage needs; this drains only the LDS counter and synchronises
// execution.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void pipe_barrier() {
    __builtin_amdgcn_s_waitcnt(LGKM0_IMM);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One row tile (NMT 16-row m-tiles, NMT*16 >= nrows) x one column block of
// the grouped GEMM.
//   8 waves; wave w owns 64 weight columns (gate/up: 32 gate + the same 32
//   up columns; down: 64 output columns) for ALL rows of the tile, so every
//   code word is dequantised once per tile and column block.
//   A: 128-wide K chunks of the activation rows (gathered by token for
//   gate/up) move from global memory straight into LDS (buffer loads with an
//   LDS destination) through a 3-stage pipeline; the 16 B pieces of a row are
//   XOR-swizzled by (row & 15) so the 16 rows of an MFMA operand read hit 16
//   distinct LDS bank groups.
//   B: each lane loads 16 B of codes per column per chunk, one chunk ahead,
//   and rebuilds fp16 weights in registers (dequant8).
//   MFMA: v_mfma_f32_16x16x32_f16, fp32 accumulation.
template <int KDIM, int MODE, int NMT>
__device__ __forceinline__ void gemm_tile(const GemmArgs& A, const Tile& tl, const moe_qffn& q,
                                          int e, int nb, uint8_t* As, float* coef) {
    constexpr bool GATEUP = MODE == GM_GATEUP;
    constexpr int NCH = KDIM / 128;              // K chunks
    constexpr int WPR = KDIM / 8;                // code words per weight row
    constexpr int SPR = KDIM / G;                // groups per weight row
    constexpr int ROWS_W = GATEUP ? I : H;       // weight rows per expert
    constexpr int NBW = GATEUP ? GW * 32 : GW * 64;   // output columns per block
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, j = lane >> 4;
    const int nr = tl.nrows;

    // ---- B: resources for the expert's matrices and per-lane offsets
    const uint32_t qbytes = (uint32_t)ROWS_W * WPR * 4, sbytes = (uint32_t)ROWS_W * SPR * 2;
    __amdgpu_buffer_rsrc_t rq[2], rs[2], rb[2];
    if (GATEUP) {
        rq[0] = buf_rsrc(q.gate_q + (size_t)e * ROWS_W * WPR, qbytes);
        rq[1] = buf_rsrc(q.up_q + (size_t)e * ROWS_W * WPR, qbytes);
        rs[0] = buf_rsrc(q.gate_s + (size_t)e * ROWS_W * SPR, sbytes);
        rs[1] = buf_rsrc(q.up_s + (size_t)e * ROWS_W * SPR, sbytes);
        rb[0] = buf_rsrc(q.gate_b + (size_t)e * ROWS_W * SPR, sbytes);
        rb[1] = buf_rsrc(q.up_b + (size_t)e * ROWS_W * SPR, sbytes);
    } else {
        rq[0] = rq[1] = buf_rsrc(q.down_q + (size_t)e * ROWS_W * WPR, qbytes);
        rs[0] = rs[1] = buf_rsrc(q.down_s + (size_t)e * ROWS_W * SPR, sbytes);
        rb[0] = rb[1] = buf_rsrc(q.down_b + (size_t)e * ROWS_W * SPR, sbytes);
    }
    uint32_t qoff[4], soff[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int n = GATEUP ? nb * NBW + wave * 32 + (nt & 1) * 16 + r
                             : nb * NBW + wave * 64 + nt * 16 + r;
        qoff[nt] = ((uint32_t)n * WPR + 4 * j) * 4;
        soff[nt] = ((uint32_t)n * SPR + (j >> 1)) * 2;
    }
    auto mat = [](int nt) { return GATEUP ? (nt >> 1) : 0; };

    // ---- A: per-lane source offsets of the 4 pieces moved per chunk.
    // Load instruction i of wave w fills tile rows w*16 + 4i .. +3 (1 KB):
    // lane -> row w*16 + 4i + (lane >> 4), LDS slot (lane & 15), holding the
    // row's piece (lane & 15) ^ (row & 15).
    const __amdgpu_buffer_rsrc_t ra = buf_rsrc(A.ain, A.ain_bytes);
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wave * 16 + i * 4 + (lane >> 4);
        const int rr = row < nr ? row : 0;
        const int src = GATEUP ? row_token(tl.row0 + rr, A.T, A.perm) : tl.row0 + rr;
        aoff[i] = (uint32_t)src * (uint32_t)(KDIM * 2) + 16u * (uint32_t)((lane & 15) ^ (row & 15));
    }
    // rows this wave moves: w*16 .. w*16+15, needed only below NMT*16
    const bool amove = wave * 16 < NMT * 16;
    auto issue_a = [&](int kc) {
        uint8_t* dst = As + (kc % GSTAGES) * BUFB + wave * 16 * CHB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (amove)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(dst + i * 4 * CHB), 16,
                                                         aoff[i], kc * CHB, 0, 0);
    };

    float4v acc[NMT][4];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (float4v){0.f, 0.f, 0.f, 0.f};

    // B of the next chunk is loaded into registers one chunk ahead.  Scale
    // and bias stay raw fp16 bits until they are used, so that no arithmetic
    // on a just-issued load forces the wave to wait for it.
    uint4v bw[4];
    uint32_t bs[4], bb[4];
    issue_a(0);
    if (NCH > 1) issue_a(1);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        bw[nt] = __builtin_amdgcn_raw_buffer_load_b128(rq[mat(nt)], qoff[nt], 0, 0);
        bs[nt] = __builtin_amdgcn_raw_buffer_load_b16(rs[mat(nt)], soff[nt], 0, 0);
        bb[nt] = __builtin_amdgcn_raw_buffer_load_b16(rb[mat(nt)], soff[nt], 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kc = 0; kc < NCH; ++kc) {
        uint4v cw[4];
        half2v cs[4], cb[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            cw[nt] = bw[nt];
            cs[nt] = splat_h((uint16_t)bs[nt]);
            cb[nt] = splat_h((uint16_t)bb[nt]);
        }
        if (kc + 1 < NCH) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                bw[nt] = __builtin_amdgcn_raw_buffer_load_b128(rq[mat(nt)], qoff[nt], (kc + 1) * 64, 0);
                bs[nt] = __builtin_amdgcn_raw_buffer_load_b16(rs[mat(nt)], soff[nt], (kc + 1) * 4, 0);
                bb[nt] = __builtin_amdgcn_raw_buffer_load_b16(rb[mat(nt)], soff[nt], (kc + 1) * 4, 0);
            }
        }
        const bool more = kc + 2 < NCH;
        if (more) issue_a(kc + 2);
        const uint8_t* Ab = As + (kc % GSTAGES) * BUFB;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8 a[NMT], bf[4];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
                a[mt] = *reinterpret_cast<const half8*>(&Ab[(mt * 16 + r) * CHB + 16 * ((4 * j + s) ^ r)]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) bf[nt] = dequant8(cw[nt][s], cs[nt], cb[nt]);
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        }
        // chunk kc+1 (A and B) must have landed; chunk kc+2's A may stay in flight
        if (more && amove) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        pipe_barrier();
    }

    if constexpr (GATEUP) {
        // h = bf16(silu(g) * u) stored as fp16 (exact) in chunk-slot order,
        // staged through LDS for 16-byte stores.
        uint16_t* Hs = reinterpret_cast<uint16_t*>(As);    // [128][NBW + 8] halves
        constexpr int HST = NBW + 8;                         // NBW h columns per block
        static_assert(MT_ROWS * HST * 2 <= GSTAGES * BUFB, "staging tile exceeds the A buffers");
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = mt * 16 + 4 * j + i;
                    const int col = wave * 32 + nt * 16 + r;
                    const float g = acc[mt][nt][i], u = acc[mt][nt + 2][i];
                    const float hv = (g / (1.f + __expf(-g))) * u;
                    const _Float16 hh = (_Float16)bf16_to_f32(f32_to_bf16(hv));
                    Hs[row * HST + (col & ~7) + chunk_slot(col & 7)] =
                        __builtin_bit_cast(uint16_t, hh);
                }
            }
        }
        __syncthreads();
        constexpr int PR = NBW / 8;          // 16-byte pieces per staged row
        for (int c = tid; c < nr * PR; c += GW * 64) {
            const int row = c / PR, col = (c % PR) * 8;
            *reinterpret_cast<uint4v*>(A.hout + (size_t)(tl.row0 + row) * I + nb * NBW + col) =
                *reinterpret_cast<const uint4v*>(&Hs[row * HST + col]);
        }
    } else if constexpr (MODE == GM_DOWN_F32) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = mt * 16 + 4 * j + i;
                    if (row < nr)
                        A.dout32[(size_t)(tl.row0 + row) * H + nb * NBW + wave * 64 + nt * 16 + r] =
                            acc[mt][nt][i];
                }
            }
        }
    } else {
        // fp16 rows of coef * d, staged through LDS for 16-byte stores, one
        // half of the block's columns (four waves) at a time
        uint16_t* Ds = reinterpret_cast<uint16_t*>(As);
        constexpr int HALF = NBW / 2;
        constexpr int DST = HALF + 8;
        static_assert(MT_ROWS * DST * 2 <= GSTAGES * BUFB, "staging tile exceeds the A buffers");
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if ((wave >> 2) == hf) {
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int row = mt * 16 + 4 * j + i;
                            const int col = (wave & 3) * 64 + nt * 16 + r;
                            const float v = row < nr ? coef[row] * acc[mt][nt][i] : 0.f;
                            Ds[row * DST + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
                        }
                    }
                }
            }
            __syncthreads();
            constexpr int PR = HALF / 8;
            for (int c = tid; c < nr * PR; c += GW * 64) {
                const int row = c / PR, col = (c % PR) * 8;
                *reinterpret_cast<uint4v*>(A.dout16 + (size_t)(tl.row0 + row) * H + nb * NBW +
                                           hf * HALF + col) =
                    *reinterpret_cast<const uint4v*>(&Ds[row * DST + col]);
            }
            __syncthreads();
        }
    }
}

// Grouped expert GEMM: a 1-D grid of (row tile, column block) work items.
// Work is split into 8 contiguous ranges, one per XCD (workgroup ids are
// dealt to the 8 XCDs round-robin), so the column blocks of a tile run back
// to back on the same XCD and re-read its activation rows from that XCD's
// L2.  The tile's m-tile count selects a fully unrolled instance.
//   GM_GATEUP:    K = 2048, 256 gate + 256 up columns per block,
//                 h = bf16(silu(g) u) written as fp16 in chunk-slot order
//   GM_DOWN_F32:  K = 512, 512 output columns per block, fp32 rows
//   GM_DOWN_F16W: as above, fp16 rows pre-multiplied by the routing weight
//                 (or the shared gate) for the fused combine
template <int KDIM, int MODE>
__global__ __launch_bounds__(GW * 64, 1) void expert_gemm(GemmArgs args,
                                                          const Tile* __restrict__ tiles,
                                                          const int* __restrict__ tile_count,
                                                          moe_qffn routed, moe_qffn shared) {
    constexpr int NB = MODE == GM_GATEUP ? I / (GW * 32) : H / (GW * 64);
    __shared__ __attribute__((aligned(16))) uint8_t As[GSTAGES * BUFB];
    __shared__ float coef[MT_ROWS];
    const int total = *tile_count * NB;
    const int per_xcd = (total + 7) / 8;
    const int local = blockIdx.x / 8;
    if (local >= per_xcd) return;
    const int w = (blockIdx.x % 8) * per_xcd + local;
    if (w >= total) return;
    const Tile tl = tiles[w / NB];
    const int nb = w % NB;
    const bool sh = tl.group >= E;
    const int e = sh ? 0 : tl.group;
    const moe_qffn& q = sh ? shared : routed;
    if (MODE == GM_DOWN_F16W && (int)threadIdx.x < tl.nrows) {
        const int p = tl.row0 + threadIdx.x;
        const int T = args.T;
        coef[threadIdx.x] = p < TOPK * T ? args.wts[min(max(args.perm[p], 0), TOPK * T - 1)]
                                         : args.sg[p - TOPK * T];
    }
    switch ((tl.nrows + 15) >> 4) {
        case 1: gemm_tile<KDIM, MODE, 1>(args, tl, q, e, nb, As, coef); break;
        case 2: gemm_tile<KDIM, MODE, 2>(args, tl, q, e, nb, As, coef); break;
        case 3: gemm_tile<KDIM, MODE, 3>(args, tl, q, e, nb, As, coef); break;
        case 4: gemm_tile<KDIM, MODE, 4>(args, tl, q, e, nb, As, coef); break;
        case 5: gemm_tile<KDIM, MODE, 5>(args, tl, q, e, nb, As, coef); break;
        case 6: gemm_tile<KDIM, MODE, 6>(args, tl, q, e, nb, As, coef); break;
        case 7: gemm_tile<KDIM, MODE, 7>(args, tl, q, e, nb, As, coef); break;
        default: gemm_tile<KDIM, MODE, 8>(args, tl, q, e, nb, As, coef); break;
    }
}

// grid size for a GEMM over at most max_tiles tiles and nb column blocks
static unsigned gemm_grid(int max_tiles, int nb) {
    const int total = max_tiles * nb;
    return (unsigned)(8 * ((total + 7) / 8));
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

static GemmArgs gemm_args(const uint16_t* ain, uint32_t ain_bytes, int T, const int32_t* perm) {
    GemmArgs a;
    a.ain = ain;
    a.ain_bytes = ain_bytes;
    a.T = T;
    a.perm = perm;
    a.hout = nullptr;
    a.dout32 = nullptr;
    a.dout16 = nullptr;
    a.wts = nullptr;
    a.sg = nullptr;
    return a;
}

void launch_expert_prefill(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                           const int* tile_count, int max_tiles, const moe_qffn& routed,
                           const moe_qffn& shared, uint16_t* xh, uint16_t* hbuf, float* dout,
                           hipStream_t st) {
    const size_t chunks = (size_t)T * (H / 8);
    hipLaunchKernelGGL(prep_x_f16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, x, T,
                       xh);
    GemmArgs gu = gemm_args(xh, (uint32_t)((size_t)T * H * 2), T, perm);
    gu.hout = hbuf;
    hipLaunchKernelGGL((expert_gemm<H, GM_GATEUP>), dim3(gemm_grid(max_tiles, I / (GW * 32))),
                       dim3(GW * 64), 0, st, gu, tiles, tile_count, routed, shared);
    GemmArgs dn = gemm_args(hbuf, (uint32_t)((size_t)(TOPK + 1) * T * I * 2), T, perm);
    dn.dout32 = dout;
    hipLaunchKernelGGL((expert_gemm<I, GM_DOWN_F32>), dim3(gemm_grid(max_tiles, H / (GW * 64))),
                       dim3(GW * 64), 0, st, dn, tiles, tile_count, routed, shared);
}

// Whole-layer prefill expert part: gate/up, then down writing fp16 rows of
// (routing weight or shared gate) * d, summed per token by combine_f16.
void launch_expert_prefill_fused(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                                 const int* tile_count, int max_tiles, const moe_qffn& routed,
                                 const moe_qffn& shared, uint16_t* xh, uint16_t* hbuf,
                                 uint16_t* d16, const float* wts, const float* sg,
                                 hipStream_t st) {
    const size_t chunks = (size_t)T * (H / 8);
    hipLaunchKernelGGL(prep_x_f16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, x, T,
                       xh);
    GemmArgs gu = gemm_args(xh, (uint32_t)((size_t)T * H * 2), T, perm);
    gu.hout = hbuf;
    hipLaunchKernelGGL((expert_gemm<H, GM_GATEUP>), dim3(gemm_grid(max_tiles, I / (GW * 32))),
                       dim3(GW * 64), 0, st, gu, tiles, tile_count, routed, shared);
    GemmArgs dn = gemm_args(hbuf, (uint32_t)((size_t)(TOPK + 1) * T * I * 2), T, perm);
    dn.dout16 = d16;
    dn.wts = wts;
    dn.sg = sg;
    hipLaunchKernelGGL((expert_gemm<I, GM_DOWN_F16W>), dim3(gemm_grid(max_tiles, H / (GW * 64))),
                       dim3(GW * 64), 0, st, dn, tiles, tile_count, routed, shared);
}

}  // namespace moe
