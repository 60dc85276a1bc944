// expert.hip -- SwiGLU expert FFNs with 4-bit weights dequantised inside the
// kernels (the weights are never expanded in memory: "Perplexity Open-Sources
// Lily ...", section "The optimizations follow the workload"; "A Rust + Metal
// Inference Engine for Qwen3.6-35B-A3B on Apple Silicon", paragraph 4).
//
// Work is described by the row-tile list built on the device (plan_tiles):
// tile = (expert or shared group, first row, row count <= MT_ROWS).
//
//   decode_down    split interface, few tokens: 16 lanes per output row
//                  (16 B of codes each), 4 rows per wave; exact codes
//                  through v_dot2_f32_f16 (dot8_codes), group scale/bias
//                  applied once per lane; writes fp32 expert rows.  (The
//                  gate/up GEMV it follows and the fused whole-layer decode
//                  kernels live in decode.hip.)
//   grouped_gemm   prefill: persistent grouped GEMM on fp16 MFMA (below).
#include "block_util.hpp"

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
                                                   QFFN routed, QFFN shared,
                                                   float* __restrict__ out) {
    if ((int)blockIdx.x >= *tile_count) return;
    const Tile tl = tiles[blockIdx.x];
    const bool sh = tl.group >= E;
    const int e = sh ? 0 : tl.group;
    const QFFN q = sh ? shared : routed;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int m = blockIdx.y * 16 + (threadIdx.x >> 6) * 4 + (lane >> 4);
    const size_t row = m;
    const uint4v dw = reinterpret_cast<const uint4v*>(expert_at(q.down_q, e, q.sq) + row * (I / 8))[c];
    const float s = fp16_to_f32(expert_at(q.down_s, e, q.ss)[row * (I / G) + (c >> 1)]);
    const float b = fp16_to_f32(expert_at(q.down_b, e, q.ss)[row * (I / G) + (c >> 1)]);
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
// (k = 0,4,1,5,2,6,3,7).  OR-ing an exponent into a masked pair of nibbles
// gives exact fp16 values: nibbles at bits 0..3 of each half under 0x6400
// are 1024 + q, nibbles at bits 4..7 under 0x5400 are 64 + q (mantissa
// 16q, exponent 2^6), so one shift of the word by 8 serves all eight
// codes.  One packed subtraction recovers q exactly and one packed FMA
// applies the group's scale and bias with a single rounding.
__device__ __forceinline__ half8 dequant8(uint32_t w, half2v s2, half2v b2) {
    const uint32_t w8 = w >> 8;
    const uint32_t p[4] = {and_or(w, 0x000F000Fu, 0x64006400u), and_or(w, 0x00F000F0u, 0x54005400u),
                           and_or(w8, 0x000F000Fu, 0x64006400u), and_or(w8, 0x00F000F0u, 0x54005400u)};
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const _Float16 off = (i & 1) ? (_Float16)64.f : (_Float16)1024.f;
        half2v h = __builtin_bit_cast(half2v, p[i]) - (half2v){off, off};
        h = __builtin_elementwise_fma(h, s2, b2);
        r[2 * i] = h[0];
        r[2 * i + 1] = h[1];
    }
    return r;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum GemmMode { GM_GATEUP = 0, GM_DOWN_F32 = 1, GM_DOWN_F16W = 2 };

// Raw buffer resource over [p, p + bytes): loads beyond the range return 0,
// stores beyond it write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// Persistent grouped GEMM (prefill).
//
// Work items are (row tile, block of 256 weight rows) pairs: gate/up has 4
// blocks per tile (128 gate + the same 128 up rows each), down has 8.  A
// grid of 8-wave workgroups, one per compute unit (two for 32-row tiles),
// walks the items with a fixed stride.  Consecutive items (the blocks of
// one tile, which share their activation rows) are dealt to workgroups of
// the same XCD, so the rows are fetched once into that XCD's L2.  Row tiles
// hold up to 160 rows, or 32 rows up to a few hundred tokens (experts then
// have a few dozen rows at most).
//
// K advances in chunks of two quantisation groups (128), or one (64) in the
// 160-row down GEMM.  Everything a chunk needs -- the activation rows (A,
// fp16, gathered by token for gate/up), the 4-bit codes of the 256 weight
// rows (B) and their scales and biases -- moves from global memory straight
// into LDS (buffer loads with an LDS destination) through a ring of STAGES
// stages, STAGES-1 chunks ahead of the MFMAs (2 stages of 128 k; 5 of
// 64 k).  The ring runs on across
// item boundaries: the last chunks of an item prefetch the first ones of
// the next, so no workgroup ever waits for a pipeline fill except at its
// very first item.
//
// Every wave issues exactly LPC loads per chunk (plus one metadata load at
// the first chunk of an item and a fixed number of stores per epilogue;
// missing rows and items become out-of-range buffer offsets, which access no
// memory), so the number of memory operations issued after any chunk's
// loads is a compile-time constant and the wait for a chunk is an exact
// s_waitcnt vmcnt.
//
// Wave w computes 32 weight rows (gate/up: 16 gate + the same 16 up rows;
// down: 32 output columns) for all rows of the tile, each code word being
// dequantised once per item (dequant8: fp16 weights in registers) and fed to v_mfma_f32_32x32x16_f16 with fp32
// accumulation.  SwiGLU is applied in the gate/up epilogue (h =
// bf16(silu(g) u), stored as fp16); down writes fp32 rows (split interface)
// or fp16 rows of (routing weight or shared gate) x d.
//
// Measured limits (4096 tokens, 160-row gate/up): removing the
// dequantisation saves 7-10% of the kernel, removing the activation reads
// from LDS 14%, removing every global load 21-24%, and all three together
// leave 54% -- the MFMAs, barriers, epilogues and the last items' tail.  A
// second wave per SIMD changes none of these shares: VALU work overlaps the
// MFMAs of its own wave, but a VALU wave and an MFMA wave on one SIMD slow
// each other down.
//
// LDS layouts (per stage; a_swz and b_swz below):
//   A   [rows][8 or 16 pieces of 16 B], piece p of row R at slot
//       p ^ a_swz(R): the 16 rows of an MFMA operand read cover all 64 banks.
//   B   [256 columns][2 or 4 pieces of 16 B], piece p of column C at slot
//       p ^ b_swz(C): a 128-bit read by 16 lanes is conflict free.
//   S, Bi [256 columns] dwords holding the fp16 scale (bias) of two
//       consecutive groups.  With one group per chunk they are loaded by the
//       even chunks only: the odd chunk's loads are out-of-range stand-ins
//       (its S and Bi are never read) and its operands use the upper halves,
//       kept in registers by read_b.  With two groups per chunk, each chunk
//       loads its own and lane half g uses half g.
// K order inside a chunk: lane half g of MFMA step s covers k-piece
// STEPS g + s.

struct GemmArgs {
    const uint16_t* ain;      // A rows: x (fp16, slot order) [T][2048] or h [9T][512]
    uint32_t ain_bytes;
    int T;
    const int32_t* perm;      // sorted position -> flat slot 8t+j (gate/up gathers x rows)
    uint16_t* hout;           // gate/up: h fp16 [9T][512]
    float* dout32;            // down, split interface: d fp32 [9T][2048]
    uint16_t* dout16;         // down, fused layer: fp16 coef*d [9T][2048]
    const float* wsorted;     // routing weight of each sorted position [8T]
    const float* sg;          // shared-expert gate per token [T]
};

constexpr uint32_t OOB_OFF = 0x80000000u;   // beyond every buffer: no memory access

// Tile geometry of one instantiation: MTR = rows per row tile, at most (160
// for large T; 32 for small T); KCH = K per pipeline chunk, one quantisation
// group (64) or two (128: each weight row's code request then fetches 64
// bytes instead of 32, half the L1 line requests of the code stream, which
// bound the small-tile gate/up GEMM).
template <int MTR, int KCH>
struct PG {
    // 8 waves, each owning one 32-column n-tile of the item's 256 weight
    // rows (gate/up: 16 gate and the same 16 up rows); two waves per SIMD
    // (one workgroup per CU, or two 8-wave workgroups for 32-row tiles).
    static constexpr int WAVES = 8;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int NT = 1;                        // 32-column n-tiles per wave
    static constexpr int MT = MTR;                      // rows per tile, at most
    static constexpr int NMT_MAX = MT / 32;             // 32-row m-tiles
    static constexpr int KC = KCH;                      // K per chunk
    static_assert(KC == G || KC == 2 * G, "one or two quantisation groups per chunk");
    static constexpr int STEPS = KC / 16;               // MFMA k-steps per chunk
    // ring depth: chunk c+STAGES refills chunk c's stage once every wave is
    // past its last read of it (5 stages with 64 k per chunk; 2 with 128 k,
    // whose 160-row stages take 58 KB and whose 32-row stages then fit two
    // workgroups per CU)
    static constexpr int STAGES = KCH == 2 * G ? 2 : 5;
    static constexpr int AROW = KC * 2;                 // bytes of one A row per chunk
    static constexpr int A_PIECES = AROW / 16;          // 16-byte pieces of an A row (8 or 16)
    static constexpr int A_BYTES = MT * AROW;
    static constexpr int NCOL = 256;                    // weight rows per item
    static constexpr int BCOL = KC / 2;                 // code bytes of one weight row per chunk
    static constexpr int B_PIECES = BCOL / 16;          // (2 or 4)
    static constexpr int B_BYTES = NCOL * BCOL;
    static constexpr int S_BYTES = NCOL * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + 2 * S_BYTES;
    static constexpr int A_RPL = 1024 / AROW;           // A rows per 1 KB load instruction
    static constexpr int A_REAL = MT / A_RPL;           // 1 KB A loads per chunk
    static constexpr int A_LOADS = (A_REAL + WAVES - 1) / WAVES;   // per wave; the excess are
                                                        // stand-ins landing in DUMMY
    static constexpr int B_CPL = 1024 / BCOL;           // weight rows per 1 KB load instruction
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int SB_LOADS = 1;                  // scale/bias dword loads per wave per chunk
                                                        // (waves 0-3 scales, 4-7 biases)
    static constexpr int LPC = A_LOADS + B_LOADS + SB_LOADS;   // loads per wave per chunk
    static constexpr int DUMMY = A_LOADS * WAVES > A_REAL ? 1024 : 0;   // stand-in A landing area
    static constexpr int META = 4 * 256;                // per-item row metadata (tokens or weights):
                                                        // waves 0-2 load rows 0..191, one 4-byte
                                                        // direct load each; the other waves' loads
                                                        // land in the fourth 256 B
    static constexpr int STG = KCH == 2 * G ? 2048 : 512;   // per-wave epilogue staging: a whole
                                                        // m-tile of h or coef*d rows at once,
                                                        // or 512 B rounds where the LDS is full
    static constexpr int CLAIM = 16 + 256;              // the claimed item index (16 B) and the
                                                        // landing area of the other waves'
                                                        // stand-in loads
    static constexpr int RING = STAGES * STAGE;
    static constexpr int META_OFF = RING + DUMMY;       // [2][META], then [WAVES][STG], then CLAIM
    static constexpr int LDS_BYTES = META_OFF + 2 * META + WAVES * STG + CLAIM;
    static constexpr uint32_t OOB = OOB_OFF;
    static constexpr int WG_PER_CU = 160 * 1024 / LDS_BYTES;   // workgroups the LDS holds per CU
    static constexpr int WAVES_PER_SIMD = WG_PER_CU * WAVES / 4;
    static_assert(B_BYTES % (1024 * WAVES) == 0, "code loads must split evenly over the waves");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(META >= MT * 4 && MT <= 192, "row metadata must cover a tile");
    static_assert((STAGES - 2) * LPC + 2 <= 63, "vmcnt range");
};
constexpr int MT_LARGE = MT_ROWS, MT_SMALL = 32;
// The chunk width of an instantiation: two groups (128 k, 2-stage ring)
// everywhere except the split interface's 160-row down GEMM (fp32 rows),
// whose 128-k instance would spill.  Same-run timings: 160-row gate/up
// 212.5 against 227.1 us at 4096 tokens with one group and 5 stages (half
// the barriers and half the code line requests); 32-row down 45.3 against
// 52.6 us in the 512-token chain.
template <int KDIM, int MODE, int MTR>
constexpr int gemm_kc() { return (MTR == MT_LARGE && MODE == GM_DOWN_F32) ? G : 2 * G; }
static_assert(PG<MT_SMALL, 2 * G>::WG_PER_CU == 2 && PG<MT_LARGE, G>::WG_PER_CU == 1 &&
              PG<MT_LARGE, 2 * G>::WG_PER_CU == 1, "tile LDS footprints");

typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

struct GItem {
    int valid;       // 0: past the last item (its loads are dummies)
    int shared;      // group 256 (the shared expert)
    int e;           // routed expert (0 for the shared one)
    int row0, nrows, nb;
};

// Item j of XCD x: column block j % NB of tile x + 8 (j / NB).  nx: the
// XCD's item count.  j is wave-uniform, so the tile is read with scalar
// loads (which the pipeline's vector-memory wait counts do not see).
template <int NB>
__device__ __forceinline__ GItem gemm_item(int j, int nx, int xcd, const Tile* __restrict__ tiles) {
    GItem m;
    m.valid = j < nx;
    const Tile tl = tiles[m.valid ? xcd + 8 * (j / NB) : 0];
    m.shared = tl.group >= E;
    m.e = (m.shared || !m.valid) ? 0 : tl.group;
    m.row0 = tl.row0;
    m.nrows = m.valid ? tl.nrows : 0;
    m.nb = m.valid ? j % NB : 0;
    return m;
}

// Claiming work: wave 0 takes the next index from the XCD's counter; the
// other waves issue a stand-in load that touches no memory, so that every
// wave has issued the same number of vector-memory operations.
__device__ __forceinline__ uint32_t claim_item(int* ctr, uint8_t* claim) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    uint32_t t = 0;
    if (wave == 0) {
        if (lane == 0) t = (uint32_t)atomicAdd(ctr, 1);
    } else {
        // (every such load writes zeros to the same 256 B, which nothing reads)
        const __amdgpu_buffer_rsrc_t r = buf_rsrc(ctr, 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(claim + 16), 4, OOB_OFF, 0, 0, 0);
    }
    return t;
}

// LDS swizzles.  A rows are 128 B (one group per chunk) or 256 B (two): the
// 16 rows of one MFMA operand read (16 lanes x 16 B) must cover all 64
// banks.  At 128 B two consecutive rows fill the 64 banks, so the piece is
// XORed with (R >> 1) & 7; at 256 B every row spans them, so with R & 15.
// B columns are 32 B (two pieces: XOR with (C >> 3) & 1, so 16 lanes reading
// one piece of 16 consecutive columns hit distinct banks) or 64 B (four
// pieces: XOR with (C >> 2) & 3).
template <int KCH>
__device__ __forceinline__ int a_swz(int R) { return KCH == G ? ((R >> 1) & 7) : (R & 15); }
template <int KCH>
__device__ __forceinline__ int b_swz(int C) { return KCH == G ? ((C >> 3) & 1) : ((C >> 2) & 3); }

// A wave-uniform pointer as a scalar value.  The compiler cannot always
// prove an item's matrix pointers uniform (they flow through the item loop's
// merges), and a buffer resource it holds in vector registers costs a
// waterfall loop around every load that uses it.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// Where one item's chunks come from, per lane: the A rows this lane moves
// and the code/scale words of this wave's weight rows.  Chunk kc adds a
// wave-uniform offset (the soffset operand of the loads), so issuing a chunk
// costs no vector arithmetic.  Rows past the tile and items past the last
// get out-of-range offsets (the loads access no memory and fill zeros).
//
// Instruction i of wave w moves A rows (8i + w)*A_RPL + .. (consecutive
// instructions of a wave are 8*A_RPL rows apart, a multiple of the swizzle
// period, so a lane reads the same piece of each row) and B columns
// (w*B_LOADS + i)*B_CPL + .. .  Where the rows are contiguous (down: h
// rows; B: weight rows) only instruction 0's offset is kept per lane and the
// others add a wave-uniform step in the scalar offset: fewer registers.
// Gate/up gathers its A rows by token, so each instruction has its own.
template <int MTR, int KCH>
struct GSrc {
    __amdgpu_buffer_rsrc_t rq, rs, rb;   // this wave's code / scale / bias matrix
    uint32_t a[PG<MTR, KCH>::A_LOADS];   // A offsets (only a[0] without the gather)
    uint32_t b;                          // B offset of instruction 0
    uint32_t s;                          // scale/bias dword of column (w % 4)*64 + lane
};

// The code/scale/bias pointers of one weight matrix of one expert stack.
struct WPtr {
    const uint32_t* q;
    const uint16_t* s;
    const uint16_t* b;
    uint32_t sq, ss;     // bytes between consecutive experts (codes, scales/biases)
};

// The matrices this wave loads from (down: down; gate/up: the codes of item
// columns 0-127 are gate rows and 128-255 the same up rows, loaded by waves
// 0-3 and 4-7; the scale/bias dwords of the 64 columns of wave pair w,
// w+4 come from gate for the first 128) of one stack, as opaque register
// values: a later choice between the routed and the shared stack is then a
// select of values, never of the argument structs' addresses (which would
// force the structs into scratch memory).
template <int MODE>
__device__ __forceinline__ WPtr wave_ptrs(const QFFN& f) {
    WPtr w;
    const int wave = wave_id();
    if (MODE != GM_GATEUP) {
        w.q = f.down_q; w.s = f.down_s; w.b = f.down_b;
    } else {
        const bool up_codes = wave >= 4;
        const bool up_scales = (wave & 3) >= 2;
        w.q = up_codes ? f.up_q : f.gate_q;
        w.s = up_scales ? f.up_s : f.gate_s;
        w.b = up_scales ? f.up_b : f.gate_b;
    }
    asm volatile("" : "+s"(w.q), "+s"(w.s), "+s"(w.b));
    w.sq = f.sq;
    w.ss = f.ss;
    return w;
}

template <int KDIM, int MODE, int MTR, int KCH>
__device__ __forceinline__ GSrc<MTR, KCH> gemm_src(const GItem& m, const int32_t* tok, int T,
                                                   const WPtr& pr, const WPtr& ps) {
    using pg = PG<MTR, KCH>;
    constexpr bool GATEUP = MODE == GM_GATEUP;
    constexpr int WPR = KDIM / 8, SPR = KDIM / G, ROWS_W = GATEUP ? I : H;
    const int lane = threadIdx.x & 63, wave = wave_id();
    GSrc<MTR, KCH> g;
    // A: LDS slot (lane % A_PIECES) of row R holds the row's piece
    // slot ^ a_swz(R)
#pragma unroll
    for (int i = 0; i < (GATEUP ? pg::A_LOADS : 1); ++i) {
        const int R = (i * pg::WAVES + wave) * pg::A_RPL + lane / pg::A_PIECES;
        const int p = (lane % pg::A_PIECES) ^ a_swz<KCH>(R);
        int src = m.row0 + R;
        if (GATEUP) src = m.shared ? m.row0 + R - TOPK * T : min(max(tok[R] >> 3, 0), T - 1);
        // (without the gather the later instructions' rows past the tile read
        // other rows or, past the buffer, zeros: never stored)
        g.a[i] = R < m.nrows ? (uint32_t)src * (uint32_t)(KDIM * 2) + 16u * (uint32_t)p : pg::OOB;
    }
    const uint32_t* code = m.shared ? ps.q : pr.q;
    const uint16_t* sc = m.shared ? ps.s : pr.s;
    const uint16_t* bi = m.shared ? ps.b : pr.b;
    const uint32_t sq = m.shared ? ps.sq : pr.sq, ss = m.shared ? ps.ss : pr.ss;
    g.rq = buf_rsrc(uniform_ptr(expert_at(code, m.e, sq)), ROWS_W * WPR * 4);
    g.rs = buf_rsrc(uniform_ptr(expert_at(sc, m.e, ss)), ROWS_W * SPR * 2);
    g.rb = buf_rsrc(uniform_ptr(expert_at(bi, m.e, ss)), ROWS_W * SPR * 2);
    auto wrow = [&](int C) { return GATEUP ? m.nb * 128 + (C & 127) : m.nb * 256 + C; };
    // B: LDS slot (lane % B_PIECES) of column C holds the column's piece
    // slot ^ b_swz(C)
    {
        // (a wave's B_LOADS * B_CPL columns stay inside one half, gate or up,
        // and B_CPL is a multiple of the swizzle period)
        const int C = wave * pg::B_LOADS * pg::B_CPL + lane / pg::B_PIECES;
        const int p = (lane % pg::B_PIECES) ^ b_swz<KCH>(C);
        g.b = m.valid ? (uint32_t)(wrow(C) * WPR * 4 + 16 * p) : pg::OOB;
    }
    g.s = m.valid ? (uint32_t)(wrow((wave & 3) * 64 + lane) * SPR * 2) : pg::OOB;
    return g;
}

template <int SIZE>
__device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff,
                                         uint32_t soff) {
    static_assert(SIZE == 4 || SIZE == 16, "direct-to-LDS load size");
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 4, voff, soff, 0, 0);
}

// The LPC loads of chunk kc of an item into one stage (KDIM: the row
// length of the A and code matrices; GATHER: per-instruction A offsets).
template <int KDIM, bool GATHER, int MTR, int KCH>
__device__ __forceinline__ void issue_chunk(const GSrc<MTR, KCH>& g, int kc,
                                            __amdgpu_buffer_rsrc_t ra, uint8_t* stage,
                                            uint8_t* lds) {
    using pg = PG<MTR, KCH>;
    constexpr uint32_t A_STEP = GATHER ? 0 : pg::WAVES * pg::A_RPL * KDIM * 2;
    constexpr uint32_t B_STEP = pg::B_CPL * (KDIM / 2);
    const int wave = wave_id();
#pragma unroll
    for (int i = 0; i < pg::A_LOADS; ++i) {
        // (stand-ins past the tile's last 1 KB land in the dummy area after the ring)
        const int idx = i * pg::WAVES + wave;
        uint8_t* dst = stage + idx * 1024;
        if (pg::DUMMY && idx >= pg::A_REAL) dst = lds + pg::RING;
        load_lds<16>(ra, dst, GATHER ? g.a[i] : g.a[0], kc * pg::AROW + i * A_STEP);
    }
#pragma unroll
    for (int i = 0; i < pg::B_LOADS; ++i)
        load_lds<16>(g.rq, stage + pg::A_BYTES + (wave * pg::B_LOADS + i) * 1024, g.b,
                     kc * pg::BCOL + i * B_STEP);
    // one scale and one bias dword covers two groups.  One group per chunk:
    // the dword of chunks kc & ~1 and kc | 1, loaded by the even chunk; the
    // odd chunk's loads are out-of-range stand-ins (no memory access), and
    // its operands reuse the even chunk's dwords (read_b).  Two groups per
    // chunk: every chunk loads its own dword.
    const uint32_t so = (KCH == G && (kc & 1)) ? pg::OOB : g.s;
    const uint32_t sb = KCH == G ? (uint32_t)((kc & ~1) * 2) : (uint32_t)(kc * 4);
    // waves 0-3 the scales, 4-7 the biases of columns (w % 4)*64 ..
    uint8_t* sbase = stage + pg::A_BYTES + pg::B_BYTES;
    const bool bias = wave >= 4;
    load_lds<4>(bias ? g.rb : g.rs, sbase + (bias ? pg::S_BYTES : 0) + (wave & 3) * 256, so, sb);
}

// MFMA: v_mfma_f32_32x32x16_f16 (32 rows x 32 columns x 16 k).  Lane l
// holds A row l%32 and B column l%32 for k = 8*(l/32)..+7, and accumulator
// element i of row 8*(i/4) + 4*(l/32) + i%4, column l%32.  (The 16x16x32
// shape issues at well under half the matrix-core rate on this chip.)
typedef float float16v __attribute__((ext_vector_type(16)));

// LDS column (0..255 of the item) of wave w's n-tile, lane column l%32:
// gate/up lanes l%32 < 16 take gate rows w*16 + l%32, lanes l%32 >= 16 the
// same up rows (so each gate value and its up value sit in lanes l and
// l ^ 16 of one wave); down: 32 consecutive rows per wave.
template <bool GATEUP>
__device__ __forceinline__ int gemm_col(int wave, int l32) {
    return GATEUP ? (l32 >> 4) * 128 + wave * 16 + (l32 & 15) : wave * 32 + l32;
}

// K order inside a chunk of STEPS k-steps: MFMA step s, lane half g = l/32
// covers the 8-wide k-piece STEPS g + s.  A lane therefore needs one
// contiguous run of STEPS code words (the half g of each of its columns'
// code bytes of the chunk), and with two groups per chunk lane half g works
// in group 2 kc + g throughout.
template <int NT>
struct BFrag {
    uint4v w[NT][2];      // per n-tile: words of steps 0..3 (and 4..7)
    half2v s[NT], b[NT];  // fp16 scale / bias, splat
};

// Even chunks read the scale and bias dwords from the stage and keep their
// upper halves (the next chunk's group) in `carry`; odd chunks, whose stage
// holds no scales, take them from there.  Every call site's chunk parity is
// a compile-time constant after unrolling, so the branch folds away.
template <int NT>
struct SCarry {
    half2v s[NT], b[NT];
};

template <bool GATEUP, int MTR, int KCH>
__device__ __forceinline__ BFrag<PG<MTR, KCH>::NT> read_b(const uint8_t* stage, int kc,
                                                          SCarry<PG<MTR, KCH>::NT>& carry) {
    using pg = PG<MTR, KCH>;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int l32 = lane & 31, g = lane >> 5;
    BFrag<pg::NT> B;
#pragma unroll
    for (int nt = 0; nt < pg::NT; ++nt) {
        const int C = gemm_col<GATEUP>(wave, l32);
        const uint8_t* col = stage + pg::A_BYTES + C * pg::BCOL;
        if constexpr (KCH != G) {
            // two groups: pieces 2g and 2g+1, and half g of the stage's dwords
            B.w[nt][0] = *reinterpret_cast<const uint4v*>(col + 16 * ((2 * g) ^ b_swz<KCH>(C)));
            B.w[nt][1] = *reinterpret_cast<const uint4v*>(col + 16 * ((2 * g + 1) ^ b_swz<KCH>(C)));
            const uint32_t sd = *reinterpret_cast<const uint32_t*>(stage + pg::A_BYTES + pg::B_BYTES + C * 4);
            const uint32_t bd =
                *reinterpret_cast<const uint32_t*>(stage + pg::A_BYTES + pg::B_BYTES + pg::S_BYTES + C * 4);
            B.s[nt] = splat_h((uint16_t)(g ? sd >> 16 : sd));
            B.b[nt] = splat_h((uint16_t)(g ? bd >> 16 : bd));
            continue;
        }
        B.w[nt][0] = *reinterpret_cast<const uint4v*>(col + 16 * (g ^ b_swz<KCH>(C)));
        if (kc & 1) {
            B.s[nt] = carry.s[nt];
            B.b[nt] = carry.b[nt];
        } else {
            const uint32_t sd = *reinterpret_cast<const uint32_t*>(stage + pg::A_BYTES + pg::B_BYTES + C * 4);
            const uint32_t bd =
                *reinterpret_cast<const uint32_t*>(stage + pg::A_BYTES + pg::B_BYTES + pg::S_BYTES + C * 4);
            B.s[nt] = splat_h((uint16_t)sd);
            B.b[nt] = splat_h((uint16_t)bd);
            carry.s[nt] = splat_h((uint16_t)(sd >> 16));
            carry.b[nt] = splat_h((uint16_t)(bd >> 16));
        }
    }
    return B;
}

// A operand of K-step s: row mt*32 + l%32, k-piece STEPS g + s.
template <int NMT, int MTR, int KCH>
__device__ __forceinline__ void read_a(const uint8_t* stage, int s, half8 (&a)[NMT]) {
    using pg = PG<MTR, KCH>;
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int R = mt * 32 + l32;
        a[mt] = *reinterpret_cast<const half8*>(stage + R * pg::AROW +
                                                16 * ((pg::STEPS * g + s) ^ a_swz<KCH>(R)));
    }
}

template <int NT>
__device__ __forceinline__ void dequant_step(const BFrag<NT>& B, int s, half8 (&bf)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const uint32_t wv = B.w[nt][s >> 2][s & 3];
        bf[nt] = dequant8(wv, B.s[nt], B.b[nt]);
    }
}

template <int NMT, int NT>
__device__ __forceinline__ void mfma_step(const half8 (&a)[NMT], const half8 (&bf)[NT],
                                          float16v (&acc)[NMT][NT]) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mt], bf[nt], acc[mt][nt], 0, 0, 0);
}

// Scheduling hint for one MFMA step: its operand reads first, then MFMAs
// alternating with the VALU work of the next step's dequantisation.
template <int NMT, int NT, int DS_READS>
__device__ __forceinline__ void sched_step() {
    constexpr int NM = NT * NMT;
    constexpr int V = (16 * NT + NM - 1) / NM;    // ~15 VALU per n-tile's dequantisation
    __builtin_amdgcn_sched_group_barrier(0x100, DS_READS, 0);      // DS read
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);          // VALU
    }
}

// Stores per wave per epilogue: per 32-row m-tile, gate/up one (2 KB
// staging) or two, fp16 down two or four, fp32 down eight.
template <int MODE, int MTR, int KCH>
constexpr int epi_stores() {
    constexpr int n = PG<MTR, G>::NMT_MAX;
    constexpr bool wide = PG<MTR, KCH>::STG >= 2048;
    return MODE == GM_GATEUP ? (wide ? 1 : 2) * n : MODE == GM_DOWN_F16W ? (wide ? 2 : 4) * n : 8 * n;
}

// Staging through LDS moves values between lanes of one wave.  The wave's
// LDS operations execute in program order, but the compiler reasons per
// lane: a lane's read of its own 16 bytes does not alias its own writes, so
// without this fence it could hoist the read above the other lanes' writes
// (or the next round's writes above the read).
__device__ __forceinline__ void lane_exchange_fence() {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// Output buffer resources are based at the item's first row and cover only
// its rows, so every store offset is below MT_ROWS rows whatever T is (the
// whole fp32 output of the largest call, 9 * 65536 rows of 8 KB, is beyond
// the 32-bit range of a buffer resource).
static_assert((uint64_t)MT_ROWS * H * 4 < (1ull << 31), "per-item output range");
static_assert((uint64_t)(TOPK + 1) * MOE_T_MAX * I * 2 < (1ull << 32),
              "A rows of the down GEMM (h) are addressed with 32-bit buffer offsets");
static_assert((uint64_t)MOE_T_MAX * H * 2 < (1ull << 32),
              "A rows of the gate/up GEMM (x) are addressed with 32-bit buffer offsets");

template <typename P>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t item_rows(P* base, const GItem& m, int row_elems) {
    return buf_rsrc(base + (size_t)m.row0 * row_elems,
                    (uint32_t)m.nrows * (uint32_t)row_elems * (uint32_t)sizeof(P));
}

// One n-tile per wave.  Accumulator element i of lane l holds row
// 8*(i/4) + 4*(l/32) + i%4 of the m-tile.
//   gate/up: lanes l%32 < 16 (gate) and l ^ 16 (up) exchange half of their
//     elements, so that the first lane forms h for elements 0..7 (rows
//     0..15) and the second for elements 8..15 (rows 16..31).  With 2 KB of
//     staging the m-tile is staged at once as [32 rows][16 columns] and
//     stored 16 bytes per lane; with 512 B, one half at a time, 8 bytes.
//   down, fp16 rows of coef x d: with 2 KB the m-tile at once as [32][32],
//     two 16-byte stores per lane; with 512 B elements 4b..4b+3 (rows
//     8b..8b+7) per b as [8][32].  fp32 rows: [8][16] per b and half of the
//     columns.
template <int MODE, int NMT, int MTR, int KCH>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& A, const GItem& m,
                                                 float16v (&acc)[NMT][1], uint8_t* stg,
                                                 const float* coef) {
    using pg = PG<MTR, G>;
    constexpr bool WIDE = PG<MTR, KCH>::STG >= 2048;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int l32 = lane & 31, g = lane >> 5;
    if constexpr (MODE == GM_GATEUP) {
        const __amdgpu_buffer_rsrc_t rh = item_rows(A.hout, m, I);
        uint16_t* st = reinterpret_cast<uint16_t*>(stg);    // [16][16] fp16, slot order
        const bool lo = l32 < 16;
        const int j = l32 & 15;                              // h column of the wave's 16
#pragma unroll
        for (int mt = 0; mt < pg::NMT_MAX; ++mt) {
            uint16_t hv[8];
            if (mt < NMT) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float a0 = acc[mt < NMT ? mt : 0][0][q], a1 = acc[mt < NMT ? mt : 0][0][8 + q];
                    const float mine = lo ? a0 : a1;            // gate (elem q) / up (elem 8+q)
                    // lane l ^ 16's value: v_permlane16_swap exchanges the
                    // odd 16-lane rows of its first operand with the even
                    // rows of its second, so each half takes its partner's
                    // value from one of the two results
                    const uint32_t snd = __builtin_bit_cast(uint32_t, lo ? a1 : a0);
                    const auto sw = __builtin_amdgcn_permlane16_swap(snd, snd, false, false);
                    const float other = __builtin_bit_cast(float, lo ? sw[1] : sw[0]);
                    const float gv = lo ? mine : other, uv = lo ? other : mine;
                    const float h = __fdividef(gv, 1.f + __expf(-gv)) * uv;
                    hv[q] = __builtin_bit_cast(uint16_t, (_Float16)bf16_to_f32(f32_to_bf16(h)));
                }
            }
            if constexpr (WIDE) {
                uint4v v = (uint4v){0u, 0u, 0u, 0u};
                uint32_t off = pg::OOB;
                if (mt < NMT) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int row = (lo ? 0 : 16) + 8 * (q >> 2) + 4 * g + (q & 3);
                        st[row * 16 + (j & ~7) + chunk_slot(j & 7)] = hv[q];
                    }
                    lane_exchange_fence();
                    v = reinterpret_cast<const uint4v*>(stg)[lane];
                    lane_exchange_fence();
                    const int R = mt * 32 + (lane >> 1);
                    if (R < m.nrows)
                        off = (uint32_t)((R * I + m.nb * 128 + wave * 16 + (lane & 1) * 8) * 2);
                }
                __builtin_amdgcn_raw_buffer_store_b128(v, rh, off, 0, 0);
                continue;
            }
#pragma unroll
            for (int hr = 0; hr < 2; ++hr) {
                uint2v v = (uint2v){0u, 0u};
                uint32_t off = pg::OOB;
                if (mt < NMT) {
                    if ((lo ? 0 : 1) == hr) {
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int row = 8 * (q >> 2) + 4 * g + (q & 3);
                            st[row * 16 + (j & ~7) + chunk_slot(j & 7)] = hv[q];
                        }
                    }
                    lane_exchange_fence();
                    v = reinterpret_cast<const uint2v*>(stg)[lane];
                    lane_exchange_fence();
                    const int R = mt * 32 + hr * 16 + (lane >> 2);
                    if (R < m.nrows)
                        off = (uint32_t)((R * I + m.nb * 128 + wave * 16 + (lane & 3) * 4) * 2);
                }
                __builtin_amdgcn_raw_buffer_store_b64(v, rh, off, 0, 0);
            }
        }
    } else if constexpr (MODE == GM_DOWN_F16W) {
        const __amdgpu_buffer_rsrc_t rd = item_rows(A.dout16, m, H);
        uint16_t* st = reinterpret_cast<uint16_t*>(stg);    // [32][32] or [8][32] fp16
        if constexpr (WIDE) {
#pragma unroll
            for (int mt = 0; mt < pg::NMT_MAX; ++mt) {
                uint4v v[2] = {(uint4v){0u, 0u, 0u, 0u}, (uint4v){0u, 0u, 0u, 0u}};
                uint32_t off[2] = {pg::OOB, pg::OOB};
                if (mt < NMT) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float4v cf = *reinterpret_cast<const float4v*>(coef + mt * 32 + 8 * b + 4 * g);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float d = acc[mt < NMT ? mt : 0][0][4 * b + r] * cf[r];
                            st[(8 * b + 4 * g + r) * 32 + l32] = __builtin_bit_cast(uint16_t, (_Float16)d);
                        }
                    }
                    lane_exchange_fence();
                    v[0] = reinterpret_cast<const uint4v*>(stg)[lane];
                    v[1] = reinterpret_cast<const uint4v*>(stg)[lane + 64];
                    lane_exchange_fence();
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int R = mt * 32 + 16 * h + (lane >> 2);
                        if (R < m.nrows)
                            off[h] = (uint32_t)((R * H + m.nb * 256 + wave * 32 + (lane & 3) * 8) * 2);
                    }
                }
                __builtin_amdgcn_raw_buffer_store_b128(v[0], rd, off[0], 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(v[1], rd, off[1], 0, 0);
            }
            return;
        }
#pragma unroll
        for (int mt = 0; mt < pg::NMT_MAX; ++mt)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint2v v = (uint2v){0u, 0u};
                uint32_t off = pg::OOB;
                if (mt < NMT) {
                    const float4v cf = *reinterpret_cast<const float4v*>(coef + mt * 32 + 8 * b + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float d = acc[mt < NMT ? mt : 0][0][4 * b + r] * cf[r];
                        st[(4 * g + r) * 32 + l32] = __builtin_bit_cast(uint16_t, (_Float16)d);
                    }
                    lane_exchange_fence();
                    v = reinterpret_cast<const uint2v*>(stg)[lane];
                    lane_exchange_fence();
                    const int R = mt * 32 + 8 * b + (lane >> 3);
                    if (R < m.nrows)
                        off = (uint32_t)((R * H + m.nb * 256 + wave * 32 + (lane & 7) * 4) * 2);
                }
                __builtin_amdgcn_raw_buffer_store_b64(v, rd, off, 0, 0);
            }
    } else {
        const __amdgpu_buffer_rsrc_t rd = item_rows(A.dout32, m, H);
        float* st = reinterpret_cast<float*>(stg);          // [8][16] fp32
#pragma unroll
        for (int mt = 0; mt < pg::NMT_MAX; ++mt)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    uint2v v = (uint2v){0u, 0u};
                    uint32_t off = pg::OOB;
                    if (mt < NMT) {
                        if ((l32 >> 4) == ch) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                st[(4 * g + r) * 16 + (l32 & 15)] = acc[mt < NMT ? mt : 0][0][4 * b + r];
                        }
                        lane_exchange_fence();
                        v = reinterpret_cast<const uint2v*>(stg)[lane];
                        lane_exchange_fence();
                        const int R = mt * 32 + 8 * b + (lane >> 3);
                        if (R < m.nrows)
                            off = (uint32_t)((R * H + m.nb * 256 + wave * 32 + ch * 16 + (lane & 7) * 2) * 4);
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(v, rd, off, 0, 0);
                }
    }
}

// Per-item row metadata, one load per wave at the first chunk of an item:
// gate/up loads the NEXT item's permutation entries (token of each row),
// down/fp16 loads the CURRENT item's row weights.  Waves 0-2 cover rows
// 0..191; the other waves' loads are dummies that keep the count uniform
// (they all land in the fourth 256 B).
template <int MODE>
__device__ __forceinline__ void issue_meta(const GemmArgs& A, const GItem& m, uint8_t* meta) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int R = wave * 64 + lane;
    const int T = A.T;
    const bool use = m.valid && wave < 3 && R < m.nrows;
    if constexpr (MODE == GM_GATEUP) {
        const __amdgpu_buffer_rsrc_t rp = buf_rsrc(A.perm, (uint32_t)(TOPK * T * 4));
        const uint32_t off = use && !m.shared ? (uint32_t)((m.row0 + R) * 4) : OOB_OFF;
        load_lds<4>(rp, meta + min(wave, 3) * 256, off, 0);
    } else if constexpr (MODE == GM_DOWN_F16W) {
        const __amdgpu_buffer_rsrc_t rw =
            m.shared ? buf_rsrc(A.sg, (uint32_t)(T * 4)) : buf_rsrc(A.wsorted, (uint32_t)(TOPK * T * 4));
        const int idx = m.shared ? m.row0 + R - TOPK * T : m.row0 + R;
        const uint32_t off = use ? (uint32_t)(idx * 4) : OOB_OFF;
        load_lds<4>(rw, meta + min(wave, 3) * 256, off, 0);
    } else {
        const __amdgpu_buffer_rsrc_t rp = buf_rsrc(A.perm, 4);
        load_lds<4>(rp, meta + min(wave, 3) * 256, OOB_OFF, 0);
    }
}

// Dynamic schedule of one workgroup: its XCD's counter and item count, the
// first claimable index (the first two items per workgroup are static).
struct Sched {
    int* ctr;
    int nx, xcd, jbase;
    const Tile* tiles;
};

// One item: NCH chunks of MFMAs, then the epilogue.  Each chunk is
// software-pipelined around the workgroup barrier: K-steps 0..2 run before
// it (each step's MFMAs hide the next step's operand reads and
// dequantisation); after it, while step 3's MFMAs run, this chunk's stage is
// refilled with chunk c+5 (the ring runs on into the next item) and the next
// chunk's operands are read and its step 0 dequantised.  Only the first
// chunk of an item dequantises with no MFMAs to hide under.
template <int KDIM, int MODE, int NMT, int MTR, int KCH>
__device__ __forceinline__ void gemm_run_item(const GemmArgs& A, const GItem& cur, GItem& nxt,
                                              const GSrc<MTR, KCH>& src_cur, GSrc<MTR, KCH>& src_nxt, int& gc, int k,
                                              bool first, __amdgpu_buffer_rsrc_t ra,
                                              const WPtr& pr, const WPtr& ps, uint8_t* lds,
                                              const Sched& sc, uint32_t& tick) {
    using pg = PG<MTR, KCH>;
    constexpr bool GATEUP = MODE == GM_GATEUP;
    constexpr int NB = GATEUP ? 2 * I / pg::NCOL : H / pg::NCOL;
    constexpr int NCH = KDIM / pg::KC;
    constexpr int S_EPI = epi_stores<MODE, MTR, KCH>();
    constexpr int S = pg::STAGES;
    constexpr int BASE = (S - 2) * pg::LPC;     // loads of the chunks behind the awaited one
    // (a count larger than the operations really issued after the awaited
    // chunk would not wait for it; a smaller one only waits longer)
    constexpr int W_S = BASE + S_EPI < 63 ? BASE + S_EPI : 63;
    constexpr int W_XS = BASE + 2 + S_EPI < 63 ? BASE + 2 + S_EPI : 63;
    uint8_t* meta = lds + pg::META_OFF;
    uint8_t* stg = meta + 2 * pg::META + wave_id() * pg::STG;
    uint8_t* claim = meta + 2 * pg::META + pg::WAVES * pg::STG;
    constexpr int NT = pg::NT;
    float16v acc[NMT][NT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (float16v)0.f;

    half8 a_cur[NMT], bf_cur[NT];
    SCarry<NT> carry;
    BFrag<NT> B = read_b<GATEUP, MTR, KCH>(lds + (gc % pg::STAGES) * pg::STAGE, 0, carry);
    read_a<NMT, MTR, KCH>(lds + (gc % pg::STAGES) * pg::STAGE, 0, a_cur);
    dequant_step(B, 0, bf_cur);

    // One chunk.  `refill(stage)` issues the loads of chunk c+S into the
    // stage chunk c has just released.
    auto chunk = [&](int c, auto&& refill) {
        const uint8_t* st = lds + (gc % pg::STAGES) * pg::STAGE;
#pragma unroll
        for (int s = 0; s < pg::STEPS - 1; ++s) {
            half8 a_nx[NMT], bf_nx[NT];
            read_a<NMT, MTR, KCH>(st, s + 1, a_nx);
            dequant_step(B, s + 1, bf_nx);
            mfma_step<NMT, NT>(a_cur, bf_cur, acc);
            sched_step<NMT, NT, NMT>();
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) a_cur[mt] = a_nx[mt];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bf_cur[nt] = bf_nx[nt];
        }

        // chunk c+1 must have landed (issued S-1 refills ago).  Issued after
        // it and allowed to stay in flight: the loads of the next S-2 chunks
        // (BASE), this item's metadata load and work claim (issued after the
        // wait of c = 0, counted for c = 1..S-1) and, for c <= S-2, the
        // previous item's epilogue stores.
        if (!first && c == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(W_S));
        else if (!first && c <= S - 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(W_XS));
        else if (c >= 1 && c <= S - 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(BASE + 2));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(BASE));
        pipe_barrier();

        // the last step of this chunk under the next chunk's reads, the
        // refill and the next chunk's first dequantisation
        // (the sched_barrier fences keep the refill loads in issue order
        // relative to the other vector-memory operations: the wait counts
        // above depend on that order)
        const bool more = c + 1 < NCH;
        half8 a_nx[NMT], bf_nx[NT];
        if (more) {
            const uint8_t* sn = lds + ((gc + 1) % pg::STAGES) * pg::STAGE;
            B = read_b<GATEUP, MTR, KCH>(sn, c + 1, carry);
            read_a<NMT, MTR, KCH>(sn, 0, a_nx);
        }
        __builtin_amdgcn_sched_barrier(0);
        refill(const_cast<uint8_t*>(st));
        __builtin_amdgcn_sched_barrier(0);
        if (more) dequant_step(B, 0, bf_nx);
        mfma_step<NMT, NT>(a_cur, bf_cur, acc);
#pragma unroll
        for (int i = 0; i < NT * NMT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, (20 * NT + NT * NMT - 1) / (NT * NMT), 0);
        }
        if (more) {
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) a_cur[mt] = a_nx[mt];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bf_cur[nt] = bf_nx[nt];
        }
        ++gc;
    };
    auto own = [&](int c) {
        return [&, c](uint8_t* st) { issue_chunk<KDIM, GATEUP>(src_cur, c + pg::STAGES, ra, st, lds); };
    };
    auto next = [&](int c) {
        return [&, c](uint8_t* st) { issue_chunk<KDIM, GATEUP>(src_nxt, c + pg::STAGES - NCH, ra, st, lds); };
    };
    // the next item's sources (its row tokens arrived with this item's first chunk)
    auto make_next = [&]() {
        src_nxt = gemm_src<KDIM, MODE, MTR, KCH>(nxt, reinterpret_cast<const int32_t*>(meta + ((k + 1) & 1) * pg::META),
                                       A.T, pr, ps);
    };

    constexpr int MAIN = NCH - S;               // chunks whose refill stays in this item
    constexpr int HEAD = S;                     // chunks with special wait counts
    static_assert(MAIN >= 1, "an item needs more chunks than pipeline stages");
    // head: unrolled, so every wait count and refill target is a constant
    chunk(0, [&](uint8_t* st) {
        issue_chunk<KDIM, GATEUP>(src_cur, pg::STAGES, ra, st, lds);
        __builtin_amdgcn_sched_barrier(0);      // the metadata load goes after the chunk's loads
        // the item after this one, claimed during the previous item (its
        // index was written to LDS before this chunk's barrier)
        if (!first)
            nxt = gemm_item<NB>(sc.jbase + __builtin_amdgcn_readfirstlane(*(const int*)claim),
                                sc.nx, sc.xcd, sc.tiles);
        issue_meta<MODE>(A, GATEUP ? nxt : cur, meta + ((GATEUP ? k + 1 : k) & 1) * pg::META);
        tick = claim_item(sc.ctr, claim);       // the one after that
        __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int c = 1; c < HEAD; ++c) {
        if (c < MAIN) chunk(c, own(c));
        else {
            if (c == MAIN) make_next();
            chunk(c, next(c));
        }
    }
    // main: one basic block per two chunks (an even number of them, so each
    // call's chunk parity is a constant)
    static_assert(MAIN <= HEAD || (MAIN - HEAD) % 2 == 0, "main chunk pairs");
    for (int i = 0; i < (MAIN - HEAD) / 2; ++i) {
        const int c = HEAD + 2 * i;
        chunk(c, own(c));
        chunk(c + 1, own(c + 1));
    }
    if (MAIN >= HEAD) make_next();
    // tail: refills from the next item
#pragma unroll
    for (int c = (MAIN > HEAD ? MAIN : HEAD); c < NCH; ++c) chunk(c, next(c));
    __builtin_amdgcn_sched_barrier(0);          // epilogue stores after the last refill
    gemm_epilogue<MODE, NMT, MTR, KCH>(A, cur, acc, stg, reinterpret_cast<const float*>(meta + (k & 1) * pg::META));
    __builtin_amdgcn_sched_barrier(0);
}

// Work split: workgroups are dealt to the 8 XCDs in turn, so XCD x =
// blockIdx.x mod 8 takes tiles x, x+8, ... (the planner sorts tiles by
// cost, so every XCD gets a similar share); a tile's column blocks then run
// on one XCD and share its L2 for the tile's rows.  Within an XCD the first
// two items of each workgroup are static and the rest are claimed from the
// XCD's counter in order -- longest first.
template <int KDIM, int MODE, int MTR>
__global__ __launch_bounds__((PG<MTR, gemm_kc<KDIM, MODE, MTR>()>::THREADS))
__attribute__((amdgpu_waves_per_eu(PG<MTR, gemm_kc<KDIM, MODE, MTR>()>::WAVES_PER_SIMD)))
void grouped_gemm(GemmArgs args, const Tile* __restrict__ tiles, int* __restrict__ tile_count,
                  QFFN routed, QFFN shared) {
    constexpr int KCH = gemm_kc<KDIM, MODE, MTR>();
    using pg = PG<MTR, KCH>;
    constexpr bool GATEUP = MODE == GM_GATEUP;
    constexpr int NB = GATEUP ? 2 * I / pg::NCOL : H / pg::NCOL;
    __shared__ __attribute__((aligned(16))) uint8_t lds[pg::LDS_BYTES];
    const int xcd = blockIdx.x & 7, wl = blockIdx.x >> 3, nwl = gridDim.x >> 3;
    const int ntiles = tile_count[0];
    const int nx = max(ntiles - xcd + 7, 0) / 8 * NB;
    if (wl >= nx) return;
    const Sched sc{tile_count + (GATEUP ? GEMM_CTR_GATEUP : GEMM_CTR_DOWN) + xcd, nx, xcd, 2 * nwl,
                   tiles};
    uint8_t* meta = lds + pg::META_OFF;
    const __amdgpu_buffer_rsrc_t ra = buf_rsrc(args.ain, args.ain_bytes);

    GItem cur = gemm_item<NB>(wl, nx, xcd, tiles);
    GItem nxt = gemm_item<NB>(wl + nwl, nx, xcd, tiles);
    if (GATEUP) {
        // the first item's permutation entries, before any of its rows can move
        issue_meta<MODE>(args, cur, meta);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
    }
    const WPtr pr = wave_ptrs<MODE>(routed), ps = wave_ptrs<MODE>(shared);
    GSrc<MTR, KCH> src_cur =
        gemm_src<KDIM, MODE, MTR, KCH>(cur, reinterpret_cast<const int32_t*>(meta), args.T, pr, ps);
    GSrc<MTR, KCH> src_nxt = src_cur;
    for (int c = 0; c < pg::STAGES; ++c) issue_chunk<KDIM, GATEUP>(src_cur, c, ra, lds + c * pg::STAGE, lds);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((pg::STAGES - 1) * pg::LPC));   // chunk 0 landed
    pipe_barrier();

    int gc = 0;
    uint32_t tick = 0;
    for (int k = 0;; ++k) {
        switch ((cur.nrows + 31) >> 5) {
    // (a tile never has more than NMT_MAX m-tiles; cases from NMT_MAX up run
    // that instance, so every case processes its item)
#define PG_CASE(n)                                                                           \
    case n:                                                                                  \
        gemm_run_item<KDIM, MODE, (n < pg::NMT_MAX ? n : pg::NMT_MAX), MTR, KCH>(            \
            args, cur, nxt, src_cur, src_nxt, gc, k, k == 0, ra, pr, ps, lds, sc, tick);     \
        break;
            PG_CASE(1) PG_CASE(2) PG_CASE(3) PG_CASE(4)
            default: gemm_run_item<KDIM, MODE, pg::NMT_MAX, MTR, KCH>(args, cur, nxt, src_cur, src_nxt,
                                                                      gc, k, k == 0, ra, pr, ps, lds,
                                                                      sc, tick);
                     break;
#undef PG_CASE
        }
        // no workgroup processes more items than its XCD has: the bound ends
        // the loop even if the claimed indices were corrupted
        if (!nxt.valid || k + 1 >= nx) break;
        cur = nxt;
        src_cur = src_nxt;
        // the claimed index, for the next item's first chunk (after its barrier)
        if (threadIdx.x == 0) *reinterpret_cast<int*>(meta + 2 * pg::META + pg::WAVES * pg::STG) = (int)tick;
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
                          const int* tile_count, int max_tiles, const QFFN& routed,
                          const QFFN& shared, uint16_t* hbuf, hipStream_t st);

void launch_expert_decode(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                          const int* tile_count, int max_tiles, const QFFN& routed,
                          const QFFN& shared, uint16_t* xh, uint16_t* hbuf, float* dout,
                          hipStream_t st) {
    const size_t chunks = (size_t)T * (H / 8);
    hipLaunchKernelGGL(prep_x_f16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, x, T,
                       xh);
    launch_decode_gateup(xh, T, perm, tiles, tile_count, max_tiles, routed, shared, hbuf, st);
    hipLaunchKernelGGL(decode_down, dim3(max_tiles, H / 16), dim3(256), 0, st, hbuf, T, tiles,
                       tile_count, routed, shared, dout);
}

static GemmArgs gemm_args(const uint16_t* ain, size_t ain_bytes, int T, const int32_t* perm) {
    GemmArgs a;
    a.ain = ain;
    a.ain_bytes = (uint32_t)ain_bytes;
    a.T = T;
    a.perm = perm;
    a.hout = nullptr;
    a.dout32 = nullptr;
    a.dout16 = nullptr;
    a.wsorted = nullptr;
    a.sg = nullptr;
    return a;
}

// Row-tile height of the grouped GEMMs at T tokens: 32-row tiles (two
// workgroups per CU) while the experts average at most 16 rows, 160 above.
// The small tiles stream the weights better up to several hundred tokens
// (T = 768: 209-217 against 247 us per layer on 160-row tiles; T = 1024:
// 274-279 against 263-265), so the switch sits in between.
#ifndef MOE_SMALL_TILE_T
#define MOE_SMALL_TILE_T 896
#endif
int gemm_tile_rows(int T) { return T <= MOE_SMALL_TILE_T ? MT_SMALL : MT_LARGE; }

// One persistent grouped GEMM: as many workgroups as the LDS lets each CU
// hold (a multiple of the 8 XCDs).
template <int KDIM, int MODE>
static void launch_gemm(const GemmArgs& a, const Tile* tiles, int* tile_count, const QFFN& routed,
                        const QFFN& shared, int mt_rows, hipStream_t st) {
    if (mt_rows == MT_SMALL)
        hipLaunchKernelGGL((grouped_gemm<KDIM, MODE, MT_SMALL>),
                           dim3(256 * PG<MT_SMALL, gemm_kc<KDIM, MODE, MT_SMALL>()>::WG_PER_CU),
                           dim3(PG<MT_SMALL, gemm_kc<KDIM, MODE, MT_SMALL>()>::THREADS), 0, st, a, tiles,
                           tile_count, routed, shared);
    else
        hipLaunchKernelGGL((grouped_gemm<KDIM, MODE, MT_LARGE>),
                           dim3(256 * PG<MT_LARGE, gemm_kc<KDIM, MODE, MT_LARGE>()>::WG_PER_CU),
                           dim3(PG<MT_LARGE, gemm_kc<KDIM, MODE, MT_LARGE>()>::THREADS), 0, st, a, tiles,
                           tile_count, routed, shared);
}

// xh_ready: the fp16 activations are already in xh (the router wrote them).
static void launch_gateup(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                          int* tile_count, const QFFN& routed, const QFFN& shared,
                          uint16_t* xh, uint16_t* hbuf, bool xh_ready, hipStream_t st) {
    const size_t chunks = (size_t)T * (H / 8);
    if (!xh_ready)
        hipLaunchKernelGGL(prep_x_f16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, x,
                           T, xh);
    GemmArgs gu = gemm_args(xh, (size_t)T * H * 2, T, perm);
    gu.hout = hbuf;
    launch_gemm<H, GM_GATEUP>(gu, tiles, tile_count, routed, shared, gemm_tile_rows(T), st);
}

void launch_expert_prefill(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                           int* tile_count, int /*max_tiles*/, const QFFN& routed,
                           const QFFN& shared, uint16_t* xh, uint16_t* hbuf, float* dout,
                           hipStream_t st) {
    launch_gateup(x, T, perm, tiles, tile_count, routed, shared, xh, hbuf, false, st);
    GemmArgs dn = gemm_args(hbuf, (size_t)(TOPK + 1) * T * I * 2, T, perm);
    dn.dout32 = dout;
    launch_gemm<I, GM_DOWN_F32>(dn, tiles, tile_count, routed, shared, gemm_tile_rows(T), st);
}

// Whole-layer prefill expert part: gate/up, then down writing fp16 rows of
// (routing weight or shared gate) * d, summed per token by combine_f16.
void launch_expert_prefill_fused(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                                 int* tile_count, int /*max_tiles*/, const QFFN& routed,
                                 const QFFN& shared, uint16_t* xh, uint16_t* hbuf,
                                 uint16_t* d16, const float* wsorted, const float* sg,
                                 bool xh_ready, hipStream_t st) {
    launch_gateup(x, T, perm, tiles, tile_count, routed, shared, xh, hbuf, xh_ready, st);
    GemmArgs dn = gemm_args(hbuf, (size_t)(TOPK + 1) * T * I * 2, T, perm);
    dn.dout16 = d16;
    dn.wsorted = wsorted;
    dn.sg = sg;
    launch_gemm<I, GM_DOWN_F16W>(dn, tiles, tile_count, routed, shared, gemm_tile_rows(T), st);
}

}  // namespace moe
