// permute.hip -- token -> expert permutation (stable counting sort) and the
// row-tile list of the grouped expert kernels.
//
// The permutation is a pure integer function of the expert ids, so it is
// computed bit-exactly: a histogram, an exclusive scan and a stable scatter
// whose in-block ranks come from wave ballots (no order-dependent atomics
// decide a position).  Each expert's segment lists its slots f = 8t + j in
// ascending order.
//
//   perm_small      one workgroup does everything (8T <= PERM_SMALL_MAX entries)
//   perm_count      larger T: per-chunk expert histograms      (grid: chunks)
//   perm_scan_scatter  up to SCAN_CHUNKS chunks: every workgroup derives its
//                   chunk's bases from all the histograms, then scatters it;
//                   one more workgroup writes the counts and offsets and
//                   plans the row tiles meanwhile            (grid: chunks + 1)
//   perm_scan       more chunks: column scans -> per-chunk bases (one workgroup)
//   perm_scatter    more chunks: stable scatter of every chunk   (grid: chunks)
//   plan_tiles      row tiles of <= mt_rows rows per expert (expert 256 is the
//                   shared expert over all T tokens), read by the expert
//                   kernels from device memory so the host never needs the
//                   expert counts.  The layer call plans inside perm_small /
//                   perm_scan (one launch fewer); the split interface plans
//                   from the caller's offsets with the plan_tiles kernel.
#include "block_util.hpp"

namespace moe {

// (PERM_CHUNK entries per chunk in the large path: two rounds of the block
// scatter per workgroup; PERM_SMALL_MAX entries handled by perm_small)
constexpr int SCAN_CHUNKS = 64;    // chunks handled by perm_scan_scatter (T <= 4096); each of
                                   // its workgroups reads every chunk's histogram

// Row tiles: routed expert e owns rows offsets[e] .. offsets[e+1]-1, the
// shared expert (group 256) owns rows 8T .. 9T-1.  A group of n rows is cut
// into nt = ceil(n/mt_rows) tiles of as equal a size as possible (the first
// n % nt tiles get one row more), so no group leaves a small remainder tile.
// At most `cap` tiles are written (offsets from moe_permute never need more
// than max_tiles(T); malformed caller offsets cannot overrun the buffer).
__device__ inline Tile balanced_tile(int group, int r0, int n, int nt, int i) {
    const int base = n / nt, rem = n % nt;
    Tile tl;
    tl.group = group;
    tl.row0 = r0 + i * base + min(i, rem);
    tl.nrows = base + (i < rem ? 1 : 0);
    tl.pad = 0;
    return tl;
}

// Tiles are written in descending order of their count of 32-row MFMA
// tiles (their cost in the grouped GEMMs, whose dynamic schedule then runs
// longest-first); within a class, routed experts in order, then the shared
// expert.  Also zeroes the GEMMs' work counters.  Thread e of the 256-thread
// block passes expert e's rows [o0, o1) (caller-provided offsets are clamped
// into the routed row space [0, 8T)); scr: 4 ints of LDS; mt_rows: tile
// height, a multiple of 32 in [MT_MIN_ROWS, MT_ROWS].
__device__ void plan_block(int o0, int o1, int T, int cap, int mt_rows, Tile* __restrict__ tiles,
                           int* __restrict__ tile_count, int* scr) {
    const int tid = threadIdx.x;
    const int lim = TOPK * T;
    const int r0 = min(max(o0, 0), lim);
    const int r1 = min(max(o1, r0), lim);
    const int n = r1 - r0;
    const int nt = (n + mt_rows - 1) / mt_rows;
    const int ns = (T + mt_rows - 1) / mt_rows;
    auto cls = [](const Tile& t) { return (t.nrows + 31) >> 5; };
    int before = 0;
    for (int c = mt_rows / 32; c >= 1; --c) {
        int mine = 0;
        for (int i = 0; i < nt; ++i) mine += cls(balanced_tile(tid, r0, n, nt, i)) == c;
        for (int i = tid; i < ns; i += 256) mine += cls(balanced_tile(E, lim, T, ns, i)) == c;
        int tot;
        int pos = before + block_excl_scan256(mine, scr, &tot);
        for (int i = 0; i < nt; ++i) {
            const Tile tl = balanced_tile(tid, r0, n, nt, i);
            if (cls(tl) == c) {
                if (pos < cap) tiles[pos] = tl;
                ++pos;
            }
        }
        for (int i = tid; i < ns; i += 256) {
            const Tile tl = balanced_tile(E, lim, T, ns, i);
            if (cls(tl) == c) {
                if (pos < cap) tiles[pos] = tl;
                ++pos;
            }
        }
        before += tot;
    }
    if (tid == 0) *tile_count = min(before, cap);
    if (tid >= GEMM_CTR_GATEUP && tid < TILE_COUNT_WORDS) tile_count[tid] = 0;
}

__global__ __launch_bounds__(256) void plan_tiles(const int32_t* __restrict__ offsets, int T,
                                                  int cap, int mt_rows, Tile* __restrict__ tiles,
                                                  int* __restrict__ tile_count) {
    __shared__ int scr[4];
    plan_block(offsets[threadIdx.x], offsets[threadIdx.x + 1], T, cap, mt_rows, tiles, tile_count,
               scr);
}

// Tiles any plan of T tokens can need (at the smallest tile height).
__host__ __device__ int max_tiles(int T) {
    const int n = TOPK * T;
    return n / MT_MIN_ROWS + (n < E ? n : E) + (T + MT_MIN_ROWS - 1) / MT_MIN_ROWS;
}

__global__ __launch_bounds__(256) void perm_small(const int32_t* __restrict__ ids, int n,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm,
                                                  int32_t* __restrict__ inv,
                                                  const float* __restrict__ wsrc,
                                                  float* __restrict__ wsorted, int T,
                                                  int mt_rows, Tile* __restrict__ tiles,
                                                  int* __restrict__ tile_count) {
    __shared__ int hist[256];
    __shared__ int base[256];
    __shared__ int wcnt[4 * 256];
    __shared__ int scr[4];
    const int tid = threadIdx.x;
    hist[tid] = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w * 256 + tid] = 0;
    __syncthreads();
    for (int f = tid; f < n; f += 256) {
        int e = ids[f];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    const int c = hist[tid];
    int total;
    const int off = block_excl_scan256(c, scr, &total);
    counts[tid] = c;
    offsets[tid] = off;
    if (tid == 0) offsets[E] = total;
    base[tid] = off;
    __syncthreads();
    stable_scatter(ids, 0, n, base, wcnt, perm, inv, wsrc, wsorted);
    if (tiles) plan_block(off, off + c, T, max_tiles(T), mt_rows, tiles, tile_count, scr);
}

__global__ __launch_bounds__(256) void perm_count(const int32_t* __restrict__ ids, int n,
                                                  int32_t* __restrict__ chunk_counts) {
    __shared__ int hist[256];
    const int tid = threadIdx.x;
    hist[tid] = 0;
    __syncthreads();
    const int f0 = blockIdx.x * PERM_CHUNK, f1 = min(n, f0 + PERM_CHUNK);
    for (int f = f0 + tid; f < f1; f += 256) {
        int e = ids[f];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    chunk_counts[(size_t)blockIdx.x * 256 + tid] = hist[tid];
}

// One workgroup: chunk_counts[b][e] becomes the first position of chunk
// b's entries of expert e relative to the expert's segment (the scatter adds
// offsets[e]); counts and offsets are written, and the row tiles planned if
// `tiles` is given.  Thread e reads its column 64 chunks at a time (every
// chunk of a 4096-token call at once), so the loads of a batch are in
// flight together.
__global__ __launch_bounds__(256) void perm_scan(int nchunks, int32_t* __restrict__ chunk_counts,
                                                 int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ offsets, int T,
                                                 int mt_rows, Tile* __restrict__ tiles,
                                                 int* __restrict__ tile_count) {
    __shared__ int scr[4];
    const int tid = threadIdx.x;
    int run = 0;
    for (int b0 = 0; b0 < nchunks; b0 += 64) {
        int c[64];
#pragma unroll
        for (int i = 0; i < 64; ++i)
            c[i] = b0 + i < nchunks ? chunk_counts[(size_t)(b0 + i) * 256 + tid] : 0;
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            if (b0 + i < nchunks) chunk_counts[(size_t)(b0 + i) * 256 + tid] = run;
            run += c[i];
        }
    }
    int total;
    const int off = block_excl_scan256(run, scr, &total);
    counts[tid] = run;
    offsets[tid] = off;
    if (tid == 0) offsets[E] = total;
    if (tiles) plan_block(off, off + run, T, max_tiles(T), mt_rows, tiles, tile_count, scr);
}

__global__ __launch_bounds__(256) void perm_scatter(const int32_t* __restrict__ ids, int n,
                                                    const int32_t* __restrict__ chunk_base,
                                                    const int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ inv,
                                                    const float* __restrict__ wsrc,
                                                    float* __restrict__ wsorted) {
    __shared__ int base[256];
    __shared__ int wcnt[4 * 256];
    const int tid = threadIdx.x;
    base[tid] = chunk_base[(size_t)blockIdx.x * 256 + tid] + offsets[tid];
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w * 256 + tid] = 0;
    __syncthreads();
    const int f0 = blockIdx.x * PERM_CHUNK, f1 = min(n, f0 + PERM_CHUNK);
    stable_scatter(ids, f0, f1, base, wcnt, perm, inv, wsrc, wsorted);
}

// Up to SCAN_CHUNKS chunks.  Thread e reads expert e's count in every chunk
// (all loads in flight together): its entries in chunks before this one
// give the chunk's base inside the expert's segment, the total its segment
// length; a block scan of the totals gives the segment starts.  The scan
// is repeated by every workgroup instead of run once between two launches.
// Workgroup `nchunks` (the last) scatters nothing: it writes counts and
// offsets and plans the row tiles while the others scatter.
__global__ __launch_bounds__(256) void perm_scan_scatter(const int32_t* __restrict__ ids, int n,
                                                         int nchunks,
                                                         const int32_t* __restrict__ chunk_counts,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv,
                                                         const float* __restrict__ wsrc,
                                                         float* __restrict__ wsorted, int T,
                                                         int mt_rows, Tile* __restrict__ tiles,
                                                         int* __restrict__ tile_count) {
    __shared__ int base[256];
    __shared__ int wcnt[4 * 256];
    __shared__ int scr[4];
    const int tid = threadIdx.x, b = blockIdx.x;
    int c[SCAN_CHUNKS];
#pragma unroll
    for (int i = 0; i < SCAN_CHUNKS; ++i) c[i] = i < nchunks ? chunk_counts[(size_t)i * 256 + tid] : 0;
    int pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < SCAN_CHUNKS; ++i) {
        pre += i < b ? c[i] : 0;
        tot += c[i];
    }
    int total;
    const int off = block_excl_scan256(tot, scr, &total);
    base[tid] = off + pre;
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w * 256 + tid] = 0;
    __syncthreads();
    if (b == nchunks) {
        counts[tid] = tot;
        offsets[tid] = off;
        if (tid == 0) offsets[E] = total;
        if (tiles) plan_block(off, off + tot, T, max_tiles(T), mt_rows, tiles, tile_count, scr);
        return;
    }
    const int f0 = b * PERM_CHUNK, f1 = min(n, f0 + PERM_CHUNK);
    stable_scatter(ids, f0, f1, base, wcnt, perm, inv, wsrc, wsorted);
}

int perm_chunks(int T) { return (TOPK * T + PERM_CHUNK - 1) / PERM_CHUNK; }

// wts/wsorted: optional (both or neither): wsorted[p] = wts[perm[p]], the
// routing weight of each sorted position.
int gemm_tile_rows(int T);

// tiles/tile_count: optional (both or neither): also plan the row tiles
// (and zero the GEMMs' work counters), as launch_plan would.
// counted: chunk_counts already holds the chunk histograms (the layer
// call's top-8 kernel accumulates them).
void launch_permute(const int32_t* ids, int T, int32_t* counts, int32_t* offsets, int32_t* perm,
                    int32_t* inv, int32_t* chunk_counts, hipStream_t st, const float* wts,
                    float* wsorted, Tile* tiles, int* tile_count, bool counted) {
    const int mt = gemm_tile_rows(T);
    const int n = TOPK * T;
    if (n <= PERM_SMALL_MAX) {
        hipLaunchKernelGGL(perm_small, dim3(1), dim3(256), 0, st, ids, n, counts, offsets, perm,
                           inv, wts, wsorted, T, mt, tiles, tile_count);
        return;
    }
    const int nb = perm_chunks(T);
    if (!counted) hipLaunchKernelGGL(perm_count, dim3(nb), dim3(256), 0, st, ids, n, chunk_counts);
    if (nb <= SCAN_CHUNKS) {
        hipLaunchKernelGGL(perm_scan_scatter, dim3(nb + 1), dim3(256), 0, st, ids, n, nb, chunk_counts,
                           counts, offsets, perm, inv, wts, wsorted, T, mt, tiles, tile_count);
        return;
    }
    hipLaunchKernelGGL(perm_scan, dim3(1), dim3(256), 0, st, nb, chunk_counts, counts, offsets, T,
                       mt, tiles, tile_count);
    hipLaunchKernelGGL(perm_scatter, dim3(nb), dim3(256), 0, st, ids, n, chunk_counts, offsets,
                       perm, inv, wts, wsorted);
}

void launch_plan(const int32_t* offsets, int T, Tile* tiles, int* tile_count, hipStream_t st) {
    hipLaunchKernelGGL(plan_tiles, dim3(1), dim3(256), 0, st, offsets, T, max_tiles(T),
                       gemm_tile_rows(T), tiles, tile_count);
}

}  // namespace moe
