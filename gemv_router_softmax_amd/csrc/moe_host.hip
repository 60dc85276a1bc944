// moe_host.hip -- the C ABI of libmoe.so: argument validation, workspace
// layout and kernel launches.  Nothing here allocates device memory, copies
// device data to the host or waits on the GPU: every call validates on the
// host and then only enqueues on the caller's stream, so routing results
// never leave the GPU ("Perplexity Open-Sources Lily ...", section "The
// optimizations follow the workload").
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "common.hpp"

namespace moe {
void launch_route(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                  const uint16_t* wsg, float* logits, int32_t* ids, float* wts, float* sg,
                  hipStream_t st, uint16_t* xh = nullptr, float* part = nullptr);
// The router's K-split partials (up to 8 slices of T x E fp32) live in the
// h rows, which nothing reads before the gate/up GEMM rewrites them.
static_assert((size_t)(TOPK + 1) * I * 2 >= (size_t)8 * E * 4, "router partials fit the h rows");
void launch_route_logits(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                         float* logits, hipStream_t st);
void launch_route_select(const float* logits, const uint16_t* x, const uint16_t* wsg, int T,
                         int32_t* ids, float* wts, float* sg, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv, Tile* tiles, int* tile_count,
                         uint16_t* xh, hipStream_t st);
void launch_decode_gateup(const uint16_t* xh, int T, const int32_t* perm, const Tile* tiles,
                          const int* tile_count, int max_tiles, const QFFN& routed,
                          const QFFN& shared, uint16_t* hbuf, hipStream_t st);
void launch_decode_down_combine(const uint16_t* hbuf, int T, const int32_t* perm,
                                const Tile* tiles, const int* tile_count, const float* wts,
                                const float* sg, const QFFN& routed, const QFFN& shared,
                                uint16_t* y, const uint16_t* x, uint16_t* res, hipStream_t st);
void launch_layer_decode_small(const uint16_t* x, int T, const moe_layer& L, float* logits,
                               float* z, uint16_t* xh, uint16_t* hbuf, unsigned* counter,
                               void* rec, uint16_t* y, uint16_t* res, const void* prefetch,
                               size_t prefetch_bytes, hipStream_t st);
size_t route_rec_bytes();
void launch_zero_words(unsigned* p, int n, hipStream_t st);
void launch_permute(const int32_t* ids, int T, int32_t* counts, int32_t* offsets, int32_t* perm,
                    int32_t* inv, int32_t* chunk_counts, hipStream_t st,
                    const float* wts = nullptr, float* wsorted = nullptr, Tile* tiles = nullptr,
                    int* tile_count = nullptr);
void launch_plan(const int32_t* offsets, int T, Tile* tiles, int* tile_count, hipStream_t st);
int perm_chunks(int T);
int max_tiles(int T);
void launch_expert_decode(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                          const int* tile_count, int max_tiles, const QFFN& routed,
                          const QFFN& shared, uint16_t* xh, uint16_t* hbuf, float* dout,
                          hipStream_t st);
void launch_expert_prefill(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                           int* tile_count, int max_tiles, const QFFN& routed,
                           const QFFN& shared, uint16_t* xh, uint16_t* hbuf, float* dout,
                           hipStream_t st);
void launch_expert_prefill_fused(const uint16_t* x, int T, const int32_t* perm, const Tile* tiles,
                                 int* tile_count, int max_tiles, const QFFN& routed,
                                 const QFFN& shared, uint16_t* xh, uint16_t* hbuf,
                                 uint16_t* d16, const float* wsorted, const float* sg,
                                 bool xh_ready, hipStream_t st);
void launch_combine_f16(const uint16_t* d16, const int32_t* inv, int T, uint16_t* y,
                        const uint16_t* x, uint16_t* res, hipStream_t st);
void launch_combine(const float* out, const int32_t* inv, const float* wts, const float* sg, int T,
                    uint16_t* y, const uint16_t* x, uint16_t* res, hipStream_t st);
void launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t st);
void launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t st);

namespace {

constexpr int SYNC_WORDS = 64;

// Workspace regions (byte offsets, each 256-byte aligned).
struct WsLayout {
    size_t sync, rec, logits, ids, wts, sg, counts, offsets, perm, inv, wsorted, chunk_counts, tiles,
        tile_count, xh, h, dout, total;
};

WsLayout ws_layout(int T) {
    WsLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t t = (size_t)T;
    L.sync = take(SYNC_WORDS * 4);      // counters: zero before first use, zero after every call
    L.rec = take(route_rec_bytes());
    L.logits = take(t * E * 4);
    L.ids = take(t * TOPK * 4);
    L.wts = take(t * TOPK * 4);
    L.sg = take(t * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.perm = take(t * TOPK * 4);
    L.inv = take(t * TOPK * 4);
    L.wsorted = take(t * TOPK * 4);
    L.chunk_counts = take((size_t)perm_chunks(T) * E * 4);
    L.tiles = take((size_t)max_tiles(T) * sizeof(Tile));
    L.tile_count = take(TILE_COUNT_WORDS * 4);
    L.xh = take(t * H * 2);
    // h rows: 9T for the tile-based kernels; the few-token layer indexes them
    // (slot * T + token) with up to 1 + 8T slots
    // (kept monotone in T: beyond the few-token range it never shrinks)
    const size_t ts = t < MOE_DECODE_T ? t : MOE_DECODE_T;
    const size_t hrows = std::max((1 + TOPK * ts) * ts, (TOPK + 1) * t);
    L.h = take(hrows * I * 2);
    L.dout = take(t * (TOPK + 1) * H * 4);
    L.total = off;
    return L;
}

template <typename P>
P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool a4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int check_qffn(const moe_qffn* q) {
    if (!q) return MOE_ERR_INVALID_ARG;
    const void* ps[9] = {q->gate_q, q->up_q, q->down_q, q->gate_s, q->gate_b,
                         q->up_s,   q->up_b, q->down_s, q->down_b};
    for (const void* p : ps)
        if (!p) return MOE_ERR_INVALID_ARG;
    for (const void* p : ps)
        if (!a16(p)) return MOE_ERR_ALIGN;
    // 0 (dense) or a per-expert block of at least one code matrix, 256-byte
    // granular, small enough for the kernels' 32-bit strides
    const int64_t st = q->expert_stride;
    if (st != 0 && (st < (int64_t)DENSE_SQ || st % 256 != 0 || st > (int64_t)(1u << 31)))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int check_T(int T) { return (T < 0 || T > MOE_T_MAX) ? MOE_ERR_INVALID_ARG : MOE_OK; }

int launch_status() {
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int pick_path(int T, const moe_options* opt, int* path) {
    const int want = opt ? opt->path : MOE_PATH_AUTO;
    if (want == MOE_PATH_AUTO) {
        *path = T <= MOE_DECODE_T ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
        return MOE_OK;
    }
    if (want == MOE_PATH_DECODE) {
        if (T > MOE_DECODE_T_MAX) return MOE_ERR_INVALID_ARG;
        *path = want;
        return MOE_OK;
    }
    if (want == MOE_PATH_PREFILL) {
        *path = want;
        return MOE_OK;
    }
    return MOE_ERR_INVALID_ARG;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(int T) {
    if (T < 0 || T > MOE_T_MAX) return 0;
    return ws_layout(T).total;
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

int moe_route(const uint16_t* x, int T, const uint16_t* w_router, const float* router_bias,
              const uint16_t* w_shared_gate, int32_t* topk_ids, float* topk_w,
              float* shared_gate, void* ws, size_t ws_bytes, void* stream) {
    if (check_T(T)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !w_shared_gate || !topk_ids || !topk_w || !shared_gate || !ws)
        return MOE_ERR_INVALID_ARG;
    if (!a16(x) || !a16(w_router) || !a16(w_shared_gate) || !a16(ws) ||
        (router_bias && !a4(router_bias)) || !a4(topk_ids) || !a4(topk_w) || !a4(shared_gate))
        return MOE_ERR_ALIGN;
    const WsLayout L = ws_layout(T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (T <= MOE_DECODE_T_MAX) {
        launch_route_logits(x, T, w_router, router_bias, at<float>(ws, L.logits), st);
        launch_route_select(at<float>(ws, L.logits), x, w_shared_gate, T, topk_ids, topk_w,
                            shared_gate, at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                            at<int32_t>(ws, L.perm), at<int32_t>(ws, L.inv), at<Tile>(ws, L.tiles),
                            at<int>(ws, L.tile_count), at<uint16_t>(ws, L.xh), st);
    } else {
        launch_route(x, T, w_router, router_bias, w_shared_gate, at<float>(ws, L.logits),
                     topk_ids, topk_w, shared_gate, st, nullptr, at<float>(ws, L.h));
    }
    return launch_status();
}

int moe_permute(const int32_t* topk_ids, int T, int32_t* expert_counts, int32_t* expert_offsets,
                int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
    if (check_T(T)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !expert_counts || !expert_offsets || !perm || !inv_perm || !ws)
        return MOE_ERR_INVALID_ARG;
    if (!a4(topk_ids) || !a4(expert_counts) || !a4(expert_offsets) || !a4(perm) ||
        !a4(inv_perm) || !a16(ws))
        return MOE_ERR_ALIGN;
    const WsLayout L = ws_layout(T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    launch_permute(topk_ids, T, expert_counts, expert_offsets, perm, inv_perm,
                   at<int32_t>(ws, L.chunk_counts),
                   (hipStream_t)stream);
    return launch_status();
}

int moe_expert_ffn(const uint16_t* x, int T, const moe_qffn* routed, const moe_qffn* shared,
                   const int32_t* expert_offsets, const int32_t* perm, float* expert_out,
                   void* ws, size_t ws_bytes, void* stream, const moe_options* opt) {
    if (check_T(T)) return MOE_ERR_INVALID_ARG;
    int path;
    if (pick_path(T, opt, &path)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !expert_offsets || !perm || !expert_out || !ws) return MOE_ERR_INVALID_ARG;
    if (int rc = check_qffn(routed)) return rc;
    if (int rc = check_qffn(shared)) return rc;
    if (!a16(x) || !a4(expert_offsets) || !a4(perm) || !a16(expert_out) || !a16(ws))
        return MOE_ERR_ALIGN;
    const WsLayout L = ws_layout(T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    Tile* tiles = at<Tile>(ws, L.tiles);
    int* tcount = at<int>(ws, L.tile_count);
    uint16_t* hbuf = at<uint16_t>(ws, L.h);
    launch_plan(expert_offsets, T, tiles, tcount, st);
    if (path == MOE_PATH_DECODE)
        launch_expert_decode(x, T, perm, tiles, tcount, max_tiles(T), qffn_view(*routed),
                             qffn_view(*shared),
                             at<uint16_t>(ws, L.xh), hbuf, expert_out, st);
    else
        launch_expert_prefill(x, T, perm, tiles, tcount, max_tiles(T), qffn_view(*routed),
                              qffn_view(*shared),
                              at<uint16_t>(ws, L.xh), hbuf,
                              expert_out, st);
    return launch_status();
}

int moe_combine(const float* expert_out, const int32_t* inv_perm, const float* topk_w,
                const float* shared_gate, int T, uint16_t* y, void* stream) {
    if (check_T(T)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!expert_out || !inv_perm || !topk_w || !shared_gate || !y) return MOE_ERR_INVALID_ARG;
    if (!a16(expert_out) || !a4(inv_perm) || !a4(topk_w) || !a4(shared_gate) || !a16(y))
        return MOE_ERR_ALIGN;
    launch_combine(expert_out, inv_perm, topk_w, shared_gate, T, y, nullptr, nullptr,
                   (hipStream_t)stream);
    return launch_status();
}

int moe_layer_forward_ex(const uint16_t* x, int T, const moe_layer* layer, uint16_t* y, void* ws,
                         size_t ws_bytes, void* stream, const moe_options* opt) {
    if (check_T(T)) return MOE_ERR_INVALID_ARG;
    int path;
    if (pick_path(T, opt, &path)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !layer || !y || !ws || !layer->w_router || !layer->w_shared_gate)
        return MOE_ERR_INVALID_ARG;
    if (int rc = check_qffn(&layer->routed)) return rc;
    if (int rc = check_qffn(&layer->shared)) return rc;
    uint16_t* res = opt ? opt->residual_out : nullptr;
    const void* pf = opt ? opt->prefetch : nullptr;
    const size_t pf_bytes = pf ? opt->prefetch_bytes : 0;
    if (pf && (pf_bytes % 16 != 0 || pf_bytes > MOE_PREFETCH_MAX)) return MOE_ERR_INVALID_ARG;
    if (!a16(x) || !a16(y) || !a16(ws) || !a16(layer->w_router) || !a16(layer->w_shared_gate) ||
        (layer->router_bias && !a4(layer->router_bias)) || (res && !a16(res)) || (pf && !a16(pf)))
        return MOE_ERR_ALIGN;
    const WsLayout L = ws_layout(T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int32_t* ids = at<int32_t>(ws, L.ids);
    float* wts = at<float>(ws, L.wts);
    float* sg = at<float>(ws, L.sg);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    Tile* tiles = at<Tile>(ws, L.tiles);
    int* tcount = at<int>(ws, L.tile_count);
    uint16_t* hbuf = at<uint16_t>(ws, L.h);
    float* dout = at<float>(ws, L.dout);

    if (path == MOE_PATH_DECODE && T <= MOE_DECODE_T) {
        // three kernels: logits (+ shared gate logit, fp16 x) | gate/up | down+combine;
        // the routing is recomputed inside the two expert kernels
        launch_layer_decode_small(x, T, *layer, at<float>(ws, L.logits), sg,
                                  at<uint16_t>(ws, L.xh), hbuf, at<unsigned>(ws, L.sync),
                                  at<char>(ws, L.rec), y, res, pf, pf_bytes, st);
        return launch_status();
    }
    if (path == MOE_PATH_DECODE) {
        // four kernels: logits | select (top-8, permutation, tiles) | gate/up | down+combine
        launch_route_logits(x, T, layer->w_router, layer->router_bias, at<float>(ws, L.logits),
                            st);
        uint16_t* xh = at<uint16_t>(ws, L.xh);
        launch_route_select(at<float>(ws, L.logits), x, layer->w_shared_gate, T, ids, wts, sg,
                            counts, offsets, perm, inv, tiles, tcount, xh, st);
        launch_decode_gateup(xh, T, perm, tiles, tcount, max_tiles(T), qffn_view(layer->routed),
                             qffn_view(layer->shared), hbuf, st);
        launch_decode_down_combine(hbuf, T, perm, tiles, tcount, wts, sg,
                                   qffn_view(layer->routed), qffn_view(layer->shared), y, x, res,
                                   st);
        return launch_status();
    }
    // the top-8 kernel also writes the fp16 activations the grouped GEMM reads
    uint16_t* xh = at<uint16_t>(ws, L.xh);
    launch_route(x, T, layer->w_router, layer->router_bias, layer->w_shared_gate,
                 at<float>(ws, L.logits), ids, wts, sg, st, xh, at<float>(ws, L.h));
    float* wsorted = at<float>(ws, L.wsorted);
    launch_permute(ids, T, counts, offsets, perm, inv, at<int32_t>(ws, L.chunk_counts), st, wts,
                   wsorted, tiles, tcount);
    // fp16 rows of weight * d (half the bytes of fp32 expert outputs)
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dout);
    launch_expert_prefill_fused(x, T, perm, tiles, tcount, max_tiles(T), qffn_view(layer->routed),
                                qffn_view(layer->shared), xh, hbuf, d16, wsorted, sg,
                                /*xh_ready=*/true, st);
    launch_combine_f16(d16, inv, T, y, x, res, st);
    return launch_status();
}

int moe_layer_forward(const uint16_t* x, int T, const moe_layer* layer, uint16_t* y, void* ws,
                      size_t ws_bytes, void* stream) {
    return moe_layer_forward_ex(x, T, layer, y, ws, ws_bytes, stream, nullptr);
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    if (!a16(ws)) return MOE_ERR_ALIGN;
    if (ws_bytes < moe_workspace_bytes(0)) return MOE_ERR_WORKSPACE;
    launch_zero_words(at<unsigned>(ws, ws_layout(0).sync), SYNC_WORDS, (hipStream_t)stream);
    return launch_status();
}

int moe_probe_read(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink || bytes == 0 || (bytes & 15)) return MOE_ERR_INVALID_ARG;
    if (!a16(src) || !a4(sink)) return MOE_ERR_ALIGN;
    launch_probe_read(src, bytes, sink, (hipStream_t)stream);
    return launch_status();
}

int moe_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!src || !dst || bytes == 0 || (bytes & 15)) return MOE_ERR_INVALID_ARG;
    if (!a16(src) || !a16(dst)) return MOE_ERR_ALIGN;
    launch_probe_copy(dst, src, bytes, (hipStream_t)stream);
    return launch_status();
}

}  // extern "C"
