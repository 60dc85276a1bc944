// moe_host.hip -- the C ABI of libmoe.so: argument validation, workspace
// layout and kernel launches.  Nothing here allocates device memory, copies
// device data to the host or waits on the GPU: every call validates on the
// host and then only enqueues on the caller's stream, so routing results
// never leave the GPU ("Perplexity Open-Sources Lily ...", section "The
// optimizations follow the workload").
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace moe {
void launch_route(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                  const uint16_t* wsg, float* logits, int32_t* ids, float* wts, float* sg,
                  hipStream_t st, uint16_t* xh = nullptr, float* part = nullptr,
                  int32_t* chunk_counts = nullptr);
bool route_counts_chunks(int T);
// The router's K-split partials (up to 8 slices of T x E fp32) live in the
// h rows, which nothing reads before the gate/up GEMM rewrites them.
static_assert((size_t)(TOPK + 1) * I * 2 >= (size_t)8 * E * 4, "router partials fit the h rows");
void launch_route_logits(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                         float* logits, hipStream_t st, int32_t* zero = nullptr, int nzero = 0);
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
void launch_layer_decode_small(const uint16_t* x, int T, const moe_layer& L, bool first,
                               long long* acc_cur, long long* acc_next, const moe_layer* next,
                               uint16_t* xh, uint16_t* hbuf, void* rec, uint16_t* y,
                               uint16_t* res, int32_t* ids_out, float* w_out, float* sg_out,
                               hipStream_t st);
size_t route_rec_bytes();
size_t route_acc_bytes(int T);
void launch_permute(const int32_t* ids, int T, int32_t* counts, int32_t* offsets, int32_t* perm,
                    int32_t* inv, int32_t* chunk_counts, hipStream_t st,
                    const float* wts = nullptr, float* wsorted = nullptr, Tile* tiles = nullptr,
                    int* tile_count = nullptr, bool counted = false);
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
void launch_router_transpose(const uint16_t* wr, uint16_t* wrt, hipStream_t st);
size_t head_part_bytes();
void launch_head_argmax(const uint16_t* x, int T, const uint16_t* w, int V, int32_t* token,
                        unsigned long long* part, hipStream_t st);
void launch_embed(const int32_t* token, int T, const uint16_t* emb, int V, uint16_t* x,
                  hipStream_t st);
void launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t st);
void launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t st);

namespace {

// Workspace regions (byte offsets, each 256-byte aligned).
struct WsLayout {
    size_t rec, acc, head, logits, ids, wts, sg, counts, offsets, perm, inv, wsorted, chunk_counts,
        tiles, tile_count, xh, h, dout, chain, total;
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
    // (kept monotone in T: the few-token regions never shrink beyond that range)
    const size_t ts = t < MOE_DECODE_T ? t : MOE_DECODE_T;
    L.rec = take(route_rec_bytes());
    L.acc = take(route_acc_bytes((int)ts));     // two sets of fixed-point logits
    L.head = take(head_part_bytes());           // greedy selection: per-workgroup keys
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
    L.h = take((TOPK + 1) * t * I * 2);
    L.dout = take(t * (TOPK + 1) * H * 4);
    L.chain = take(3 * t * H * 2);              // chains: two residual buffers and a y buffer
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

}  // extern "C"

namespace moe {
namespace {

// Validation shared by the layer and chain calls (one layer descriptor).
int check_layer(const moe_layer* layer) {
    if (!layer || !layer->w_router || !layer->w_shared_gate) return MOE_ERR_INVALID_ARG;
    if (int rc = check_qffn(&layer->routed)) return rc;
    if (int rc = check_qffn(&layer->shared)) return rc;
    if (!a16(layer->w_router) || !a16(layer->w_shared_gate) ||
        (layer->router_bias && !a4(layer->router_bias)) ||
        (layer->w_router_t && !a16(layer->w_router_t)))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

// Route outputs requested through moe_options: all three or none.
int check_route_out(const moe_options* opt) {
    if (!opt) return MOE_OK;
    const int n = (opt->route_ids != nullptr) + (opt->route_w != nullptr) + (opt->route_sg != nullptr);
    if (n != 0 && n != 3) return MOE_ERR_INVALID_ARG;
    if (n == 3 && (!a4(opt->route_ids) || !a4(opt->route_w) || !a4(opt->route_sg))) return MOE_ERR_ALIGN;
    return MOE_OK;
}

// The prefill path of one layer in two halves: the front (router GEMM,
// top-8, permutation and tile plan) writes only the workspace; the back
// (grouped GEMMs, combine) reads the workspace and writes y (and res).
// ids/wts/sg: where the front puts the routing (the caller's route outputs
// or the workspace's); the back reads sg from the same place.
void prefill_front(const uint16_t* x, int T, const moe_layer* layer, void* ws, const WsLayout& L,
                   int32_t* ids, float* wts, float* sg, hipStream_t st) {
    // the top-8 kernel also writes the fp16 activations the grouped GEMM reads
    // and, for chunked permutations, the chunk histograms
    launch_route(x, T, layer->w_router, layer->router_bias, layer->w_shared_gate,
                 at<float>(ws, L.logits), ids, wts, sg, st, at<uint16_t>(ws, L.xh),
                 at<float>(ws, L.h), at<int32_t>(ws, L.chunk_counts));
    launch_permute(ids, T, at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                   at<int32_t>(ws, L.perm), at<int32_t>(ws, L.inv),
                   at<int32_t>(ws, L.chunk_counts), st, wts, at<float>(ws, L.wsorted),
                   at<Tile>(ws, L.tiles), at<int>(ws, L.tile_count), route_counts_chunks(T));
}

void prefill_back(const uint16_t* x, int T, const moe_layer* layer, uint16_t* y, uint16_t* res,
                  void* ws, const WsLayout& L, const float* sg, hipStream_t st) {
    // fp16 rows of weight * d (half the bytes of fp32 expert outputs)
    uint16_t* d16 = at<uint16_t>(ws, L.dout);
    launch_expert_prefill_fused(x, T, at<int32_t>(ws, L.perm), at<Tile>(ws, L.tiles),
                                at<int>(ws, L.tile_count), max_tiles(T), qffn_view(layer->routed),
                                qffn_view(layer->shared), at<uint16_t>(ws, L.xh),
                                at<uint16_t>(ws, L.h), d16, at<float>(ws, L.wsorted), sg,
                                /*xh_ready=*/true, st);
    launch_combine_f16(d16, at<int32_t>(ws, L.inv), T, y, x, res, st);
}

// One layer, arguments already validated.  ids_out/w_out/sg_out: the
// caller's route outputs, or NULL (the routing then stays in the workspace).
void layer_forward(const uint16_t* x, int T, int path, const moe_layer* layer, uint16_t* y,
                   uint16_t* res, void* ws, const WsLayout& L, int32_t* ids_out, float* w_out,
                   float* sg_out, hipStream_t st) {
    int32_t* ids = ids_out ? ids_out : at<int32_t>(ws, L.ids);
    float* wts = ids_out ? w_out : at<float>(ws, L.wts);
    float* sg = ids_out ? sg_out : at<float>(ws, L.sg);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    Tile* tiles = at<Tile>(ws, L.tiles);
    int* tcount = at<int>(ws, L.tile_count);
    uint16_t* hbuf = at<uint16_t>(ws, L.h);
    float* dout = at<float>(ws, L.dout);
    uint16_t* xh = at<uint16_t>(ws, L.xh);

    if (path == MOE_PATH_DECODE && T <= MOE_DECODE_T) {
        // router logits, gate/up (routing inside), down + combine
        launch_layer_decode_small(x, T, *layer, /*first=*/true, at<long long>(ws, L.acc), nullptr,
                                  nullptr, xh, hbuf, at<char>(ws, L.rec), y, res, ids_out, w_out,
                                  sg_out, st);
        return;
    }
    if (path == MOE_PATH_DECODE) {
        // four kernels: logits | select (top-8, permutation, tiles) | gate/up | down+combine
        launch_route_logits(x, T, layer->w_router, layer->router_bias, at<float>(ws, L.logits), st);
        launch_route_select(at<float>(ws, L.logits), x, layer->w_shared_gate, T, ids, wts, sg,
                            counts, offsets, perm, inv, tiles, tcount, xh, st);
        launch_decode_gateup(xh, T, perm, tiles, tcount, max_tiles(T), qffn_view(layer->routed),
                             qffn_view(layer->shared), hbuf, st);
        launch_decode_down_combine(hbuf, T, perm, tiles, tcount, wts, sg, qffn_view(layer->routed),
                                   qffn_view(layer->shared), y, x, res, st);
        return;
    }
    prefill_front(x, T, layer, ws, L, ids, wts, sg, st);
    prefill_back(x, T, layer, y, res, ws, L, sg, st);
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_layer_forward_ex(const uint16_t* x, int T, const moe_layer* layer, uint16_t* y, void* ws,
                         size_t ws_bytes, void* stream, const moe_options* opt) {
    if (check_T(T)) return MOE_ERR_INVALID_ARG;
    int path;
    if (pick_path(T, opt, &path)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !y || !ws) return MOE_ERR_INVALID_ARG;
    if (int rc = check_layer(layer)) return rc;
    if (int rc = check_route_out(opt)) return rc;
    uint16_t* res = opt ? opt->residual_out : nullptr;
    if (!a16(x) || !a16(y) || !a16(ws) || (res && !a16(res))) return MOE_ERR_ALIGN;
    const WsLayout L = ws_layout(T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    const bool ro = opt && opt->route_ids;
    layer_forward(x, T, path, layer, y, res, ws, L, ro ? opt->route_ids : nullptr,
                  ro ? opt->route_w : nullptr, ro ? opt->route_sg : nullptr, (hipStream_t)stream);
    return launch_status();
}

int moe_layer_forward(const uint16_t* x, int T, const moe_layer* layer, uint16_t* y, void* ws,
                      size_t ws_bytes, void* stream) {
    return moe_layer_forward_ex(x, T, layer, y, ws, ws_bytes, stream, nullptr);
}

int moe_chain_forward(const uint16_t* x, int T, const moe_layer* layers, int nlayers,
                      uint16_t* x_out, uint16_t* y_layers, void* ws, size_t ws_bytes, void* stream,
                      const moe_options* opt) {
    if (check_T(T) || nlayers < 0) return MOE_ERR_INVALID_ARG;
    int path;
    if (pick_path(T, opt, &path)) return MOE_ERR_INVALID_ARG;
    if (opt && opt->residual_out) return MOE_ERR_INVALID_ARG;     // the chain's output is x_out
    if (T == 0 || nlayers == 0) return MOE_OK;
    if (!x || !layers || !x_out || !ws) return MOE_ERR_INVALID_ARG;
    for (int l = 0; l < nlayers; ++l)
        if (int rc = check_layer(&layers[l])) return rc;
    if (int rc = check_route_out(opt)) return rc;
    if (!a16(x) || !a16(x_out) || !a16(ws) || (y_layers && !a16(y_layers))) return MOE_ERR_ALIGN;
    const WsLayout L = ws_layout(T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const size_t tH = (size_t)T * H;
    uint16_t* xb[2] = {at<uint16_t>(ws, L.chain), at<uint16_t>(ws, L.chain) + tH};
    uint16_t* yscratch = at<uint16_t>(ws, L.chain) + 2 * tH;
    const bool ro = opt && opt->route_ids;
    const bool few = path == MOE_PATH_DECODE && T <= MOE_DECODE_T;
    long long* acc[2] = {at<long long>(ws, L.acc),
                         at<long long>(ws, L.acc) + route_acc_bytes(T) / 2 / sizeof(long long)};
    for (int l = 0; l < nlayers; ++l) {
        const uint16_t* xl = l == 0 ? x : xb[(l - 1) & 1];
        uint16_t* res = l == nlayers - 1 ? x_out : xb[l & 1];
        uint16_t* yl = y_layers ? y_layers + (size_t)l * tH : yscratch;
        int32_t* ids = ro ? opt->route_ids + (size_t)l * T * TOPK : nullptr;
        float* w = ro ? opt->route_w + (size_t)l * T * TOPK : nullptr;
        float* sg = ro ? opt->route_sg + (size_t)l * T : nullptr;
        if (few) {
            // two kernels per layer after the first: each down kernel also
            // forms the next layer's router logits and fp16 input (when the
            // next layer carries its transposed router matrix)
            const bool fused_in = l > 0 && layers[l].w_router_t != nullptr;
            const moe_layer* next =
                l + 1 < nlayers && layers[l + 1].w_router_t ? &layers[l + 1] : nullptr;
            launch_layer_decode_small(xl, T, layers[l], !fused_in, acc[l & 1], acc[(l + 1) & 1], next,
                                      at<uint16_t>(ws, L.xh), at<uint16_t>(ws, L.h),
                                      at<char>(ws, L.rec), y_layers ? yl : nullptr, res, ids, w, sg,
                                      st);
        } else {
            layer_forward(xl, T, path, &layers[l], yl, res, ws, L, ids, w, sg, st);
        }
    }
    return launch_status();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Chunked prefill: a second stream per device (default priority), created on
// the first chunked call on that device, and the events that order it
// against the caller's stream.
namespace {
struct ChunkStreams {
    hipStream_t aux = nullptr;
    hipEvent_t fork = nullptr, routed[2] = {}, done[2] = {};
};
std::mutex g_chunk_mutex;
ChunkStreams g_chunk[64];

// The current device's stream and events (NULL on a HIP error).
ChunkStreams* chunk_streams() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_chunk_mutex);
    ChunkStreams& c = g_chunk[dev];
    if (!c.aux) {
        ChunkStreams n;
        bool ok = hipStreamCreateWithFlags(&n.aux, hipStreamNonBlocking) == hipSuccess;
        hipEvent_t* evs[5] = {&n.fork, &n.routed[0], &n.routed[1], &n.done[0], &n.done[1]};
        for (hipEvent_t* e : evs)
            ok = ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
        if (!ok) return nullptr;      // (a partial set is not kept; the call reports the error)
        c = n;
    }
    return &c;
}
}  // namespace

extern "C" {

int moe_layer_forward_chunked(const uint16_t* x, int T, const moe_layer* layer, uint16_t* y,
                              int chunk, void* ws0, void* ws1, size_t ws_bytes, void* stream) {
    if (check_T(T) || chunk < 1 || chunk > MOE_T_MAX) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !y || !ws0 || !ws1) return MOE_ERR_INVALID_ARG;
    if (int rc = check_layer(layer)) return rc;
    if (!a16(x) || !a16(y) || !a16(ws0) || !a16(ws1)) return MOE_ERR_ALIGN;
    const size_t need = ws_layout(chunk).total;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    {   // the two workspaces must not overlap
        const char *a = static_cast<const char*>(ws0), *b = static_cast<const char*>(ws1);
        if (a < b + need && b < a + need) return MOE_ERR_INVALID_ARG;
    }
    hipStream_t st = (hipStream_t)stream;
    const int nch = (T + chunk - 1) / chunk;
    void* ws[2] = {ws0, ws1};
    auto part = [&](int c, const uint16_t*& xc, uint16_t*& yc, int& tc) {
        xc = x + (size_t)c * chunk * H;
        yc = y + (size_t)c * chunk * H;
        tc = std::min(chunk, T - c * chunk);
    };
    if (nch == 1) {
        const WsLayout L = ws_layout(T);
        prefill_front(x, T, layer, ws0, L, at<int32_t>(ws0, L.ids), at<float>(ws0, L.wts),
                      at<float>(ws0, L.sg), st);
        prefill_back(x, T, layer, y, nullptr, ws0, L, at<float>(ws0, L.sg), st);
        return launch_status();
    }
    ChunkStreams* cs = chunk_streams();
    if (!cs) return MOE_ERR_HIP;
    // fork: the second stream starts after the caller's earlier work
    if (hipEventRecord(cs->fork, st) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamWaitEvent(cs->aux, cs->fork, 0) != hipSuccess) return MOE_ERR_HIP;
    auto front = [&](int c) -> bool {
        const uint16_t* xc; uint16_t* yc; int tc;
        part(c, xc, yc, tc);
        const int p = c & 1;
        // chunk c - 2's back half is done with this workspace
        if (c >= 2 && hipStreamWaitEvent(cs->aux, cs->done[p], 0) != hipSuccess) return false;
        const WsLayout L = ws_layout(tc);
        prefill_front(xc, tc, layer, ws[p], L, at<int32_t>(ws[p], L.ids), at<float>(ws[p], L.wts),
                      at<float>(ws[p], L.sg), cs->aux);
        return hipEventRecord(cs->routed[p], cs->aux) == hipSuccess;
    };
    auto back = [&](int c) -> bool {
        const uint16_t* xc; uint16_t* yc; int tc;
        part(c, xc, yc, tc);
        const int p = c & 1;
        if (hipStreamWaitEvent(st, cs->routed[p], 0) != hipSuccess) return false;
        const WsLayout L = ws_layout(tc);
        prefill_back(xc, tc, layer, yc, nullptr, ws[p], L, at<float>(ws[p], L.sg), st);
        return hipEventRecord(cs->done[p], st) == hipSuccess;
    };
    // the front of chunk c + 1 is queued before the back of chunk c, so the
    // second stream runs one chunk ahead; the last back half waits for the
    // last front half, which joins the second stream's work into the caller's
    if (!front(0)) return MOE_ERR_HIP;
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch && !front(c + 1)) return MOE_ERR_HIP;
        if (!back(c)) return MOE_ERR_HIP;
    }
    return launch_status();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The workspace of moe_chain_forward_noalloc: a fixed device array that the
// library owns (each GPU the library runs on holds its own copy until the
// process ends), for callers that cannot allocate.  In host code the array's
// name is only a stand-in for its device address; the address each device
// actually uses is taken once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WS_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's scratch address (NULL on a HIP error).
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int moe_chain_forward_noalloc(const uint16_t* x, int T, const moe_layer* layers, int nlayers,
                              uint16_t* x_out, uint16_t* y_layers, void* stream,
                              const moe_options* opt) {
    if (T < 0 || T > MOE_NOALLOC_T_MAX) return MOE_ERR_INVALID_ARG;
    static_assert(MOE_NOALLOC_WS_BYTES % 256 == 0, "scratch size");
    const size_t need = moe_workspace_bytes(T);
    if (need > MOE_NOALLOC_WS_BYTES) return MOE_ERR_WORKSPACE;   // (never, for T in range)
    if (T == 0 || nlayers == 0) return moe_chain_forward(x, T, layers, nlayers, x_out, y_layers,
                                                         nullptr, 0, stream, opt);
    void* ws = scratch_ptr();
    if (!ws) return MOE_ERR_HIP;
    return moe_chain_forward(x, T, layers, nlayers, x_out, y_layers, ws, MOE_NOALLOC_WS_BYTES,
                             stream, opt);
}

int moe_lm_head_argmax(const uint16_t* x, int T, const uint16_t* w_head, int V, int32_t* token,
                       void* ws, size_t ws_bytes, void* stream) {
    if (T < 1 || T > MOE_DECODE_T || V < 1) return MOE_ERR_INVALID_ARG;
    if (!x || !w_head || !token || !ws) return MOE_ERR_INVALID_ARG;
    if (!a16(x) || !a16(w_head) || !a4(token) || !a16(ws)) return MOE_ERR_ALIGN;
    const WsLayout L = ws_layout(T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    launch_head_argmax(x, T, w_head, V, token, at<unsigned long long>(ws, L.head),
                       (hipStream_t)stream);
    return launch_status();
}

int moe_embed(const int32_t* token, int T, const uint16_t* emb, int V, uint16_t* x, void* stream) {
    if (check_T(T) || V < 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!token || !emb || !x) return MOE_ERR_INVALID_ARG;
    if (!a4(token) || !a16(emb) || !a16(x)) return MOE_ERR_ALIGN;
    launch_embed(token, T, emb, V, x, (hipStream_t)stream);
    return launch_status();
}

int moe_router_transpose(const uint16_t* w_router, uint16_t* w_router_t, void* stream) {
    if (!w_router || !w_router_t) return MOE_ERR_INVALID_ARG;
    if (!a16(w_router) || !a16(w_router_t)) return MOE_ERR_ALIGN;
    launch_router_transpose(w_router, w_router_t, (hipStream_t)stream);
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
