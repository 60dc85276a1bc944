/*
 * moe.h -- C ABI of libmoe.so, the sparse mixture-of-experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer: every token is routed to 8 of 256 experts plus one shared
 * expert ("Perplexity Open-Sources Lily, a Qwen-Specific Mac Engine That
 * Beats MLX-LM in Its Test", section "A runtime shaped around one model").
 * Routing stays on the GPU with no host synchronisation, and 4-bit expert
 * weights are rebuilt inside the matrix products instead of being expanded
 * in memory (same page, section "The optimizations follow the workload";
 * "A Rust + Metal Inference Engine for Qwen3.6-35B-A3B on Apple Silicon",
 * paragraph 4).  Decode is a memory-bound sparse GEMV (leslieli.dev note on
 * the Lily engine, paragraph 5).
 *
 * Fixed layer format (the pages give no numbers; this is the library's
 * format):
 *   hidden H = 2048, expert width I = 512, E = 256 routed experts, top-8,
 *   one shared expert.
 *   x, y                 bf16 [T][2048], row-major
 *   w_router             bf16 [256][2048]
 *   router_bias          fp32 [256] or NULL (added to the logits)
 *   w_shared_gate        bf16 [2048]
 *   gate_q, up_q         uint32 [n][512][256]  eight 4-bit codes per word along
 *                        K, code k in bits 4*(k%8)..4*(k%8)+3 of word k/8
 *   down_q               uint32 [n][2048][64]
 *   gate_s/_b, up_s/_b   fp16 bits [n][512][32]  one scale and one bias per
 *   down_s/_b            fp16 bits [n][2048][8]  64-wide group along K
 *   weight               w(n,k) = code(n,k) * scale[n][k/64] + bias[n][k/64]
 *   n = 256 for the routed stack, 1 for the shared expert.
 *   SwiGLU:  h = bf16( silu(x Wg^T) * (x Wu^T) ),  d = h Wd^T
 *   routing: softmax over 256 logits, top-8 (ties -> lower expert index),
 *            weights renormalised to sum to 1; shared gate sigmoid(x . w_sg)
 *   output:  y = bf16( sum_j w_j d_j + sigmoid(x . w_sg) d_shared )
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers owned by the caller; the
 *     moe_layer / moe_qffn / moe_options structs are host memory, read
 *     during the call and not retained.
 *   - The library never allocates or frees memory and never synchronises:
 *     each call validates its arguments on the host and then only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   - x, y, weights, scales and the workspace must be 16-byte aligned.
 *   - On an error status nothing has been enqueued.  A launch failure is
 *     reported as MOE_ERR_HIP.
 *   - T == 0 is a no-op returning MOE_OK.  T may not exceed MOE_T_MAX.
 *   - The workspace (moe_workspace_bytes(T) bytes, caller owned) must be
 *     prepared once with moe_workspace_init (or be zero-filled) before its
 *     first use; every call leaves it ready for the next one.  Calls that
 *     share a workspace must be ordered on one stream; calls on different
 *     streams need different workspaces.  Everything is deterministic: the
 *     same inputs give bit-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_HIDDEN 2048
#define MOE_INTER 512
#define MOE_EXPERTS 256
#define MOE_TOPK 8
#define MOE_GROUP 64
#define MOE_T_MAX 65536
/* Decode path (dequantising GEMV) is the default for T <= MOE_DECODE_T;
 * it may be forced for T <= MOE_DECODE_T_MAX.  Larger T use the grouped
 * MFMA GEMM path, which can be forced for any T. */
#define MOE_DECODE_T 8
#define MOE_DECODE_T_MAX 32

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* NULL pointer, T out of range, bad option */
    MOE_ERR_ALIGN = 2,       /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 3,   /* ws_bytes below moe_workspace_bytes(T) */
    MOE_ERR_HIP = 4          /* a kernel launch failed */
} moe_status;

typedef enum {
    MOE_PATH_AUTO = 0,       /* decode for T <= MOE_DECODE_T, else prefill */
    MOE_PATH_DECODE = 1,     /* dequantising GEMV (T <= MOE_DECODE_T_MAX) */
    MOE_PATH_PREFILL = 2     /* grouped GEMM on fp16 MFMA */
} moe_path;

/* One quantised SwiGLU expert stack (see the format above).
 *
 * expert_stride: 0 = each of the nine arrays is dense, [n][rows][cols] as
 * above.  Otherwise it is the byte distance between expert e and expert
 * e + 1 in EVERY one of the nine arrays (a multiple of 256, at least
 * 524288 = one expert's code matrix), so that all of one expert's codes,
 * scales and biases can sit together in one block of memory; within an
 * expert each array keeps the row-major shape above (the library's
 * binding offers 2 MiB-aligned 2 MiB blocks per expert as an option).
 * Blocks must not overlap (not checked). */
typedef struct {
    const uint32_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b, *down_s, *down_b;
    int64_t expert_stride;
} moe_qffn;

/* One MoE layer: router, shared-expert gate, routed stack (n = 256) and
 * shared expert (n = 1). */
typedef struct {
    const uint16_t *w_router;
    const float *router_bias;       /* may be NULL */
    const uint16_t *w_shared_gate;
    moe_qffn routed;
    moe_qffn shared;
} moe_layer;

typedef struct {
    int path;                       /* moe_path */
    uint16_t *residual_out;         /* if non-NULL: also write bf16(x + y) here,
                                       bf16 [T][2048] (the chain's next input) */
    const void *prefetch;           /* if non-NULL: device bytes the call reads
                                       once and discards, to pull them toward
                                       the caches for a later call -- e.g. the
                                       next layer's router matrix in a decode
                                       chain (the next layer's first kernel
                                       then reads it from the memory-side
                                       cache).  Never written.  16-byte aligned;
                                       prefetch_bytes a multiple of 16, at most
                                       MOE_PREFETCH_MAX.  Read by the few-token
                                       (decode) layer path; other paths ignore
                                       it.  Prefetching the next layer's
                                       weights while this one runs is "fusing
                                       kernel chains" in "A Rust + Metal
                                       Inference Engine for Qwen3.6-35B-A3B on
                                       Apple Silicon", paragraph 5. */
    size_t prefetch_bytes;
} moe_options;

#define MOE_PREFETCH_MAX 2097152    /* bytes: one 16-byte load per thread of the
                                       decode down kernel (512 x 256) */

/* Workspace bytes sufficient for ANY call below with this T (monotone in T).
 * Returns 0 for T < 0 or T > MOE_T_MAX. */
size_t moe_workspace_bytes(int T);

/* Prepares a workspace for its first use (clears the library's
 * synchronisation words at its start; the rest is scratch).  Enqueues one
 * small fill kernel on `stream` (capturable in a graph).  ws_bytes must be
 * at least moe_workspace_bytes(0). */
int moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Human-readable name of a status code. */
const char *moe_status_string(int status);

/* Router (routing kept on the GPU: "Perplexity Open-Sources Lily ...",
 * section "The optimizations follow the workload").  For each token t:
 * logits l = x[t] W_r^T (+ router_bias), fp32 accumulation of exact bf16
 * products; topk_ids[t][0..7] = the 8 largest logits in descending order,
 * ties to the lower expert index; topk_w[t][j] = softmax(l)[id_j]
 * renormalised over the 8; shared_gate[t] = sigmoid(x[t] . w_shared_gate).
 * Outputs: topk_ids int32 [T][8], topk_w fp32 [T][8], shared_gate fp32 [T].
 * ws: workspace of moe_workspace_bytes(T) bytes. */
int moe_route(const uint16_t *x, int T, const uint16_t *w_router,
              const float *router_bias, const uint16_t *w_shared_gate,
              int32_t *topk_ids, float *topk_w, float *shared_gate,
              void *ws, size_t ws_bytes, void *stream);

/* Token -> expert permutation: a stable counting sort of the flat slots
 * f = 8t + j by expert id (histogram, exclusive scan, scatter; bit-exact).
 * expert_counts int32 [256]; expert_offsets int32 [257] (offsets[256] = 8T);
 * perm int32 [8T]: sorted position -> slot f (each expert's segment is in
 * ascending f); inv_perm int32 [8T]: slot f -> sorted position.  Ids outside
 * 0..255 are not counted or placed (their inv_perm entry is -1 and the
 * offsets then end below 8T). */
int moe_permute(const int32_t *topk_ids, int T, int32_t *expert_counts,
                int32_t *expert_offsets, int32_t *perm, int32_t *inv_perm,
                void *ws, size_t ws_bytes, void *stream);

/* Expert FFNs with the 4-bit weights dequantised inside the kernels.
 * expert_out fp32 [8T + T][2048]: row p < 8T is sorted position p (token
 * perm[p] / 8 through the expert whose offsets segment contains p), row
 * 8T + t is the shared expert on token t.  `opt` may be NULL. */
int moe_expert_ffn(const uint16_t *x, int T, const moe_qffn *routed,
                   const moe_qffn *shared, const int32_t *expert_offsets,
                   const int32_t *perm, float *expert_out, void *ws, size_t ws_bytes,
                   void *stream, const moe_options *opt);

/* Weighted un-permute plus the shared expert:
 * y[t] = bf16( sum_j topk_w[t][j] expert_out[inv_perm[8t+j]]
 *              + shared_gate[t] expert_out[8T+t] ),  fp32 accumulation. */
int moe_combine(const float *expert_out, const int32_t *inv_perm, const float *topk_w,
                const float *shared_gate, int T, uint16_t *y, void *stream);

/* The whole layer, route -> permute -> expert FFN -> combine, enqueued on
 * one stream with no host synchronisation.  y bf16 [T][2048]. */
int moe_layer_forward(const uint16_t *x, int T, const moe_layer *layer, uint16_t *y,
                      void *ws, size_t ws_bytes, void *stream);

/* As moe_layer_forward, with options (path override, residual output).
 * `opt` may be NULL. */
int moe_layer_forward_ex(const uint16_t *x, int T, const moe_layer *layer, uint16_t *y,
                         void *ws, size_t ws_bytes, void *stream, const moe_options *opt);

/* Measurement probes (the pages' method of quoting kernels against the
 * fastest sustained weight-read rate: leslieli.dev note on the Lily engine,
 * paragraph 5).  moe_probe_read streams `bytes` (a multiple of 16) from src
 * and writes one float per workgroup into sink (>= 4096 floats) so the
 * loads cannot be elided.  moe_probe_copy copies `bytes` (a multiple of 16)
 * from src to dst. */
int moe_probe_read(const void *src, size_t bytes, float *sink, void *stream);
int moe_probe_copy(void *dst, const void *src, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
