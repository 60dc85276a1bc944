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
 *   - The workspace (moe_workspace_bytes(T) bytes, caller owned) is
 *     scratch: no call reads anything a previous call left in it, so it
 *     needs no preparation.  Calls that share a workspace must be ordered on
 *     one stream; calls on different streams need different workspaces.
 *   - Everything is deterministic: the same inputs give bit-identical
 *     outputs.
 *   - Activations and the SwiGLU intermediate h are carried as fp16 inside
 *     the expert kernels (bf16 -> fp16 is exact for magnitudes in
 *     [2^-14, 65504]; smaller ones keep fp16's subnormal spacing 2^-24).
 *     Inputs are expected to keep |x| and |h| below 65504; a token whose x
 *     or h leaves that range gets a non-finite output row (other tokens are
 *     unaffected).  Routing is computed from the bf16 x in fp32 and is not
 *     affected.
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
 * 524288 = one expert's code matrix, at most 2^31), so that all of one
 * expert's codes, scales and biases can sit together in one block of memory
 * (fewer distinct pages touched per active expert; the library's binding
 * offers 2 MiB-aligned 2 MiB blocks per expert as an option); within an
 * expert each array keeps the row-major shape above.  Blocks must not
 * overlap (not checked); anything else returns MOE_ERR_INVALID_ARG. */
typedef struct {
    const uint32_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b, *down_s, *down_b;
    int64_t expert_stride;
} moe_qffn;

/* One MoE layer: router, shared-expert gate, routed stack (n = 256) and
 * shared expert (n = 1).  w_router_t (optional, may be NULL): the same
 * router matrix transposed, bf16 [2048][256] (see moe_router_transpose);
 * a chain's few-token path fuses a layer into the one before it only when
 * the layer has it (otherwise that layer runs its own router kernel). */
typedef struct {
    const uint16_t *w_router;
    const float *router_bias;       /* may be NULL */
    const uint16_t *w_shared_gate;
    moe_qffn routed;
    moe_qffn shared;
    const uint16_t *w_router_t;     /* may be NULL */
} moe_layer;

typedef struct {
    int path;                       /* moe_path */
    uint16_t *residual_out;         /* if non-NULL: also write bf16(x + y) here,
                                       bf16 [T][2048] (layer calls only; a
                                       chain call rejects it) */
    int32_t *route_ids;             /* route outputs, all three or none: the
                                       routing the call used -- ids int32
                                       [T][8] in selection order, weights fp32
                                       [T][8], shared gate fp32 [T] (chain
                                       calls: [nlayers][...], layer by layer);
                                       4-byte aligned device memory */
    float *route_w;
    float *route_sg;
} moe_options;

/* Workspace bytes sufficient for ANY call below with this T (monotone in T).
 * Returns 0 for T < 0 or T > MOE_T_MAX. */
size_t moe_workspace_bytes(int T);

/* Human-readable name of a status code. */
const char *moe_status_string(int status);

/* Router.  Every token goes to 8 of the 256 experts plus the shared expert
 * ("Perplexity Open-Sources Lily ...", section "A runtime shaped around one
 * model"), and the routing stays on the GPU with no host synchronisation
 * (same page, section "The optimizations follow the workload").  For each
 * token t: logits l = x[t] W_r^T (+ router_bias), fp32 accumulation of
 * exact bf16 products; topk_ids[t][0..7] = the 8 largest logits in
 * descending order, ties to the lower expert index; topk_w[t][j] =
 * softmax(l)[id_j] renormalised over the 8; shared_gate[t] =
 * sigmoid(x[t] . w_shared_gate).
 * In: x bf16 [T][2048], w_router bf16 [256][2048], router_bias fp32 [256] or
 * NULL, w_shared_gate bf16 [2048] (16-byte aligned except router_bias: 4).
 * Out: topk_ids int32 [T][8], topk_w fp32 [T][8], shared_gate fp32 [T].
 * ws: workspace of moe_workspace_bytes(T) bytes.
 * Errors: NULL pointer or T out of range -> MOE_ERR_INVALID_ARG; alignment
 * -> MOE_ERR_ALIGN; ws_bytes too small -> MOE_ERR_WORKSPACE. */
int moe_route(const uint16_t *x, int T, const uint16_t *w_router,
              const float *router_bias, const uint16_t *w_shared_gate,
              int32_t *topk_ids, float *topk_w, float *shared_gate,
              void *ws, size_t ws_bytes, void *stream);

/* Token -> expert permutation, the step that turns the routing into the
 * per-expert row groups of the grouped matrix products ("Perplexity
 * Open-Sources Lily ...", section "The optimizations follow the workload":
 * routing and the grouped products stay on the GPU).  A stable counting
 * sort of the flat slots f = 8t + j by expert id (histogram, exclusive scan,
 * scatter; bit-exact).
 * In: topk_ids int32 [T][8].  Out: expert_counts int32 [256];
 * expert_offsets int32 [257] (offsets[256] = 8T); perm int32 [8T]: sorted
 * position -> slot f (each expert's segment is in ascending f); inv_perm
 * int32 [8T]: slot f -> sorted position.  Ids outside 0..255 are not counted
 * or placed (their inv_perm entry is -1 and the offsets then end below 8T).
 * All arrays 4-byte aligned; ws as for moe_route.  Errors as for moe_route. */
int moe_permute(const int32_t *topk_ids, int T, int32_t *expert_counts,
                int32_t *expert_offsets, int32_t *perm, int32_t *inv_perm,
                void *ws, size_t ws_bytes, void *stream);

/* Expert FFNs with the 4-bit weights rebuilt inside the kernels rather than
 * expanded in memory ("Perplexity Open-Sources Lily ...", section "The
 * optimizations follow the workload"; "A Rust + Metal Inference Engine for
 * Qwen3.6-35B-A3B on Apple Silicon", paragraph 4).  For routed row p < 8T
 * (sorted position p: token perm[p] / 8 through the expert whose
 * expert_offsets segment contains p) and shared row 8T + t (the shared
 * expert on token t): expert_out[row] = Wd (bf16(silu(Wg x) * (Wu x))).
 * In: x bf16 [T][2048]; routed (n = 256) and shared (n = 1) stacks;
 * expert_offsets int32 [257] and perm int32 [8T] as from moe_permute.
 * Out: expert_out fp32 [9T][2048] (16-byte aligned).  opt may be NULL (only
 * opt->path is read: decode GEMVs up to MOE_DECODE_T_MAX tokens, else the
 * grouped MFMA GEMM).  Errors as for moe_route, plus MOE_ERR_INVALID_ARG for
 * a bad expert_stride or path. */
int moe_expert_ffn(const uint16_t *x, int T, const moe_qffn *routed,
                   const moe_qffn *shared, const int32_t *expert_offsets,
                   const int32_t *perm, float *expert_out, void *ws, size_t ws_bytes,
                   void *stream, const moe_options *opt);

/* Weighted un-permute plus the sigmoid-gated shared expert (the layer's
 * output: the 8 routed experts plus the shared expert, "Perplexity
 * Open-Sources Lily ...", section "A runtime shaped around one model"):
 * y[t] = bf16( sum_j topk_w[t][j] expert_out[inv_perm[8t+j]]
 *              + shared_gate[t] expert_out[8T+t] ),  fp32 accumulation in
 * that order.  In: expert_out fp32 [9T][2048] (16-byte aligned), inv_perm
 * int32 [8T] (entries outside 0..8T-1 are skipped), topk_w fp32 [T][8],
 * shared_gate fp32 [T].  Out: y bf16 [T][2048] (16-byte aligned).  Needs no
 * workspace.  Errors: NULL / T -> MOE_ERR_INVALID_ARG, alignment ->
 * MOE_ERR_ALIGN. */
int moe_combine(const float *expert_out, const int32_t *inv_perm, const float *topk_w,
                const float *shared_gate, int T, uint16_t *y, void *stream);

/* The whole layer -- route, permute, expert FFN, combine -- enqueued on one
 * stream with no host synchronisation (routing kept on the GPU:
 * "Perplexity Open-Sources Lily ...", section "The optimizations follow the
 * workload"; kernel chains fused: "A Rust + Metal Inference Engine for
 * Qwen3.6-35B-A3B on Apple Silicon", paragraph 5).  In: x bf16 [T][2048].
 * Out: y bf16 [T][2048].  Up to MOE_DECODE_T tokens run the few-token path
 * (three kernels), more the grouped-GEMM path.  Errors as for moe_route. */
int moe_layer_forward(const uint16_t *x, int T, const moe_layer *layer, uint16_t *y,
                      void *ws, size_t ws_bytes, void *stream);

/* As moe_layer_forward, with options: path override, residual output
 * (bf16(x + y)), route outputs.  opt may be NULL. */
int moe_layer_forward_ex(const uint16_t *x, int T, const moe_layer *layer, uint16_t *y,
                         void *ws, size_t ws_bytes, void *stream, const moe_options *opt);

/* A long prompt through one layer in chunks of `chunk` tokens, pipelined:
 * the routing and permutation of chunk c+1 run while the expert GEMMs and
 * the combine of chunk c run.  Long prompts are processed in chunks
 * (leslieli.dev note on the Lily engine, paragraph 3), and the runtime
 * keeps uneven expert workloads moving ("Perplexity Open-Sources Lily ...",
 * section "A runtime shaped around one model").
 * In: x bf16 [T][2048], 1 <= T <= MOE_T_MAX; 1 <= chunk <= MOE_T_MAX.
 * Out: y bf16 [T][2048].  ws0, ws1: two non-overlapping workspaces of
 * ws_bytes >= moe_workspace_bytes(chunk) bytes each; x, y, ws0, ws1 16-byte
 * aligned.  Every chunk takes the grouped-GEMM path whatever its size, and
 * y equals, bit for bit, moe_layer_forward_ex on each chunk in turn with
 * path MOE_PATH_PREFILL.
 * Streams: the front half of each chunk (router GEMM, top-8, permutation)
 * runs on a second stream the library owns (one per device, default
 * priority, created with its events on the first chunked call on that
 * device -- that first call must not be made under stream capture), the
 * back half (grouped GEMMs, combine) on `stream`; events order the two, the
 * second stream's work starts after `stream`'s earlier work and ends before
 * the call's last work on `stream`, so the call can be captured into a HIP
 * graph on `stream` like any other.  Two calls on one device must not
 * overlap (they share the second stream's events).  A single chunk
 * (T <= chunk) runs on `stream` alone.
 * Errors: NULL / T / chunk / overlapping workspaces -> MOE_ERR_INVALID_ARG;
 * alignment -> MOE_ERR_ALIGN; small workspaces -> MOE_ERR_WORKSPACE;
 * stream or event creation -> MOE_ERR_HIP. */
int moe_layer_forward_chunked(const uint16_t *x, int T, const moe_layer *layer, uint16_t *y,
                              int chunk, void *ws0, void *ws1, size_t ws_bytes, void *stream);

/* A chain of layers with residual adds: x_0 = x, y_l = layer_l(x_l),
 * x_{l+1} = bf16(x_l + y_l); x_out = x_nlayers.  The fused kernel chain of
 * decode ("A Rust + Metal Inference Engine for Qwen3.6-35B-A3B on Apple
 * Silicon", paragraph 5): on the few-token path every layer after the first
 * is two kernels, because each layer's down kernel also forms the next
 * layer's router logits and fp16 input (deterministically: fixed-point
 * integer sums).  More tokens run one grouped-GEMM layer after another.
 * In: x bf16 [T][2048]; layers[nlayers] (host array of descriptors, read
 * during the call).  Out: x_out bf16 [T][2048]; y_layers: optional bf16
 * [nlayers][T][2048], each layer's y.  opt: path override and route outputs
 * (per layer); residual_out must be NULL.  All buffers 16-byte aligned;
 * ws: moe_workspace_bytes(T) bytes (it also holds the intermediate x_l).
 * Errors as for moe_layer_forward_ex; nlayers == 0 or T == 0 is a no-op. */
int moe_chain_forward(const uint16_t *x, int T, const moe_layer *layers, int nlayers,
                      uint16_t *x_out, uint16_t *y_layers, void *ws, size_t ws_bytes,
                      void *stream, const moe_options *opt);

/* Greedy next-token selection after the last layer, kept on the GPU for
 * the next decode step ("Perplexity Open-Sources Lily ...", section
 * "Generation has a different bottleneck").  The pages give no output head;
 * the library's: a bf16 head w_head [V][2048] applied to the bf16 hidden
 * state, logit[t][v] = x[t] . w_head[v] with fp32 accumulation of exact
 * bf16 products, token[t] = argmax_v logit[t][v], ties to the lower v.
 * In: x bf16 [T][2048], 1 <= T <= MOE_DECODE_T; w_head bf16 [V][2048],
 * 1 <= V < 2^31 (16-byte aligned).  Out: token int32 [T] (device memory, 4-byte
 * aligned).  ws: moe_workspace_bytes(T) bytes.  Errors: NULL, T or V out of
 * range -> MOE_ERR_INVALID_ARG; alignment -> MOE_ERR_ALIGN; ws too small ->
 * MOE_ERR_WORKSPACE. */
int moe_lm_head_argmax(const uint16_t *x, int T, const uint16_t *w_head, int V, int32_t *token,
                       void *ws, size_t ws_bytes, void *stream);

/* The next decode step's input rows from the selected tokens, read on the
 * device: x[t] = emb[token[t]] (a row of zeros for a token outside 0..V-1).
 * In: token int32 [T] (device), emb bf16 [V][2048] (16-byte aligned).  Out:
 * x bf16 [T][2048].  T in 0..MOE_T_MAX (0: no-op).  Errors: NULL or a size
 * out of range -> MOE_ERR_INVALID_ARG; alignment -> MOE_ERR_ALIGN. */
int moe_embed(const int32_t *token, int T, const uint16_t *emb, int V, uint16_t *x, void *stream);

/* Gated delta rule scan: the recurrent (Gated DeltaNet) layers of the
 * model, whose scan the engine keeps in registers ("leslieli.dev note on
 * the Perplexity Lily engine", paragraph 3; "Perplexity Open-Sources Lily
 * ...", section "A runtime shaped around one model").  The pages do not
 * define the recurrence; this is the published gated delta rule (Yang,
 * Kautz, Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta
 * Rule").  Per value head h (key head h / (hv / hk)) with state S (128 x
 * 128, rows = value channels, columns = key channels):
 *   S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   o_t = S_t q_t.
 * q and k are used as given (any normalisation or scaling of them is the
 * caller's).  Calls of up to MOE_GDN_STEP_T_MAX tokens (decode) run the
 * recurrence token by token in fp32 with the state in registers (the
 * workspace is then not used); longer ones are computed in chunks of
 * MOE_GDN_CHUNK tokens on fp16 MFMA with fp32 accumulation and an fp32
 * state (fp16 operands: see the library's documentation for the error this
 * gives).
 * In: q, k bf16 [T][hk][128]; v bf16 [T][hv][128] (16-byte aligned);
 * g (log decay) and beta fp32 [T][hv]; s0 fp32 [hv][128][128], the state
 * entering token 0, or NULL for zero.  Out: o bf16 [T][hv][128] (rounded
 * to nearest even); s_out fp32 [hv][128][128], the state after token T-1,
 * or NULL; it may be s0 itself (the state updated in place, as a decode
 * loop does).  ws: moe_gdn_workspace_bytes(T, hv) bytes of device scratch,
 * 256-byte aligned, not read before it is written.  1 <= hk, hv <=
 * MOE_GDN_HEADS_MAX, hv a multiple of hk, 0 <= T <= MOE_T_MAX (T == 0:
 * s_out, if given, receives s0 or zeros).  Errors: NULL or a size out of
 * range -> MOE_ERR_INVALID_ARG; alignment -> MOE_ERR_ALIGN; ws too small
 * -> MOE_ERR_WORKSPACE.  Deterministic. */
#define MOE_GDN_DIM 128
#define MOE_GDN_CHUNK 64
#define MOE_GDN_STEP_T_MAX 48
#define MOE_GDN_HEADS_MAX 64
size_t moe_gdn_workspace_bytes(int T, int hv);   /* 0 for arguments out of range */
int moe_gdn_scan(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                 const float *beta, int T, int hk, int hv, const float *s0, uint16_t *o,
                 float *s_out, void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as moe_chain_forward with the workspace taken from a fixed device
 * array the library owns (MOE_NOALLOC_WS_BYTES per GPU, held until the
 * process ends), for up to MOE_NOALLOC_T_MAX tokens; larger T returns
 * MOE_ERR_INVALID_ARG.  No allocation or free happens in the call.  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or different host threads without ordering)
 * race and must not be made; calls ordered on one stream are fine.  Nothing
 * in the array needs clearing between calls.  Other arguments, outputs and
 * errors as for moe_chain_forward; a HIP error while locating the array
 * returns MOE_ERR_HIP. */
#define MOE_NOALLOC_T_MAX 64
#define MOE_NOALLOC_WS_BYTES 8388608
int moe_chain_forward_noalloc(const uint16_t *x, int T, const moe_layer *layers, int nlayers,
                              uint16_t *x_out, uint16_t *y_layers, void *stream,
                              const moe_options *opt);

/* w_router_t[k][e] = w_router[e][k]: the transposed router matrix a
 * chained layer's predecessor reads (rows k of it are the router entries
 * for hidden unit k, so a down kernel holding hidden units m0..m0+3 of the
 * layer's input reads four contiguous 512-byte rows).  In: w_router bf16
 * [256][2048]; out: w_router_t bf16 [2048][256]; both 16-byte aligned device
 * memory, not overlapping.  Enqueues one kernel on stream.  Errors: NULL ->
 * MOE_ERR_INVALID_ARG, alignment -> MOE_ERR_ALIGN. */
int moe_router_transpose(const uint16_t *w_router, uint16_t *w_router_t, void *stream);

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
