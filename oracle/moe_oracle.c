/*
 * moe_oracle.c -- plain CPU reference of the sparse mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * What it computes (structure from the pages, numbers from this library's
 * fixed layer format):
 *   - each token goes to 8 of 256 routed experts plus one shared expert
 *     ("Perplexity Open-Sources Lily, a Qwen-Specific Mac Engine ...",
 *     section "A runtime shaped around one model");
 *   - expert weights are 4-bit codes rebuilt into real weights inside the
 *     matrix product rather than expanded in memory (same page, section
 *     "The optimizations follow the workload"; "A Rust + Metal Inference
 *     Engine for Qwen3.6-35B-A3B on Apple Silicon", paragraph 4);
 *   - routing (router product, softmax, top-8, renormalisation) is part of
 *     the layer (same section of the first page cited).
 *
 * Readings taken where the pages are silent (the numeric layer format):
 *   code(n,k) = (Q[n][k/8] >> 4*(k%8)) & 15   (least significant nibble first)
 *   w(n,k)    = code * scale[n][k/G] + bias[n][k/G]   (fp16 scale and bias)
 *   l[t,e]    = x[t] . W_r[e]  (+ b_e when a router bias is given)
 *   top-8 selected on the fp32-rounded logits, descending, ties -> lower e
 *   p         = softmax over all E logits; w_j = p[id_j] / sum_j p[id_j]
 *   sg[t]     = sigmoid(x[t] . w_sg)
 *   h[n]      = bf16( silu(g[n]) * u[n] ),  g = x.Wg^T, u = x.Wu^T
 *   d[m]      = h . Wd[m]
 *   y[t]      = bf16( sum_j w_j d_{id_j} + sg * d_shared )
 * Everything else is evaluated in IEEE double; dot products accumulate in
 * ascending index order, so the result does not depend on threading.
 *
 * A compile-time ORACLE_MUTANT=<n> plants one known mistake; the test suite
 * uses such builds to show that its pins catch each of them.  The default
 * build (ORACLE_MUTANT undefined) is the oracle.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUT(n) (ORACLE_MUTANT == (n))

typedef struct {
    int E;     /* routed experts */
    int topk;  /* experts selected per token */
    int H;     /* hidden size (K of gate/up, N of down) */
    int I;     /* expert width (N of gate/up, K of down) */
    int G;     /* quantisation group length along K */
} oracle_dims;

typedef struct {
    const uint32_t *gate_q, *up_q, *down_q;                 /* code words */
    const uint16_t *gate_s, *gate_b, *up_s, *up_b,          /* fp16 bits */
                   *down_s, *down_b;
} oracle_qffn;

int oracle_mutant(void) { return ORACLE_MUTANT; }

/* Threads the OpenMP loops use (reported with the CPU baseline). */
int oracle_threads(void) { return omp_get_max_threads(); }

/* Sets the thread count of the OpenMP loops that follow (n >= 1); for timing
 * the same code on one core and on all of them.  No effect on the results:
 * every loop writes disjoint outputs. */
void oracle_set_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }

/* ---------------------------------------------------------------- formats */

/* bf16 is the upper half of an IEEE binary32 word. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_fp16_to_double(uint16_t h)
{
    int sign = h >> 15, ex = (h >> 10) & 0x1F, man = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), ex - 25);   /* (1024+man) * 2^(ex-25) */
    return sign ? -v : v;
}

/* Round a double to the nearest bf16 (ties to even), directly from double:
 * 8 significant bits, exponent range of binary32. */
uint16_t oracle_double_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v))
        return sign | 0x7FC0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);             /* a lies in [2^(e-1), 2^e) */
    int q = e - 8;                  /* quantum of an 8-significant-bit value */
    if (q < -133)
        q = -133;                   /* bf16 subnormal quantum */
#if ORACLE_MUTANT == 13
    double r = round(ldexp(a, -q));       /* ties away from zero */
#else
    double r = nearbyint(ldexp(a, -q));   /* default mode: ties to even */
#endif
    double rv = ldexp(r, q);
    if (rv > 0x1.FEp127)            /* above the largest finite bf16 */
        return sign | 0x7F80;
    float f = (float)rv;            /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

void oracle_round_bf16_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_bf16(in[i]);
}

void oracle_fp16_decode_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_fp16_to_double(in[i]);
}

void oracle_bf16_decode_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_double(in[i]);
}

/* --------------------------------------------------------- dequantisation */

static int code_at(const uint32_t *wordrow, int k)
{
#if ORACLE_MUTANT == 1
    return (wordrow[k / 8] >> (4 * (7 - k % 8))) & 0xF;     /* nibble order reversed */
#else
    return (wordrow[k / 8] >> (4 * (k % 8))) & 0xF;
#endif
}

/* Real weight w(row, k) of a [rows][K] quantised matrix.  `row` already
 * includes the expert offset (e * rows_per_expert + n). */
double oracle_dequant(const uint32_t *q, const uint16_t *s, const uint16_t *b,
                      int64_t row, int K, int G, int k)
{
    const uint32_t *wordrow = q + row * (K / 8);
    double sc = oracle_fp16_to_double(s[row * (K / G) + k / G]);
    double bi = oracle_fp16_to_double(b[row * (K / G) + k / G]);
#if ORACLE_MUTANT == 2
    bi = 0.0;                                               /* bias dropped */
#endif
    return code_at(wordrow, k) * sc + bi;
}

/* Dot product of a real vector with one quantised row, ascending k.  The
 * group's scale and bias are decoded once per group (same values as
 * oracle_dequant). */
static double qrow_dot(const uint32_t *q, const uint16_t *s, const uint16_t *b,
                       int64_t row, int K, int G, const double *v)
{
    const uint32_t *wordrow = q + row * (K / 8);
    double acc = 0.0;
    for (int g = 0; g < K / G; ++g) {
#if ORACLE_MUTANT == 3
        int gi = (g + 1) % (K / G);                         /* wrong group's scale */
#else
        int gi = g;
#endif
        double sc = oracle_fp16_to_double(s[row * (K / G) + gi]);
        double bi = oracle_fp16_to_double(b[row * (K / G) + gi]);
#if ORACLE_MUTANT == 2
        bi = 0.0;
#endif
        for (int k = g * G; k < (g + 1) * G; ++k)
            acc += v[k] * (code_at(wordrow, k) * sc + bi);
    }
    return acc;
}

/* ---------------------------------------------------------------- routing */

/* Router for T tokens.  x: bf16 [T][H]; w_router: bf16 [E][H]; router_bias:
 * fp32 [E] or NULL; w_sg: bf16 [H].  If forced_ids is non-NULL ([T][topk])
 * those experts are used instead of the top-k selection (weights are still
 * the softmax renormalised over the given set).
 * Outputs: ids [T][topk], w [T][topk], sg [T]; optional logits [T][E] and
 * gap [T] = (topk-th largest logit) - (largest unselected logit). */
int oracle_route(const oracle_dims *d, int T, const uint16_t *x,
                 const uint16_t *w_router, const float *router_bias,
                 const uint16_t *w_sg, const int32_t *forced_ids,
                 int32_t *ids, double *w, double *sg,
                 double *logits, double *gap)
{
    const int E = d->E, H = d->H, K = d->topk;
    if (T < 0 || E <= 0 || K <= 0 || K > E)
        return 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int t = 0; t < T; ++t) {
        double *l = malloc(sizeof(double) * E);
        float *l32 = malloc(sizeof(float) * E);
        char *taken = calloc(E, 1);
        double *xv = malloc(sizeof(double) * H);
        if (!l || !l32 || !taken || !xv) { bad = 1; free(l); free(l32); free(taken); free(xv); continue; }
        for (int k = 0; k < H; ++k)
            xv[k] = oracle_bf16_to_double(x[(int64_t)t * H + k]);
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int k = 0; k < H; ++k)
                acc += xv[k] * oracle_bf16_to_double(w_router[(int64_t)e * H + k]);
            if (router_bias)
                acc += (double)router_bias[e];
            l[e] = acc;
            l32[e] = (float)acc;
            if (logits)
                logits[(int64_t)t * E + e] = acc;
        }
        int32_t *tid = ids + (int64_t)t * K;
        if (forced_ids) {
            for (int j = 0; j < K; ++j) {
                int e = forced_ids[(int64_t)t * K + j];
                if (e < 0 || e >= E || taken[e]) { bad = 1; e = 0; }
                tid[j] = e;
                taken[e] = 1;
            }
        } else {
            /* top-k: repeatedly take the largest remaining fp32 logit,
             * the lower expert index winning a tie */
            for (int j = 0; j < K; ++j) {
                int best = -1;
                for (int e = 0; e < E; ++e) {
                    if (taken[e])
                        continue;
#if ORACLE_MUTANT == 4
                    if (best < 0 || l32[e] >= l32[best])             /* tie -> higher index */
#elif ORACLE_MUTANT == 5
                    if (best < 0 || l32[e] < l32[best])              /* smallest logits */
#else
                    if (best < 0 || l32[e] > l32[best])
#endif
                        best = e;
                }
                tid[j] = best;
                taken[best] = 1;
            }
        }
        if (gap) {
            double lk = l[tid[K - 1]], lmax_rest = -INFINITY;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && l[e] > lmax_rest)
                    lmax_rest = l[e];
            gap[t] = lk - lmax_rest;
        }
        /* softmax over all E experts, then renormalise over the selected */
        double m = -INFINITY;
        for (int e = 0; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double den = 0.0;
        for (int e = 0; e < E; ++e)
            den += exp(l[e] - m);
        double psel = 0.0;
        for (int j = 0; j < K; ++j)
            psel += exp(l[tid[j]] - m) / den;
        for (int j = 0; j < K; ++j) {
            double p = exp(l[tid[j]] - m) / den;
#if ORACLE_MUTANT == 6
            w[(int64_t)t * K + j] = p;                           /* not renormalised */
#else
            w[(int64_t)t * K + j] = p / psel;
#endif
        }
        /* sigmoid-gated shared expert */
        double z = 0.0;
        for (int k = 0; k < H; ++k)
            z += xv[k] * oracle_bf16_to_double(w_sg[k]);
#if ORACLE_MUTANT == 7
        sg[t] = 1.0 / (1.0 + exp(z));                            /* sign flipped */
#else
        sg[t] = 1.0 / (1.0 + exp(-z));
#endif
        free(l); free(l32); free(taken); free(xv);
    }
    return bad ? 2 : 0;
}

/* ------------------------------------------------------------ permutation */

/* Stable counting sort of the flat slots f = t*topk + j by expert id.
 * counts [E], offsets [E+1], perm [T*topk] (sorted position -> slot),
 * inv [T*topk] (slot -> sorted position).  Returns nonzero on an id
 * outside 0..E-1. */
int oracle_permute(const oracle_dims *d, int T, const int32_t *ids,
                   int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv)
{
    const int E = d->E;
    const int64_t n = (int64_t)T * d->topk;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t f = 0; f < n; ++f) {
        if (ids[f] < 0 || ids[f] >= E)
            return 1;
        counts[ids[f]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = malloc(sizeof(int32_t) * (E > 0 ? E : 1));
    if (!cursor)
        return 2;
    for (int e = 0; e < E; ++e)
        cursor[e] = 0;
#if ORACLE_MUTANT == 8
    for (int64_t f = n - 1; f >= 0; --f) {                      /* unstable order */
#else
    for (int64_t f = 0; f < n; ++f) {
#endif
        int e = ids[f];
        int32_t p = offsets[e] + cursor[e]++;
        perm[p] = (int32_t)f;
        inv[f] = p;
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------ expert FFN */

/* One SwiGLU expert on one token: out[H] = Wd ( bf16( silu(Wg x) * (Wu x) ) ).
 * h_bits (optional, [I]) receives the bf16 intermediate. */
static void ffn_row(const oracle_dims *d, const oracle_qffn *q, int e,
                    const double *xv, double *hv, double *out, uint16_t *h_bits)
{
    const int H = d->H, I = d->I, G = d->G;
    for (int n = 0; n < I; ++n) {
        int64_t row = (int64_t)e * I + n;
        double g = qrow_dot(q->gate_q, q->gate_s, q->gate_b, row, H, G, xv);
        double u = qrow_dot(q->up_q, q->up_s, q->up_b, row, H, G, xv);
#if ORACLE_MUTANT == 9
        double a = g / (1.0 + exp(g));                          /* silu sign wrong */
#else
        double a = g / (1.0 + exp(-g));
#endif
#if ORACLE_MUTANT == 10
        double hval = a * u;                                    /* no bf16 rounding */
        uint16_t hb = oracle_double_to_bf16(hval);
#else
        uint16_t hb = oracle_double_to_bf16(a * u);
        double hval = oracle_bf16_to_double(hb);
#endif
        hv[n] = hval;
        if (h_bits)
            h_bits[n] = hb;
    }
    for (int m = 0; m < H; ++m) {
#if ORACLE_MUTANT == 11
        int64_t row = (int64_t)e * H + (H - 1 - m);             /* rows reversed */
#else
        int64_t row = (int64_t)e * H + m;
#endif
        out[m] = qrow_dot(q->down_q, q->down_s, q->down_b, row, I, G, hv);
    }
}

/* Expert outputs for the permuted routed rows and the shared rows.
 * out: [(topk*T + T)][H]; row p < topk*T is sorted position p (token
 * perm[p]/topk, expert = the segment of offsets containing p); row
 * topk*T + t is the shared expert on token t.  If rows != NULL only the
 * nrows listed rows are computed, into out[i][H] for the i-th listed row.
 * h_bits (optional) mirrors out's row indexing with [I] bf16 per row. */
int oracle_expert_ffn(const oracle_dims *d, int T, const uint16_t *x,
                      const oracle_qffn *routed, const oracle_qffn *shared,
                      const int32_t *offsets, const int32_t *perm,
                      const int32_t *rows, int nrows, double *out, uint16_t *h_bits)
{
    const int H = d->H, I = d->I, K = d->topk, E = d->E;
    const int64_t nr = (int64_t)K * T;
    const int64_t total = rows ? nrows : nr + T;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t i = 0; i < total; ++i) {
        int64_t p = rows ? rows[i] : i;
        double *xv = malloc(sizeof(double) * H);
        double *hv = malloc(sizeof(double) * I);
        if (!xv || !hv || p < 0 || p >= nr + T) { bad = 1; free(xv); free(hv); continue; }
        int t, e;
        const oracle_qffn *q;
        if (p < nr) {
            t = perm[p] / K;
            e = 0;
            while (e < E && !(offsets[e] <= p && p < offsets[e + 1]))
                ++e;
            if (e == E || t < 0 || t >= T) { bad = 1; free(xv); free(hv); continue; }
            q = routed;
        } else {
            t = (int)(p - nr);
            e = 0;
            q = shared;
        }
        for (int k = 0; k < H; ++k)
            xv[k] = oracle_bf16_to_double(x[(int64_t)t * H + k]);
        ffn_row(d, q, e, xv, hv, out + i * H, h_bits ? h_bits + i * I : NULL);
        free(xv); free(hv);
    }
    return bad ? 1 : 0;
}

/* ---------------------------------------------------------------- combine */

/* y[t] = bf16( sum_j w[t][j] * out[inv[t*topk+j]] + sg[t] * out[topk*T+t] ).
 * y32 (optional) receives the unrounded sum. */
int oracle_combine(const oracle_dims *d, int T, const double *out, const int32_t *inv,
                   const double *w, const double *sg, uint16_t *y, double *y32)
{
    const int H = d->H, K = d->topk;
    const int64_t nr = (int64_t)K * T;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j) {
#if ORACLE_MUTANT == 14
                int64_t slot = (int64_t)j * T + t;                  /* transposed slot index */
                if (slot >= (int64_t)K * T) slot = (int64_t)t * K + j;
#else
                int64_t slot = (int64_t)t * K + j;
#endif
                acc += w[(int64_t)t * K + j] * out[(int64_t)inv[slot] * H + m];
            }
#if ORACLE_MUTANT != 12
            acc += sg[t] * out[(nr + t) * H + m];               /* mutant 12 drops it */
#endif
            if (y32)
                y32[(int64_t)t * H + m] = acc;
            y[(int64_t)t * H + m] = oracle_double_to_bf16(acc);
        }
    }
    return 0;
}

/* ------------------------------------------------------------ whole layer */

/* route -> permute -> expert FFN -> combine.  Optional outputs: ids, w, sg,
 * gap (per token) and y32.  forced_ids as in oracle_route. */
int oracle_layer_forward(const oracle_dims *d, int T, const uint16_t *x,
                         const uint16_t *w_router, const float *router_bias,
                         const uint16_t *w_sg, const oracle_qffn *routed,
                         const oracle_qffn *shared, const int32_t *forced_ids,
                         uint16_t *y, int32_t *ids_out, double *w_out, double *sg_out,
                         double *gap_out, double *y32)
{
    const int K = d->topk, E = d->E, H = d->H;
    const int64_t nr = (int64_t)K * T;
    if (T == 0)
        return 0;
    int32_t *ids = malloc(sizeof(int32_t) * nr);
    double *w = malloc(sizeof(double) * nr);
    double *sg = malloc(sizeof(double) * T);
    int32_t *counts = malloc(sizeof(int32_t) * E);
    int32_t *offsets = malloc(sizeof(int32_t) * (E + 1));
    int32_t *perm = malloc(sizeof(int32_t) * nr);
    int32_t *inv = malloc(sizeof(int32_t) * nr);
    double *out = malloc(sizeof(double) * (nr + T) * H);
    int rc = 3;
    if (ids && w && sg && counts && offsets && perm && inv && out) {
        rc = oracle_route(d, T, x, w_router, router_bias, w_sg, forced_ids, ids, w, sg,
                          NULL, gap_out);
        if (!rc)
            rc = oracle_permute(d, T, ids, counts, offsets, perm, inv);
        if (!rc)
            rc = oracle_expert_ffn(d, T, x, routed, shared, offsets, perm, NULL, 0, out, NULL);
        if (!rc)
            rc = oracle_combine(d, T, out, inv, w, sg, y, y32);
        if (!rc) {
            if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * nr);
            if (w_out) memcpy(w_out, w, sizeof(double) * nr);
            if (sg_out) memcpy(sg_out, sg, sizeof(double) * T);
        }
    }
    free(ids); free(w); free(sg); free(counts); free(offsets); free(perm); free(inv); free(out);
    return rc;
}

/* ------------------------------------------------------ greedy decode step */

/* Greedy next-token selection after the last layer: the token whose
 * output-head logit is largest, kept on the GPU for the next decode step
 * ("Perplexity Open-Sources Lily ...", section "Generation has a different
 * bottleneck").  The pages give no output head; the reading taken: a bf16
 * head w_head [V][H] applied to the bf16 hidden state x [T][H],
 *   logit[t][v] = fp32( x[t] . w_head[v] )   (double accumulation, one rounding)
 *   token[t]    = argmax_v logit[t][v], ties to the lower v.
 * Optional outputs: logits [T][V] (double, before the fp32 rounding) and
 * gap[t] = the selected fp32 logit minus the best other token's fp32 logit. */
int oracle_lm_head_argmax(int T, int H, int V, const uint16_t *x, const uint16_t *w_head,
                          int32_t *token, double *logits, double *gap)
{
    if (T < 0 || H <= 0 || V <= 0)
        return 1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int t = 0; t < T; ++t) {
        double *xv = malloc(sizeof(double) * H);
        float *l32 = malloc(sizeof(float) * V);
        if (!xv || !l32) { bad = 1; free(xv); free(l32); continue; }
        for (int k = 0; k < H; ++k)
            xv[k] = oracle_bf16_to_double(x[(int64_t)t * H + k]);
        for (int v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int k = 0; k < H; ++k)
                acc += xv[k] * oracle_bf16_to_double(w_head[(int64_t)v * H + k]);
            l32[v] = (float)acc;
            if (logits)
                logits[(int64_t)t * V + v] = acc;
        }
        int best = 0;
        for (int v = 1; v < V; ++v) {
#if ORACLE_MUTANT == 15
            if (l32[v] >= l32[best])                            /* tie -> higher token */
#else
            if (l32[v] > l32[best])
#endif
                best = v;
        }
        token[t] = best;
        if (gap) {
            double other = -INFINITY;
            for (int v = 0; v < V; ++v)
                if (v != best && (double)l32[v] > other)
                    other = (double)l32[v];
            gap[t] = (double)l32[best] - other;
        }
        free(xv); free(l32);
    }
    return bad ? 2 : 0;
}

/* The next step's input rows: x[t] = emb[token[t]] (bf16 [V][H] table).
 * Returns nonzero on a token outside 0..V-1. */
int oracle_embed(int T, int H, int V, const int32_t *token, const uint16_t *emb, uint16_t *x)
{
    for (int t = 0; t < T; ++t) {
        int v = token[t];
        if (v < 0 || v >= V)
            return 1;
#if ORACLE_MUTANT == 16
        v = (v + 1) % V;                                        /* neighbouring row */
#endif
        memcpy(x + (int64_t)t * H, emb + (int64_t)v * H, sizeof(uint16_t) * H);
    }
    return 0;
}
