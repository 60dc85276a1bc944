/*
 * gdn_oracle.c -- plain CPU reference of the gated delta rule scan (the
 * recurrent layers of the model the pages describe).
 *
 * TEST INFRASTRUCTURE ONLY, under the same rules as moe_oracle.c: nothing
 * in the product path calls, links or loads it, and it shares no code,
 * header or constant with the HIP library.  It is compiled into the same
 * shared object as moe_oracle.c (whose bf16 helpers it uses).
 *
 * The pages say the model's Gated DeltaNet layers keep a recurrent state
 * and that the engine holds their scan in registers ("leslieli.dev note on
 * the Perplexity Lily engine", paragraph 3; "Perplexity Open-Sources Lily
 * ...", section "A runtime shaped around one model"), but they do not
 * define the recurrence.  This file takes the published gated delta rule
 * (S. Yang, J. Kautz, A. Hatamizadeh, "Gated Delta Networks: Improving
 * Mamba2 with Delta Rule", ICLR 2025) as the definition, per value head h
 * with key head h / (hv / hk):
 *
 *   S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  a_t = exp(g_t)
 *   o_t = S_t q_t
 *
 * S is dv x dk (row r: value channel r).  q, k, v are bf16 as given (any
 * normalisation or scaling of q and k belongs to the caller); g (the log of
 * the decay, <= 0 in use) and beta are fp32; the initial state is fp32 or
 * zero.  Everything is evaluated in IEEE double, dot products in ascending
 * index order; o is also returned rounded once to bf16.
 *
 * Parity against the pages is unpinned (they do not define the recurrence);
 * the test suite pins this function against closed forms, exact-retrieval
 * cases of the delta rule, an independent chunked derivation and
 * invariants.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUT(n) (ORACLE_MUTANT == (n))

double oracle_bf16_to_double(uint16_t b);
uint16_t oracle_double_to_bf16(double v);

/* Returns 0, or 1 on a bad argument.  Layouts (row-major):
 *   q, k   bf16 [T][hk][dk]      v  bf16 [T][hv][dv]
 *   g, beta fp32 [T][hv]         s0 fp32 [hv][dv][dk] or NULL (zero state)
 *   o      double [T][hv][dv]    o_bf16 bf16 [T][hv][dv] (may be NULL)
 *   s_out  double [hv][dv][dk]   (may be NULL) */
int oracle_gdn_scan(int T, int hk, int hv, int dk, int dv, const uint16_t *q,
                    const uint16_t *k, const uint16_t *v, const float *g,
                    const float *beta, const float *s0, double *o, uint16_t *o_bf16,
                    double *s_out)
{
    if (T < 0 || hk < 1 || hv < 1 || hv % hk || dk < 1 || dv < 1 || !o) return 1;
    if (T > 0 && (!q || !k || !v || !g || !beta)) return 1;
    const int group = hv / hk;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < hv; ++h) {
        const int kh = MUT(19) ? h % hk : h / group;
        double *S = calloc((size_t)dv * dk, sizeof(double));
        double *kk = malloc(sizeof(double) * (size_t)dk);
        double *qq = malloc(sizeof(double) * (size_t)dk);
        double *vv = malloc(sizeof(double) * (size_t)dv);
        double *Sk = malloc(sizeof(double) * (size_t)dv);
        if (!S || !kk || !qq || !vv || !Sk) {
#pragma omp atomic write
            bad = 1;
            free(S); free(kk); free(qq); free(vv); free(Sk);
            continue;
        }
        if (s0)
            for (size_t i = 0; i < (size_t)dv * dk; ++i) S[i] = s0[(size_t)h * dv * dk + i];
        for (int t = 0; t < T; ++t) {
            const uint16_t *kr = k + ((size_t)t * hk + kh) * dk;
            const uint16_t *qr = q + ((size_t)t * hk + kh) * dk;
            const uint16_t *vr = v + ((size_t)t * hv + h) * dv;
            for (int c = 0; c < dk; ++c) {
                kk[c] = oracle_bf16_to_double(kr[c]);
                qq[c] = oracle_bf16_to_double(qr[c]);
            }
            for (int r = 0; r < dv; ++r) vv[r] = oracle_bf16_to_double(vr[r]);
            const double a = exp((double)g[(size_t)t * hv + h]);
            const double b = (double)beta[(size_t)t * hv + h];
            double *ot = o + ((size_t)t * hv + h) * dv;
            if (MUT(20))   /* output read from the state before this token's update */
                for (int r = 0; r < dv; ++r) {
                    double s = 0.0;
                    for (int c = 0; c < dk; ++c) s += S[(size_t)r * dk + c] * qq[c];
                    ot[r] = s;
                }
            /* S (I - b k k^T): subtract b (S k) k^T; then decay, then the write */
            for (int r = 0; r < dv; ++r) {
                double s = 0.0;
                for (int c = 0; c < dk; ++c) s += S[(size_t)r * dk + c] * kk[c];
                Sk[r] = s;
            }
            const double be = MUT(18) ? 1.0 : b;
            for (int r = 0; r < dv; ++r)
                for (int c = 0; c < dk; ++c) {
                    double *sp = &S[(size_t)r * dk + c];
                    if (MUT(17))   /* decay applied after the write as well */
                        *sp = a * (*sp - be * Sk[r] * kk[c] + b * vv[r] * kk[c]);
                    else
                        *sp = a * (*sp - be * Sk[r] * kk[c]) + b * vv[r] * kk[c];
                }
            if (!MUT(20))
                for (int r = 0; r < dv; ++r) {
                    double s = 0.0;
                    for (int c = 0; c < dk; ++c) s += S[(size_t)r * dk + c] * qq[c];
                    ot[r] = s;
                }
            if (o_bf16)
                for (int r = 0; r < dv; ++r)
                    o_bf16[((size_t)t * hv + h) * dv + r] = oracle_double_to_bf16(ot[r]);
        }
        if (s_out)
            for (size_t i = 0; i < (size_t)dv * dk; ++i) s_out[(size_t)h * dv * dk + i] = S[i];
        free(S); free(kk); free(qq); free(vv); free(Sk);
    }
    return bad;
}
