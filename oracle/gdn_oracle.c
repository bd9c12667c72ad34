/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for the Gated DeltaNet chunked prefill.
 *
 * TEST INFRASTRUCTURE ONLY, like attn_oracle.c: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; it shares no code with the HIP path.
 *
 * Source: the page "lab3：GDN Prefill 前向优化", section "算法与数据依赖" (the chunk recurrence,
 * chunk length 64, head dim 128, the framework-side inputs g_cumsum and A) and its GVA note
 * (value head h reads query/key head h / (Hv / Hqk)).
 *
 * Layouts (contiguous): q, k [B, T, Hqk, DK]; v [B, T, Hv, DV]; g (the gate's cumulative sum
 * inside each chunk) and beta [B, T, Hv]; A [B, T, Hv, C] (row t of its chunk's C x C matrix);
 * states [B, Hv, DK, DV]; o [B, T, Hv, DV].  q, k, v arrive as fp16 (dtype 0) or bf16 (dtype 1)
 * bit patterns and are decoded with this file's own decoders; everything else is fp64.
 * Chunks are [cC, cC + C) clipped to T.
 *
 * Three functions:
 *   oracle_gdn_chunked   -- the page's chunk recurrence in its order, with A given:
 *       U' = K S_c;  W' = beta (V - exp(g) U');  V_new = A W';
 *       S_{c+1} = exp(g_last) S_c + (K exp(g_last - g))^T V_new;
 *       O = scale (exp(g) (Q S_c) + scores V_new),  scores_ts = (q_t . k_s) exp(g_t - g_s), s <= t.
 *   oracle_gdn_recurrent -- the token-by-token gated delta rule the chunk form rewrites (not
 *       printed on the page; the reading that makes the page's equations exact):
 *       per token, with the gate a_t = exp(g_t - g_{t-1}) (g_{-1} = 0 at a chunk start):
 *       S <- a_t S;  u_t = beta_t (v_t - S^T k_t);  S <- S + k_t u_t^T;  o_t = scale S^T q_t.
 *   oracle_gdn_kkt       -- the A the chunk form needs for that equality: per chunk,
 *       A = (I + L)^{-1} with L_ts = beta_t (k_t . k_s) exp(g_t - g_s) for s < t (0 otherwise),
 *       by forward substitution (the page's "KKT triangular solve", with beta and the gate
 *       decay folded in, as its section on the rejected FlashQLA port says the inputs have).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double oracle_decode_f16(uint16_t bits);
double oracle_decode_bf16(uint16_t bits);

typedef struct {
    int B, T, Hqk, Hv, DK, DV, C;
    double scale;
    double *q, *k, *v; /* decoded */
    const double *g, *beta;
} gdn;

static double *decode16(const uint16_t *src, size_t n, int dtype)
{
    double *d = (double *)malloc(n * sizeof(double));
    if (!d)
        return NULL;
    for (size_t i = 0; i < n; ++i)
        d[i] = dtype == 0 ? oracle_decode_f16(src[i]) : oracle_decode_bf16(src[i]);
    return d;
}

static const double *qrow(const gdn *p, int b, int t, int hk) { return p->q + (((size_t)b * p->T + t) * p->Hqk + hk) * p->DK; }
static const double *krow(const gdn *p, int b, int t, int hk) { return p->k + (((size_t)b * p->T + t) * p->Hqk + hk) * p->DK; }
static const double *vrow(const gdn *p, int b, int t, int h) { return p->v + (((size_t)b * p->T + t) * p->Hv + h) * p->DV; }
static double gat(const gdn *p, int b, int t, int h) { return p->g[((size_t)b * p->T + t) * p->Hv + h]; }
static double bat(const gdn *p, int b, int t, int h) { return p->beta[((size_t)b * p->T + t) * p->Hv + h]; }

static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i)
        s += a[i] * b[i];
    return s;
}

static int setup(gdn *p, const uint16_t *q16, const uint16_t *k16, const uint16_t *v16, int dtype, const double *g,
                 const double *beta, int B, int T, int Hqk, int Hv, int DK, int DV, int C, double scale)
{
    if (!q16 || !k16 || !v16 || !g || !beta || B <= 0 || T <= 0 || Hqk <= 0 || Hv <= 0 || DK <= 0 || DV <= 0 ||
        C <= 0 || Hv % Hqk != 0 || (dtype != 0 && dtype != 1))
        return -1;
    p->B = B;
    p->T = T;
    p->Hqk = Hqk;
    p->Hv = Hv;
    p->DK = DK;
    p->DV = DV;
    p->C = C;
    p->scale = scale;
    p->g = g;
    p->beta = beta;
    size_t nqk = (size_t)B * T * Hqk * DK, nv = (size_t)B * T * Hv * DV;
    p->q = decode16(q16, nqk, dtype);
    p->k = decode16(k16, nqk, dtype);
    p->v = decode16(v16, nv, dtype);
    if (!p->q || !p->k || !p->v) {
        free(p->q);
        free(p->k);
        free(p->v);
        return -1;
    }
    return 0;
}

static void teardown(gdn *p)
{
    free(p->q);
    free(p->k);
    free(p->v);
}

/* ---------------------------------------------------------- token recurrence */

int oracle_gdn_recurrent(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16, int dtype, const double *g,
                         const double *beta, const double *s0, int B, int T, int Hqk, int Hv, int DK, int DV, int C,
                         double scale, double *o, double *s_final)
{
    gdn p;
    if (!o || !s_final || setup(&p, q16, k16, v16, dtype, g, beta, B, T, Hqk, Hv, DK, DV, C, scale))
        return -1;
    int err = 0;
#pragma omp parallel
    {
        double *u = (double *)malloc((size_t)DV * sizeof(double));
        if (!u) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int bh = 0; bh < B * Hv; ++bh) {
                int b = bh / Hv, h = bh % Hv, hk = h / (Hv / Hqk);
                double *S = s_final + (size_t)bh * DK * DV; /* S[d][e] */
                if (s0)
                    memcpy(S, s0 + (size_t)bh * DK * DV, (size_t)DK * DV * sizeof(double));
                else
                    memset(S, 0, (size_t)DK * DV * sizeof(double));
                for (int t = 0; t < T; ++t) {
                    double prev = (t % C == 0) ? 0.0 : gat(&p, b, t - 1, h);
                    double a = exp(gat(&p, b, t, h) - prev);
                    const double *kt = krow(&p, b, t, hk), *qt = qrow(&p, b, t, hk), *vt = vrow(&p, b, t, h);
                    double bt = bat(&p, b, t, h);
                    for (size_t i = 0; i < (size_t)DK * DV; ++i)
                        S[i] *= a;
                    for (int e = 0; e < DV; ++e) {
                        double sk = 0.0;
                        for (int d = 0; d < DK; ++d)
                            sk += S[(size_t)d * DV + e] * kt[d];
                        u[e] = bt * (vt[e] - sk);
                    }
                    for (int d = 0; d < DK; ++d)
                        for (int e = 0; e < DV; ++e)
                            S[(size_t)d * DV + e] += kt[d] * u[e];
                    double *ot = o + (((size_t)b * T + t) * Hv + h) * DV;
                    for (int e = 0; e < DV; ++e) {
                        double acc = 0.0;
                        for (int d = 0; d < DK; ++d)
                            acc += S[(size_t)d * DV + e] * qt[d];
                        ot[e] = scale * acc;
                    }
                }
            }
            free(u);
        }
    }
    teardown(&p);
    return err ? -1 : 0;
}

/* ---------------------------------------------------------------- KKT solve */

int oracle_gdn_kkt(const uint16_t *k16, int dtype, const double *g, const double *beta, int B, int T, int Hqk,
                   int Hv, int DK, int C, double *A)
{
    if (!k16 || !g || !beta || !A || B <= 0 || T <= 0 || Hqk <= 0 || Hv <= 0 || DK <= 0 || C <= 0 || Hv % Hqk)
        return -1;
    double *k = decode16(k16, (size_t)B * T * Hqk * DK, dtype);
    if (!k)
        return -1;
    int err = 0;
    const int nch = (T + C - 1) / C;
#pragma omp parallel
    {
        double *L = (double *)malloc((size_t)C * C * sizeof(double));
        double *X = (double *)malloc((size_t)C * C * sizeof(double));
        if (!L || !X) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long job = 0; job < (long)B * Hv * nch; ++job) {
                int b = (int)(job / ((long)Hv * nch)), h = (int)(job / nch % Hv), c = (int)(job % nch);
                int hk = h / (Hv / Hqk), t0 = c * C, n = T - t0 < C ? T - t0 : C;
                for (int t = 0; t < n; ++t)
                    for (int s = 0; s < n; ++s) {
                        double v = 0.0;
                        if (s < t) {
                            const double *kt = k + (((size_t)b * T + t0 + t) * Hqk + hk) * DK;
                            const double *ks = k + (((size_t)b * T + t0 + s) * Hqk + hk) * DK;
                            size_t it = ((size_t)b * T + t0 + t) * Hv + h, is = ((size_t)b * T + t0 + s) * Hv + h;
                            v = beta[it] * dot(kt, ks, DK) * exp(g[it] - g[is]);
                        }
                        L[(size_t)t * C + s] = v;
                    }
                /* (I + L) X = I, L strictly lower: row t of X = e_t - sum_{s<t} L_ts X_s */
                for (int t = 0; t < n; ++t)
                    for (int j = 0; j < n; ++j) {
                        double x = (t == j) ? 1.0 : 0.0;
                        for (int s = 0; s < t; ++s)
                            x -= L[(size_t)t * C + s] * X[(size_t)s * C + j];
                        X[(size_t)t * C + j] = x;
                    }
                for (int t = 0; t < n; ++t) {
                    double *row = A + (((size_t)b * T + t0 + t) * Hv + h) * C;
                    for (int j = 0; j < C; ++j)
                        row[j] = j < n ? X[(size_t)t * C + j] : 0.0;
                }
            }
        }
        free(L);
        free(X);
    }
    free(k);
    return err ? -1 : 0;
}

/* ------------------------------------------------------------ chunk recurrence */

int oracle_gdn_chunked(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16, int dtype, const double *g,
                       const double *beta, const double *A, const double *s0, int B, int T, int Hqk, int Hv, int DK,
                       int DV, int C, double scale, double *o, double *s_final)
{
    gdn p;
    if (!A || !o || !s_final || setup(&p, q16, k16, v16, dtype, g, beta, B, T, Hqk, Hv, DK, DV, C, scale))
        return -1;
    int err = 0;
#pragma omp parallel
    {
        double *U = (double *)malloc((size_t)C * DV * sizeof(double)); /* U' then W' */
        double *Vn = (double *)malloc((size_t)C * DV * sizeof(double));
        double *S2 = (double *)malloc((size_t)DK * DV * sizeof(double));
        if (!U || !Vn || !S2) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int bh = 0; bh < B * Hv; ++bh) {
                int b = bh / Hv, h = bh % Hv, hk = h / (Hv / Hqk);
                double *S = s_final + (size_t)bh * DK * DV;
                if (s0)
                    memcpy(S, s0 + (size_t)bh * DK * DV, (size_t)DK * DV * sizeof(double));
                else
                    memset(S, 0, (size_t)DK * DV * sizeof(double));
                for (int t0 = 0; t0 < T; t0 += C) {
                    int n = T - t0 < C ? T - t0 : C;
                    /* U' = K S_c ; W' = beta (V - exp(g) U') */
                    for (int t = 0; t < n; ++t) {
                        const double *kt = krow(&p, b, t0 + t, hk), *vt = vrow(&p, b, t0 + t, h);
                        double eg = exp(gat(&p, b, t0 + t, h)), bt = bat(&p, b, t0 + t, h);
                        for (int e = 0; e < DV; ++e) {
                            double u = 0.0;
                            for (int d = 0; d < DK; ++d)
                                u += kt[d] * S[(size_t)d * DV + e];
                            U[(size_t)t * DV + e] = bt * (vt[e] - eg * u);
                        }
                    }
                    /* V_new = A W' */
                    for (int t = 0; t < n; ++t) {
                        const double *at = A + (((size_t)b * T + t0 + t) * Hv + h) * C;
                        for (int e = 0; e < DV; ++e) {
                            double x = 0.0;
                            for (int s = 0; s < n; ++s)
                                x += at[s] * U[(size_t)s * DV + e];
                            Vn[(size_t)t * DV + e] = x;
                        }
                    }
                    /* O = scale (exp(g) Q S_c + scores V_new) */
                    for (int t = 0; t < n; ++t) {
                        const double *qt = qrow(&p, b, t0 + t, hk);
                        double gt = gat(&p, b, t0 + t, h);
                        double *ot = o + (((size_t)b * T + t0 + t) * Hv + h) * DV;
                        for (int e = 0; e < DV; ++e) {
                            double qs = 0.0;
                            for (int d = 0; d < DK; ++d)
                                qs += qt[d] * S[(size_t)d * DV + e];
                            ot[e] = exp(gt) * qs;
                        }
                        for (int s = 0; s <= t; ++s) {
                            double sc = dot(qt, krow(&p, b, t0 + s, hk), DK) * exp(gt - gat(&p, b, t0 + s, h));
                            for (int e = 0; e < DV; ++e)
                                ot[e] += sc * Vn[(size_t)s * DV + e];
                        }
                        for (int e = 0; e < DV; ++e)
                            ot[e] *= scale;
                    }
                    /* S_{c+1} = exp(g_last) S_c + (K exp(g_last - g))^T V_new */
                    double gl = gat(&p, b, t0 + n - 1, h);
                    for (int d = 0; d < DK; ++d)
                        for (int e = 0; e < DV; ++e) {
                            double x = exp(gl) * S[(size_t)d * DV + e];
                            for (int s = 0; s < n; ++s)
                                x += krow(&p, b, t0 + s, hk)[d] * exp(gl - gat(&p, b, t0 + s, h)) *
                                     Vn[(size_t)s * DV + e];
                            S2[(size_t)d * DV + e] = x;
                        }
                    memcpy(S, S2, (size_t)DK * DV * sizeof(double));
                }
            }
        }
        free(U);
        free(Vn);
        free(S2);
    }
    teardown(&p);
    return err ? -1 : 0;
}
