/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for the fused attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: it exists so that the tests, the smoke check and the benchmark's CPU
 * baseline can compare the HIP kernels against an independent, obviously correct
 * implementation.  It shares no code, header, table or constant with the HIP path.
 *
 * What it computes (all arithmetic in IEEE double, libm exp/log, index order):
 *
 *   Softmax attention written out from its definition, as stated on the page
 *   "从零开始写Qwen3" (FlashAttention derivation article), section "简易情况-三矩阵相乘"
 *   (the softmax form of O) and section "FlashAttention" (O_i = sum_j softmax(mask(Q_i K_j^T / sqrt(D))) V_j):
 *
 *     for each batch b, query head h:  hk = h / (Hq / Hkv)          (grouped KV head,
 *         same page, the "pid_kh = pid_qh // groups" mapping in the kernel listing)
 *       for each query row i:
 *         visible keys V_i = { j < N : !causal  or  j <= i + (N - M) }
 *         s_ij = scale * sum_d q[b,h,i,d] * k[b,hk,j,d]
 *         m_i  = max_{j in V_i} s_ij
 *         l_i  = sum_{j in V_i} exp(s_ij - m_i)
 *         O[b,h,i,:] = sum_{j in V_i} exp(s_ij - m_i) / l_i * v[b,hk,j,:]
 *         lse[b,h,i] = m_i + ln(l_i)
 *         V_i empty  ->  O row = 0, lse = -inf
 *
 *   Readings taken where the pages are silent: the causal mask is aligned to the
 *   bottom-right corner (j <= i + N - M), which is the pages' "i >= j" when M == N;
 *   the logsumexp is the natural log over the scaled logits of the visible keys.
 *
 * Two further modes run the pages' online-softmax algorithm in fp64, only so that
 * the tests can check the definition above against it:
 *   - blockwise: the FlashAttention-2 loop of the same page (section "FlashAttention",
 *     the kernel listing's running max / running denominator / rescaled
 *     accumulator, divided by the denominator once after the loop), over blocks of
 *     `block` visible keys;
 *   - stepnorm: the per-step-normalised recurrence of section "在线softmax",
 *     O -> O exp(M_i - M_{i+1}) S_i / S_{i+1} + exp(V' ) / S_{i+1}, applied blockwise.
 *
 * Inputs are the raw 16-bit patterns of fp16 (dtype 0) or bf16 (dtype 1) tensors in
 * contiguous [B,H,rows,D] layout; this file decodes them itself (IEEE 754 binary16,
 * and bfloat16 = the top half of an IEEE binary32).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoders */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int exp = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (exp == 0) {
        mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-10 * 2^-14 */
    } else if (exp == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(frac | 0x400), exp - 25); /* (1 + frac/1024) * 2^(exp-15) */
    }
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int exp = (bits >> 7) & 0xff;
    int frac = bits & 0x7f;
    double mag;
    if (exp == 0) {
        mag = ldexp((double)frac, -133); /* subnormal: frac * 2^-7 * 2^-126 */
    } else if (exp == 255) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(frac | 0x80), exp - 134); /* (1 + frac/128) * 2^(exp-127) */
    }
    return sign ? -mag : mag;
}

static double *decode_all(const uint16_t *src, size_t n, int dtype)
{
    double *dst = (double *)malloc(n * sizeof(double));
    if (!dst)
        return NULL;
    for (size_t i = 0; i < n; ++i)
        dst[i] = dtype == 0 ? oracle_decode_f16(src[i]) : oracle_decode_bf16(src[i]);
    return dst;
}

/* ------------------------------------------------------------ shape helpers */

typedef struct {
    int B, Hq, Hkv, M, N, D, causal;
    double scale;
    const double *q, *k, *v; /* decoded, contiguous [B,H,rows,D] */
} problem;

/* number of visible keys of query row i: they are exactly j = 0 .. nvis-1 */
static long visible_count(const problem *p, long i)
{
    if (!p->causal)
        return p->N;
    long n = i + 1 + (long)p->N - (long)p->M; /* j <= i + N - M  <=>  j < i + 1 + N - M */
    if (n < 0)
        n = 0;
    if (n > p->N)
        n = p->N;
    return n;
}

static const double *q_row(const problem *p, int b, int h, long i)
{
    return p->q + (((size_t)b * p->Hq + h) * p->M + i) * p->D;
}

static const double *k_row(const problem *p, int b, int hk, long j)
{
    return p->k + (((size_t)b * p->Hkv + hk) * p->N + j) * p->D;
}

static const double *v_row(const problem *p, int b, int hk, long j)
{
    return p->v + (((size_t)b * p->Hkv + hk) * p->N + j) * p->D;
}

static double score(const problem *p, const double *qi, const double *kj)
{
    double acc = 0.0;
    for (int d = 0; d < p->D; ++d)
        acc += qi[d] * kj[d];
    return p->scale * acc;
}

/* ------------------------------------------------------ definition, one row */

/* s is scratch of length N. Writes D outputs to o and one lse. */
static void row_definition(const problem *p, int b, int h, long i, double *s, double *o, double *lse)
{
    int hk = h / (p->Hq / p->Hkv);
    long nv = visible_count(p, i);
    const double *qi = q_row(p, b, h, i);
    for (int d = 0; d < p->D; ++d)
        o[d] = 0.0;
    if (nv == 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (long j = 0; j < nv; ++j) {
        s[j] = score(p, qi, k_row(p, b, hk, j));
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (long j = 0; j < nv; ++j)
        l += exp(s[j] - m);
    for (long j = 0; j < nv; ++j) {
        double w = exp(s[j] - m) / l;
        const double *vj = v_row(p, b, hk, j);
        for (int d = 0; d < p->D; ++d)
            o[d] += w * vj[d];
    }
    *lse = m + log(l);
}

/* ------------------------------------- online softmax, blockwise (deferred) */

static void row_blockwise(const problem *p, int b, int h, long i, long block, double *s, double *o, double *lse)
{
    int hk = h / (p->Hq / p->Hkv);
    long nv = visible_count(p, i);
    const double *qi = q_row(p, b, h, i);
    for (int d = 0; d < p->D; ++d)
        o[d] = 0.0; /* the un-normalised accumulator */
    if (nv == 0) {
        *lse = -INFINITY;
        return;
    }
    double run_max = -INFINITY, denom = 0.0;
    for (long j0 = 0; j0 < nv; j0 += block) {
        long j1 = j0 + block < nv ? j0 + block : nv;
        double tile_max = -INFINITY;
        for (long j = j0; j < j1; ++j) {
            s[j - j0] = score(p, qi, k_row(p, b, hk, j));
            if (s[j - j0] > tile_max)
                tile_max = s[j - j0];
        }
        double new_max = run_max > tile_max ? run_max : tile_max;
        double factor = exp(run_max - new_max); /* exp(-inf) = 0 on the first block */
        double tile_sum = 0.0;
        for (int d = 0; d < p->D; ++d)
            o[d] *= factor;
        for (long j = j0; j < j1; ++j) {
            double e = exp(s[j - j0] - new_max);
            tile_sum += e;
            const double *vj = v_row(p, b, hk, j);
            for (int d = 0; d < p->D; ++d)
                o[d] += e * vj[d];
        }
        denom = denom * factor + tile_sum;
        run_max = new_max;
    }
    for (int d = 0; d < p->D; ++d)
        o[d] /= denom;
    *lse = run_max + log(denom);
}

/* ------------------------------ online softmax, normalised after every step */

static void row_stepnorm(const problem *p, int b, int h, long i, long block, double *s, double *o, double *lse)
{
    int hk = h / (p->Hq / p->Hkv);
    long nv = visible_count(p, i);
    const double *qi = q_row(p, b, h, i);
    for (int d = 0; d < p->D; ++d)
        o[d] = 0.0; /* always normalised by the current S */
    if (nv == 0) {
        *lse = -INFINITY;
        return;
    }
    double Mi = -INFINITY, Si = 0.0;
    for (long j0 = 0; j0 < nv; j0 += block) {
        long j1 = j0 + block < nv ? j0 + block : nv;
        double bmax = -INFINITY;
        for (long j = j0; j < j1; ++j) {
            s[j - j0] = score(p, qi, k_row(p, b, hk, j));
            if (s[j - j0] > bmax)
                bmax = s[j - j0];
        }
        double Mn = Mi > bmax ? Mi : bmax;
        double bsum = 0.0;
        for (long j = j0; j < j1; ++j)
            bsum += exp(s[j - j0] - Mn);
        double Sn = Si * exp(Mi - Mn) + bsum;
        double keep = exp(Mi - Mn) * Si / Sn; /* factor applied to the old O */
        for (int d = 0; d < p->D; ++d)
            o[d] *= keep;
        for (long j = j0; j < j1; ++j) {
            double w = exp(s[j - j0] - Mn) / Sn;
            const double *vj = v_row(p, b, hk, j);
            for (int d = 0; d < p->D; ++d)
                o[d] += w * vj[d];
        }
        Mi = Mn;
        Si = Sn;
    }
    *lse = Mi + log(Si);
}

/* ------------------------------------------------------------ entry points */

enum { MODE_DEFINITION = 0, MODE_BLOCKWISE = 1, MODE_STEPNORM = 2 };

/*
 * Computes the rows listed in `rows` (flat index (b*Hq + h)*M + i), or every row when
 * rows == NULL (then nrows must be B*Hq*M).  o is [nrows, D] fp64, lse is [nrows] fp64.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
static int run(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16, int dtype, int B, int Hq,
               int Hkv, int M, int N, int D, double scale, int causal, const int64_t *rows, int64_t nrows,
               int mode, long block, double *o, double *lse)
{
    if (!q16 || !k16 || !v16 || !o || !lse || B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || N <= 0 || D <= 0)
        return -1;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1) || block <= 0)
        return -1;
    size_t nq = (size_t)B * Hq * M * D, nk = (size_t)B * Hkv * N * D;
    problem p;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.M = M;
    p.N = N;
    p.D = D;
    p.causal = causal;
    p.scale = scale;
    double *q = decode_all(q16, nq, dtype), *k = decode_all(k16, nk, dtype), *v = decode_all(v16, nk, dtype);
    if (!q || !k || !v) {
        free(q);
        free(k);
        free(v);
        return -1;
    }
    p.q = q;
    p.k = k;
    p.v = v;
    int64_t total = rows ? nrows : (int64_t)B * Hq * M;
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < total; ++r) {
                int64_t flat = rows ? rows[r] : r;
                long i = (long)(flat % M);
                int bh = (int)(flat / M);
                int b = bh / Hq, h = bh % Hq;
                if (flat < 0 || b >= B) {
#pragma omp atomic write
                    err = 1;
                    continue;
                }
                double *orow = o + (size_t)r * D;
                if (mode == MODE_DEFINITION)
                    row_definition(&p, b, h, i, s, orow, lse + r);
                else if (mode == MODE_BLOCKWISE)
                    row_blockwise(&p, b, h, i, block, s, orow, lse + r);
                else
                    row_stepnorm(&p, b, h, i, block, s, orow, lse + r);
            }
            free(s);
        }
    }
    free(q);
    free(k);
    free(v);
    return err ? -1 : 0;
}

int oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype, int B, int Hq, int Hkv,
                    int M, int N, int D, double scale, int causal, double *o, double *lse)
{
    return run(q, k, v, dtype, B, Hq, Hkv, M, N, D, scale, causal, NULL, 0, MODE_DEFINITION, 1, o, lse);
}

int oracle_attn_fwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype, int B, int Hq,
                         int Hkv, int M, int N, int D, double scale, int causal, const int64_t *rows,
                         int64_t nrows, double *o, double *lse)
{
    if (!rows || nrows < 0)
        return -1;
    return run(q, k, v, dtype, B, Hq, Hkv, M, N, D, scale, causal, rows, nrows, MODE_DEFINITION, 1, o, lse);
}

int oracle_attn_fwd_blockwise(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype, int B, int Hq,
                              int Hkv, int M, int N, int D, double scale, int causal, long block, double *o,
                              double *lse)
{
    return run(q, k, v, dtype, B, Hq, Hkv, M, N, D, scale, causal, NULL, 0, MODE_BLOCKWISE, block, o, lse);
}

int oracle_attn_fwd_stepnorm(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype, int B, int Hq,
                             int Hkv, int M, int N, int D, double scale, int causal, long block, double *o,
                             double *lse)
{
    return run(q, k, v, dtype, B, Hq, Hkv, M, N, D, scale, causal, NULL, 0, MODE_STEPNORM, block, o, lse);
}

/*
 * The softmax weight matrix P[i][j] of one (b, h): exp(s_ij - m_i) / l_i on visible keys,
 * exactly 0 on masked ones.  P is [M, N] fp64.  Exposed only so tests can check the
 * weights themselves (rows sum to one, zeros where masked).
 */
int oracle_attn_probs(const uint16_t *q16, const uint16_t *k16, int dtype, int B, int Hq, int Hkv, int M, int N,
                      int D, double scale, int causal, int b, int h, double *P)
{
    if (!q16 || !k16 || !P || b < 0 || b >= B || h < 0 || h >= Hq || Hq % Hkv != 0 || D <= 0)
        return -1;
    problem p;
    memset(&p, 0, sizeof(p));
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.M = M;
    p.N = N;
    p.D = D;
    p.causal = causal;
    p.scale = scale;
    double *q = decode_all(q16, (size_t)B * Hq * M * D, dtype), *k = decode_all(k16, (size_t)B * Hkv * N * D, dtype);
    if (!q || !k) {
        free(q);
        free(k);
        return -1;
    }
    p.q = q;
    p.k = k;
    int hk = h / (Hq / Hkv);
    for (long i = 0; i < M; ++i) {
        double *Pi = P + (size_t)i * N;
        long nv = visible_count(&p, i);
        for (long j = 0; j < N; ++j)
            Pi[j] = 0.0;
        if (nv == 0)
            continue;
        double m = -INFINITY;
        for (long j = 0; j < nv; ++j) {
            Pi[j] = score(&p, q_row(&p, b, h, i), k_row(&p, b, hk, j));
            if (Pi[j] > m)
                m = Pi[j];
        }
        double l = 0.0;
        for (long j = 0; j < nv; ++j)
            l += exp(Pi[j] - m);
        for (long j = 0; j < nv; ++j)
            Pi[j] = exp(Pi[j] - m) / l;
    }
    free(q);
    free(k);
    return 0;
}

/* ------------------------------------------------------------------ backward */

/*
 * Gradients of O with respect to q, k and v for an upstream gradient dO (same shape as O),
 * written out from the chain rule of the definition above (not on the pages; lse is a saved
 * statistic of the forward and is not differentiated).  With z_ij = scale * q_i . k_j the
 * logits of row i over its visible keys and P_ij = softmax_j(z_ij):
 *
 *   O_i   = sum_j P_ij v_j                       -> dv_j  += P_ij dO_i
 *                                                   dP_ij  = dO_i . v_j
 *   P_i.  = softmax(z_i.)   (Jacobian diag(P) - P P^T)
 *                                                -> dz_ij  = P_ij (dP_ij - sum_k P_ik dP_ik)
 *   z_ij  = scale q_i . k_j                      -> dq_i  += scale dz_ij k_j
 *                                                   dk_j  += scale dz_ij q_i
 *
 * A KV head's dk and dv sum the contributions of every query head that reads it (the
 * grouped mapping h -> h / (Hq / Hkv)).  A row with no visible key contributes nothing and
 * gets dq = 0.  Outputs are fp64, contiguous: dq [B,Hq,M,D], dk and dv [B,Hkv,N,D].
 * Parallel over (b, kv head): each thread owns the dk/dv of its KV head.
 */
int oracle_attn_bwd(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16, const uint16_t *do16, int dtype,
                    int B, int Hq, int Hkv, int M, int N, int D, double scale, int causal, double *dq, double *dk,
                    double *dv)
{
    if (!q16 || !k16 || !v16 || !do16 || !dq || !dk || !dv || B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || N <= 0 ||
        D <= 0)
        return -1;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1))
        return -1;
    size_t nq = (size_t)B * Hq * M * D, nk = (size_t)B * Hkv * N * D;
    problem p;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.M = M;
    p.N = N;
    p.D = D;
    p.causal = causal;
    p.scale = scale;
    double *q = decode_all(q16, nq, dtype), *k = decode_all(k16, nk, dtype), *v = decode_all(v16, nk, dtype);
    double *dO = decode_all(do16, nq, dtype);
    if (!q || !k || !v || !dO) {
        free(q);
        free(k);
        free(v);
        free(dO);
        return -1;
    }
    p.q = q;
    p.k = k;
    p.v = v;
    memset(dq, 0, nq * sizeof(double));
    memset(dk, 0, nk * sizeof(double));
    memset(dv, 0, nk * sizeof(double));
    const int g = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc((size_t)N * sizeof(double));
        double *P = (double *)malloc((size_t)N * sizeof(double));
        double *dP = (double *)malloc((size_t)N * sizeof(double));
        if (!z || !P || !dP) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int bhk = 0; bhk < B * Hkv; ++bhk) {
                int b = bhk / Hkv, hk = bhk % Hkv;
                for (int h = hk * g; h < (hk + 1) * g; ++h) {
                    for (long i = 0; i < M; ++i) {
                        long nv = visible_count(&p, i);
                        if (nv == 0)
                            continue;
                        const double *qi = q_row(&p, b, h, i);
                        const double *doi = dO + (((size_t)b * Hq + h) * M + i) * D;
                        /* P_i. = softmax over the visible keys */
                        double m = -INFINITY;
                        for (long j = 0; j < nv; ++j) {
                            z[j] = score(&p, qi, k_row(&p, b, hk, j));
                            if (z[j] > m)
                                m = z[j];
                        }
                        double l = 0.0;
                        for (long j = 0; j < nv; ++j)
                            l += exp(z[j] - m);
                        for (long j = 0; j < nv; ++j)
                            P[j] = exp(z[j] - m) / l;
                        /* dP_ij = dO_i . v_j and its P-weighted mean */
                        double mean = 0.0;
                        for (long j = 0; j < nv; ++j) {
                            const double *vj = v_row(&p, b, hk, j);
                            double acc = 0.0;
                            for (int d = 0; d < D; ++d)
                                acc += doi[d] * vj[d];
                            dP[j] = acc;
                            mean += P[j] * acc;
                        }
                        double *dqi = dq + (((size_t)b * Hq + h) * M + i) * D;
                        for (long j = 0; j < nv; ++j) {
                            double dz = P[j] * (dP[j] - mean);
                            const double *kj = k_row(&p, b, hk, j);
                            double *dkj = dk + (((size_t)b * Hkv + hk) * N + j) * D;
                            double *dvj = dv + (((size_t)b * Hkv + hk) * N + j) * D;
                            for (int d = 0; d < D; ++d) {
                                dqi[d] += scale * dz * kj[d];
                                dkj[d] += scale * dz * qi[d];
                                dvj[d] += P[j] * doi[d];
                            }
                        }
                    }
                }
            }
        }
        free(z);
        free(P);
        free(dP);
    }
    free(q);
    free(k);
    free(v);
    free(dO);
    return err ? -1 : 0;
}

/*
 * The same gradients for a slice of one (batch b, KV head hk) group, organised so that each
 * output has one owner and large problems can be checked: dk and dv of the keys j0 <= j < j1 of
 * that KV head, and dq of a list of the group's query rows.  Same chain rule as oracle_attn_bwd:
 *   pass 1, per query row i of each of the group's heads: m_i = max_j s_ij, l_i = sum_j
 *     exp(s_ij - m_i), Delta_i = sum_j P_ij dP_ij with P_ij = exp(s_ij - m_i) / l_i and
 *     dP_ij = dO_i . v_j (visible keys j);
 *   pass 2, per key j of the slice: dv_j = sum_{h,i} P_ij dO_i and dk_j = scale sum_{h,i} dS_ij q_i
 *     over the rows i that see j, dS_ij = P_ij (dP_ij - Delta_i);
 *   pass 3, per listed row: dq_i = scale sum_j dS_ij k_j.
 * rows: indices r = (h - hk g) M + i of the group's rows (g = Hq / Hkv); dq_rows [n_rows][D];
 * dk_keys, dv_keys [j1 - j0][D].  Sums run in index order (rows, then heads, for pass 2).
 */
int oracle_attn_bwd_slice(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16, const uint16_t *do16,
                          int dtype, int B, int Hq, int Hkv, int M, int N, int D, double scale, int causal, int b,
                          int hk, long j0, long j1, const int64_t *rows, int64_t n_rows, double *dq_rows,
                          double *dk_keys, double *dv_keys)
{
    if (!q16 || !k16 || !v16 || !do16 || B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || N <= 0 || D <= 0)
        return -1;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1) || b < 0 || b >= B || hk < 0 || hk >= Hkv)
        return -1;
    if (j0 < 0 || j1 < j0 || j1 > N || (j1 > j0 && (!dk_keys || !dv_keys)) || n_rows < 0 ||
        (n_rows > 0 && (!rows || !dq_rows)))
        return -1;
    const int g = Hq / Hkv;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)g * M)
            return -1;
    size_t nq = (size_t)B * Hq * M * D, nk = (size_t)B * Hkv * N * D;
    problem p;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.M = M;
    p.N = N;
    p.D = D;
    p.causal = causal;
    p.scale = scale;
    double *q = decode_all(q16, nq, dtype), *k = decode_all(k16, nk, dtype), *v = decode_all(v16, nk, dtype);
    double *dO = decode_all(do16, nq, dtype);
    double *mrow = (double *)malloc((size_t)g * M * sizeof(double));
    double *lrow = (double *)malloc((size_t)g * M * sizeof(double));
    double *drow = (double *)malloc((size_t)g * M * sizeof(double));
    int err = 0;
    if (!q || !k || !v || !dO || !mrow || !lrow || !drow) {
        err = 1;
        goto done;
    }
    p.q = q;
    p.k = k;
    p.v = v;
    /* pass 1: row statistics */
#pragma omp parallel
    {
        double *z = (double *)malloc((size_t)N * sizeof(double));
        if (!z) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 64)
            for (long r = 0; r < (long)g * M; ++r) {
                const int h = hk * g + (int)(r / M);
                const long i = r % M;
                const long nv = visible_count(&p, i);
                if (nv == 0) {
                    mrow[r] = -INFINITY;
                    lrow[r] = 0.0;
                    drow[r] = 0.0;
                    continue;
                }
                const double *qi = q_row(&p, b, h, i);
                const double *doi = dO + (((size_t)b * Hq + h) * M + i) * D;
                double m = -INFINITY;
                for (long j = 0; j < nv; ++j) {
                    z[j] = score(&p, qi, k_row(&p, b, hk, j));
                    if (z[j] > m)
                        m = z[j];
                }
                double l = 0.0;
                for (long j = 0; j < nv; ++j)
                    l += exp(z[j] - m);
                double delta = 0.0;
                for (long j = 0; j < nv; ++j) {
                    const double P = exp(z[j] - m) / l;
                    const double *vj = v_row(&p, b, hk, j);
                    double dp = 0.0;
                    for (int d = 0; d < D; ++d)
                        dp += doi[d] * vj[d];
                    delta += P * dp;
                }
                mrow[r] = m;
                lrow[r] = l;
                drow[r] = delta;
            }
        }
        free(z);
    }
    if (err)
        goto done;
    /* pass 2: dk, dv of the keys of the slice */
#pragma omp parallel for schedule(dynamic, 1)
    for (long j = j0; j < j1; ++j) {
        double *dkj = dk_keys + (size_t)(j - j0) * D;
        double *dvj = dv_keys + (size_t)(j - j0) * D;
        for (int d = 0; d < D; ++d) {
            dkj[d] = 0.0;
            dvj[d] = 0.0;
        }
        const double *kj = k_row(&p, b, hk, j);
        const double *vj = v_row(&p, b, hk, j);
        for (int hh = 0; hh < g; ++hh) {
            const int h = hk * g + hh;
            for (long i = 0; i < M; ++i) {
                if (j >= visible_count(&p, i))
                    continue;
                const long r = (long)hh * M + i;
                const double *qi = q_row(&p, b, h, i);
                const double *doi = dO + (((size_t)b * Hq + h) * M + i) * D;
                const double P = exp(score(&p, qi, kj) - mrow[r]) / lrow[r];
                double dp = 0.0;
                for (int d = 0; d < D; ++d)
                    dp += doi[d] * vj[d];
                const double dz = P * (dp - drow[r]);
                for (int d = 0; d < D; ++d) {
                    dkj[d] += scale * dz * qi[d];
                    dvj[d] += P * doi[d];
                }
            }
        }
    }
    /* pass 3: dq of the listed rows */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_rows; ++t) {
        const long r = (long)rows[t];
        const int h = hk * g + (int)(r / M);
        const long i = r % M;
        double *dqi = dq_rows + (size_t)t * D;
        for (int d = 0; d < D; ++d)
            dqi[d] = 0.0;
        const long nv = visible_count(&p, i);
        const double *qi = q_row(&p, b, h, i);
        const double *doi = dO + (((size_t)b * Hq + h) * M + i) * D;
        for (long j = 0; j < nv; ++j) {
            const double *kj = k_row(&p, b, hk, j);
            const double *vj = v_row(&p, b, hk, j);
            const double P = exp(score(&p, qi, kj) - mrow[r]) / lrow[r];
            double dp = 0.0;
            for (int d = 0; d < D; ++d)
                dp += doi[d] * vj[d];
            const double dz = P * (dp - drow[r]);
            for (int d = 0; d < D; ++d)
                dqi[d] += scale * dz * kj[d];
        }
    }
done:
    free(q);
    free(k);
    free(v);
    free(dO);
    free(mrow);
    free(lrow);
    free(drow);
    return err ? -1 : 0;
}

/* Threads for the OpenMP loops of later calls (n >= 1; n <= 0 leaves it unchanged).  Returns
 * the previous setting, so a caller can time a single-threaded run and restore it. */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    const int old = omp_get_max_threads();
    if (n >= 1) omp_set_num_threads(n);
    return old;
#else
    (void)n;
    return 1;
#endif
}
