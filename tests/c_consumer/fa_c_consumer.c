/*
 * A plain C99 consumer of libfa.so: device memory and the copies through the HIP runtime's C API,
 * the forward through fa.h alone, and the fp64 oracle (test infrastructure) for the check.
 *
 *   fa_c_consumer B Hq Hkv M N D causal      exit 0 when O and lse agree with the oracle within
 *                                            the bf16 tolerances (max-abs 1.6e-2, lse 1e-3)
 *
 * Inputs are bf16, drawn from a fixed xorshift generator (sums of uniforms, roughly N(0, 1)).
 * It also checks two error paths: an unsupported head dimension and a null pointer, both
 * rejected before any device work, and fa_strerror's text for them.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

/* oracle/attn_oracle.c (linked from oracle/liboracle.so) */
int oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype, int B, int Hq, int Hkv,
                    int M, int N, int D, double scale, int causal, double *o, double *lse);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform01(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}
/* round-to-nearest-even fp32 -> bf16 bits */
static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

#define CHECK_HIP(call)                                                                  \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));            \
            return 2;                                                                    \
        }                                                                                \
    } while (0)

int main(int argc, char **argv)
{
    if (argc != 8) {
        fprintf(stderr, "usage: %s B Hq Hkv M N D causal\n", argv[0]);
        return 2;
    }
    const int B = atoi(argv[1]), Hq = atoi(argv[2]), Hkv = atoi(argv[3]), M = atoi(argv[4]), N = atoi(argv[5]),
              D = atoi(argv[6]), causal = atoi(argv[7]);
    const size_t nq = (size_t)B * Hq * M * D, nk = (size_t)B * Hkv * N * D, nl = (size_t)B * Hq * M;
    uint16_t *hq = malloc(nq * 2), *hk = malloc(nk * 2), *hv = malloc(nk * 2), *ho = malloc(nq * 2);
    float *hl = malloc(nl * 4);
    double *ro = malloc(nq * 8), *rl = malloc(nl * 8);
    if (!hq || !hk || !hv || !ho || !hl || !ro || !rl) return 2;
    uint16_t *bufs[3] = {hq, hk, hv};
    const size_t lens[3] = {nq, nk, nk};
    for (int t = 0; t < 3; ++t)
        for (size_t i = 0; i < lens[t]; ++i)
            bufs[t][i] = to_bf16((float)(uniform01() + uniform01() + uniform01() - 1.5) * 2.0f);

    void *dq, *dk, *dv, *dout;
    float *dlse;
    CHECK_HIP(hipMalloc(&dq, nq * 2));
    CHECK_HIP(hipMalloc(&dk, nk * 2));
    CHECK_HIP(hipMalloc(&dv, nk * 2));
    CHECK_HIP(hipMalloc(&dout, nq * 2));
    CHECK_HIP(hipMalloc((void **)&dlse, nl * 4));
    CHECK_HIP(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk, hk, nk * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, hv, nk * 2, hipMemcpyHostToDevice));

    /* error paths: rejected on the host, nothing enqueued */
    int rc = fa_fwd(dq, dk, dv, dout, dlse, B, Hq, Hkv, M, N, 96, 0.1f, causal, FA_BF16, NULL);
    printf("D=96: %d (%s)\n", rc, fa_strerror(rc));
    if (rc != FA_ERR_UNSUPPORTED) return 1;
    rc = fa_fwd(NULL, dk, dv, dout, dlse, B, Hq, Hkv, M, N, D, 0.1f, causal, FA_BF16, NULL);
    printf("q=NULL: %d (%s)\n", rc, fa_strerror(rc));
    if (rc != FA_ERR_INVALID_ARG) return 1;

    const float scale = 1.0f / sqrtf((float)D);
    rc = fa_fwd(dq, dk, dv, dout, dlse, B, Hq, Hkv, M, N, D, scale, causal, FA_BF16, NULL);
    if (rc != FA_OK) {
        fprintf(stderr, "fa_fwd: %s\n", fa_strerror(rc));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(ho, dout, nq * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hl, dlse, nl * 4, hipMemcpyDeviceToHost));

    if (oracle_attn_fwd(hq, hk, hv, 1, B, Hq, Hkv, M, N, D, (double)scale, causal, ro, rl) != 0) return 2;
    double err = 0.0, lerr = 0.0;
    for (size_t i = 0; i < nq; ++i) {
        const double d = fabs(from_bf16(ho[i]) - ro[i]);
        if (!(d <= err)) err = d; /* also catches NaN */
    }
    for (size_t i = 0; i < nl; ++i) {
        if (isinf(rl[i])) {
            if (!isinf(hl[i])) lerr = INFINITY;
            continue;
        }
        const double d = fabs((double)hl[i] - rl[i]);
        if (!(d <= lerr)) lerr = d;
    }
    printf("B=%d Hq=%d Hkv=%d M=%d N=%d D=%d causal=%d: max|dO| %.3e (tol 1.6e-2), max|dlse| %.3e (tol 1e-3)\n", B, Hq,
           Hkv, M, N, D, causal, err, lerr);
    hipFree(dq);
    hipFree(dk);
    hipFree(dv);
    hipFree(dout);
    hipFree(dlse);
    return err <= 1.6e-2 && lerr <= 1e-3 ? 0 : 1;
}
