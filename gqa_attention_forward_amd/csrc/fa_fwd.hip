// fa_fwd.hip -- fused attention forward for MI355X (gfx950, CDNA4), and its C ABI.
//
// One workgroup computes one (batch b, query head h, query tile of BM = 128 rows); its four
// waves own 32 query rows each.  The key/value sequence is the inner loop, in tiles of
// BN = 64 keys ("从零开始写Qwen3", FlashAttention derivation article, section "FlashAttention"
// and its variant note: Q tiles in parallel, KV as the inner loop).  K and V tiles are staged
// through double-buffered LDS; Q stays in registers for the whole loop.
//
// Transposed formulation.  The scores are computed as S^T = K Q^T and the output as
// O^T = V^T P^T on the 32x32x16 MFMA, so the MFMA accumulator's column index -- which is
// fixed per lane -- is the query.  A lane then holds 16 keys of one query row; the row's
// other 16 keys of each 32-key block sit in the lane 32 apart.  Row max is an in-lane
// reduction plus one cross-half swap; the row sum stays split across the two halves until
// the epilogue.  The probabilities P feed the second MFMA straight from registers.
//
// Key order inside a 32-key block is permuted (pi below) so that a lane's 16 accumulator
// rows are 16 consecutive keys: the B operand of O^T += V^T P^T is then the lane's own
// probabilities, and V^T is read from row-major V in LDS with the gfx950 transposing LDS
// read.  The same permutation on the rows of V^T makes each lane own 16 consecutive output
// columns.
//
// Online softmax in fp32 ("在线softmax" section of the derivation article): running max m,
// running sum l, accumulator rescaled by exp2((m_old - m_new) * c) with c = scale * log2(e)
// ("优化点6-使用exp2而不是exp", speed-up article), probabilities exp2(fma(s, c, -m*c)) (the
// scale folded into the FMA: "第一处：推迟 scale 乘法", B300 article), O divided by l once
// after the loop ("FlashAttention" listing).  Causal query tiles visit only the key tiles
// some row can see, unmasked tiles first, then the masked diagonal band ("改进2", "改进3").
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_tiles.h"

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kWaves = 4;     // 32 query rows per wave
constexpr int kThreads = kWaves * 64;

// ---------------------------------------------------------------- element types

template <typename T> struct Elem;

template <> struct Elem<_Float16> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
    // round-to-nearest-even fp32 -> fp16, two values packed in one dword (x in the low half)
    static __device__ __forceinline__ unsigned pack2(float x, float y)
    {
        _Float16 hx = (_Float16)x, hy = (_Float16)y;
        return (unsigned)__builtin_bit_cast(unsigned short, hx) |
               ((unsigned)__builtin_bit_cast(unsigned short, hy) << 16);
    }
};

template <> struct Elem<__bf16> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y)
    {
        __bf16 bx = (__bf16)x, by = (__bf16)y;
        return (unsigned)__builtin_bit_cast(unsigned short, bx) |
               ((unsigned)__builtin_bit_cast(unsigned short, by) << 16);
    }
};

// ------------------------------------------------------------------- layouts

// Row permutation of a 32-row MFMA operand block: A-operand row i holds key (or output
// column) pi(i), chosen so that accumulator register r of a lane in half hh maps to
// 16*hh + r.  (Accumulator row of register r in half hh is 8*(r/4) + 4*hh + r%4.)
__device__ __forceinline__ int pi32(int i) { return 16 * ((i >> 2) & 1) + ((i >> 3) << 2) + (i & 3); }

// LDS tiles are row-major [BN][D] in 16-byte units, XOR-swizzled per row so that the
// 16 lanes served together by one LDS pass hit 16 distinct 16-byte bank groups (gfx950
// LDS: 64 banks of 4 bytes).
template <int D> __device__ __forceinline__ int swz_k(int row, int unit)
{
    if constexpr (D == 128)  // MFMA A-operand reads touch rows pi(0..15): bits 0,1,4,2 distinguish them
        return unit ^ ((row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3));
    else  // 128-byte rows: two rows share a 256-byte bank window, the row's parity separates them
        return unit ^ (((row >> 1) & 1) | (((row >> 4) & 1) << 1) | (((row >> 2) & 1) << 2));
}

template <int D> __device__ __forceinline__ int swz_v(int row, int unit)
{
    // transposing reads touch 4 consecutive rows x units {u, u+2}: rows' low bits pick disjoint unit pairs
    if constexpr (D == 128)
        return unit ^ ((row & 1) | (((row >> 1) & 1) << 2));
    else
        return unit ^ ((row >> 1) & 1);
}

struct Params {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, Hq, Hkv, M, N;
    int n_qt;           // query tiles per (b, h)
    long long total;    // workgroups in the grid
    float c;            // scale * log2(e)
};

// --------------------------------------------------------------------- kernel

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(Params p)
{
    constexpr int UNITS = D / 8;                       // 16-byte units per row
    constexpr int ROWB = D * 2;                        // bytes per row
    constexpr int TILE_BYTES = kBN * ROWB;             // one K or V tile
    constexpr int LOADS = kBN * UNITS / kThreads;      // 16-byte global loads per thread per tile
    constexpr int KS = D / 16;                         // MFMA k-steps over the head dimension
    constexpr int KB = kBN / 32;                       // 32-key blocks per tile
    constexpr int DB = D / 32;                         // 32-column blocks of the output
    static_assert(LOADS * kThreads == kBN * UNITS, "tile must split evenly over the threads");

    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * 2 * TILE_BYTES];
    lds_u8 *smem = (lds_u8 *)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ql = lane & 31;   // query column of this lane inside the wave's 32 rows
    const int hh = lane >> 5;   // which half of each 32-key block this lane holds

    // ---- A1: which (b, h, query tile) this workgroup computes
    const long long L = xcd_remap(blockIdx.x, p.total);
    const TileCoord tc = logical_tile(L, p.Hq, p.Hkv, p.n_qt, CAUSAL);
    const int g = p.Hq / p.Hkv;
    const int hk = tc.h / g;
    const int m0 = tc.qt * kBM;
    const int M = p.M, N = p.N;
    const KvRange kr = kv_range(m0, kBM, kBN, M, N, CAUSAL);

    const T *qg = (const T *)p.q + ((size_t)tc.b * p.Hq + tc.h) * (size_t)M * D;
    const T *kg = (const T *)p.k + ((size_t)tc.b * p.Hkv + hk) * (size_t)N * D;
    const T *vg = (const T *)p.v + ((size_t)tc.b * p.Hkv + hk) * (size_t)N * D;

    const int qrow = m0 + wave * 32 + ql;  // this lane's query row
    const bool qvalid = qrow < M;

    // ---- A2: the Q operand, resident in registers (B operand of S^T = K Q^T)
    u32x4 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qreg[ks] = qvalid ? *(const u32x4 *)(qg + (size_t)qrow * D + ks * 16 + hh * 8) : z;
    }

    // ---- A3: global -> register -> LDS staging of one K tile and one V tile
    u32x4 kst[LOADS], vst[LOADS];
    auto load_tile = [&](int t) {
        const int n0 = t * kBN;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int c = j * kThreads + tid;
            const int row = c / UNITS, unit = c % UNITS;
            const bool ok = n0 + row < N;
            const size_t off = (size_t)(n0 + row) * D + unit * 8;
            u32x4 z = {0u, 0u, 0u, 0u};
            kst[j] = ok ? *(const u32x4 *)(kg + off) : z;
            vst[j] = ok ? *(const u32x4 *)(vg + off) : z;
        }
    };
    auto store_tile = [&](int buf) {
        lds_u8 *kb = smem + buf * 2 * TILE_BYTES;
        lds_u8 *vb = kb + TILE_BYTES;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int c = j * kThreads + tid;
            const int row = c / UNITS, unit = c % UNITS;
            *(lds_u32x4 *)(kb + row * ROWB + swz_k<D>(row, unit) * 16) = kst[j];
            *(lds_u32x4 *)(vb + row * ROWB + swz_v<D>(row, unit) * 16) = vst[j];
        }
    };

    // ---- online-softmax state (A6) and output accumulator
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY;  // running max of the raw scores s (not scaled)
    float l_part = 0.f;       // running sum over this half's keys, relative to m_run
    const float c = p.c;
    const int causal_lim = qrow + (N - M);  // last visible key of this row (causal)

    // per-lane constant parts of the LDS addresses
    const int krow_in_blk = pi32(ql);
    // transposing V read: source lane (e_src, j) of a 16-lane group supplies 4 columns
    const int tr_g = (lane >> 4) & 1, tr_s = lane & 15, tr_e = tr_s >> 2, tr_j = tr_s & 3;
    const int tr_dcol = 16 * (tr_j & 1) + 8 * tr_g + 4 * (tr_j >> 1);  // column offset inside a 32-column block

    const int n_tiles = kr.n_tiles;
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        if (t + 1 < n_tiles) load_tile(t + 1);  // in flight during this tile's math
        const lds_u8 *kb_lds = smem + (t & 1) * 2 * TILE_BYTES;
        const lds_u8 *vb_lds = kb_lds + TILE_BYTES;
        const int n0 = t * kBN;

        // ---- A4: S^T = K Q^T, fp32 accumulate; lane holds keys n0 + 32*kb + 16*hh + r of row qrow
        f32x16 s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int row = kb * 32 + krow_in_blk;
                const u32x4 a = *(const lds_u32x4 *)(kb_lds + row * ROWB + swz_k<D>(row, 2 * ks + hh) * 16);
                s[kb] = Elem<T>::mfma(a, qreg[ks], s[kb]);
            }
        }

        // ---- A5: mask on the diagonal band and on a ragged last tile only
        if (t >= kr.n_full) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = n0 + kb * 32 + hh * 16 + r;
                    const bool vis = key < N && (!CAUSAL || key <= causal_lim);
                    s[kb][r] = vis ? s[kb][r] : -INFINITY;
                }
        }

        // ---- A6: online softmax for this tile
        float mt = s[0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
        {
            // the other half of the row lives in lane ^ 32
            auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mt),
                                                       __builtin_bit_cast(unsigned, mt), false, false);
            mt = fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no visible key yet: keep exp2 finite
        const float mc = m_use * c;
        const float alpha = __builtin_amdgcn_exp2f(m_run * c - mc);  // 0 on the first visible tile
        m_run = m_new;

        float psum = 0.f;
        unsigned pk[KB][8];  // probabilities rounded to T, two per dword, in key order
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -mc));
                psum += p0 + p1;
                pk[kb][r / 2] = Elem<T>::pack2(p0, p1);
            }
        l_part = l_part * alpha + psum;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }

        // ---- A7: O^T += V^T P^T; P is the B operand straight from registers
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                u32x4 bop = {pk[kb][4 * tt], pk[kb][4 * tt + 1], pk[kb][4 * tt + 2], pk[kb][4 * tt + 3]};
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    i16x4 lo, hi;
                    {
                        const int row = kb * 32 + hh * 16 + tt * 8 + tr_e;  // keys k0 .. k0+3
                        const int col = db * 32 + tr_dcol;
                        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4 *)(vb_lds + row * ROWB + swz_v<D>(row, col >> 3) * 16 + (col & 7) * 2));
                    }
                    {
                        const int row = kb * 32 + hh * 16 + tt * 8 + 4 + tr_e;  // keys k0+4 .. k0+7
                        const int col = db * 32 + tr_dcol;
                        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4 *)(vb_lds + row * ROWB + swz_v<D>(row, col >> 3) * 16 + (col & 7) * 2));
                    }
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 aop = {lo2[0], lo2[1], hi2[0], hi2[1]};
                    oacc[db] = Elem<T>::mfma(aop, bop, oacc[db]);
                }
            }
        }

        if (t + 1 < n_tiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // ---- A8: epilogue -- normalise once, write O and the logsumexp
    float l_tot;
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, l_part),
                                                   __builtin_bit_cast(unsigned, l_part), false, false);
        l_tot = __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
    }
    if (qvalid) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        T *og = (T *)p.o + (((size_t)tc.b * p.Hq + tc.h) * (size_t)M + qrow) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x4 w0, w1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                w0[r] = Elem<T>::pack2(oacc[db][2 * r] * inv, oacc[db][2 * r + 1] * inv);
                w1[r] = Elem<T>::pack2(oacc[db][8 + 2 * r] * inv, oacc[db][8 + 2 * r + 1] * inv);
            }
            u32x4 *dst = (u32x4 *)(og + db * 32 + hh * 16);
            dst[0] = w0;
            dst[1] = w1;
        }
        if (hh == 0) {
            const float lse2 = l_tot > 0.f ? m_run * c + __builtin_log2f(l_tot) : -INFINITY;
            p.lse[((size_t)tc.b * p.Hq + tc.h) * (size_t)M + qrow] = lse2 * 0.69314718055994530942f;
        }
    }
}

// ------------------------------------------------------------------ host side

static int tile_shape(int D, int *BM, int *BN)
{
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    *BM = kBM;
    *BN = kBN;
    return FA_OK;
}

template <typename T, int D>
static hipError_t launch_d(const Params &p, bool causal, hipStream_t stream)
{
    dim3 grid((unsigned)p.total), block(kThreads);
    if (causal)
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(const Params &p, int D, bool causal, hipStream_t stream)
{
    return D == 128 ? launch_d<T, 128>(p, causal, stream) : launch_d<T, 64>(p, causal, stream);
}

}  // namespace fa

extern "C" {

const char *fa_strerror(int code)
{
    switch (code) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (head dim must be 64 or 128, pointers 16-byte aligned)";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error code";
    }
}

int fa_tile_shape(int D, int *BM, int *BN)
{
    if (!BM || !BN) return FA_ERR_INVALID_ARG;
    return fa::tile_shape(D, BM, BN);
}

int fa_tile_counts(int M, int N, int BM, int BN, int causal, long long *full, long long *masked, long long *skipped)
{
    if (!full || !masked || !skipped || M <= 0 || N <= 0 || BM <= 0 || BN <= 0) return FA_ERR_INVALID_ARG;
    long long f = 0, m = 0, s = 0;
    const int n_qt = (M + BM - 1) / BM, n_kt = (N + BN - 1) / BN;
    for (int qt = 0; qt < n_qt; ++qt) {
        fa::KvRange r = fa::kv_range(qt * BM, BM, BN, M, N, causal != 0);
        f += r.n_full;
        m += r.n_tiles - r.n_full;
        s += n_kt - r.n_tiles;
    }
    *full = f;
    *masked = m;
    *skipped = s;
    return FA_OK;
}

int fa_schedule(int B, int Hq, int Hkv, int M, int D, int causal, long long wg, int *b, int *h, int *q_tile)
{
    int BM, BN;
    if (!b || !h || !q_tile || B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (fa::tile_shape(D, &BM, &BN) != FA_OK) return FA_ERR_INVALID_ARG;
    const int n_qt = (M + BM - 1) / BM;
    const long long total = (long long)B * Hq * n_qt;
    if (wg < 0 || wg >= total) return FA_ERR_INVALID_ARG;
    fa::TileCoord c = fa::logical_tile(fa::xcd_remap(wg, total), Hq, Hkv, n_qt, causal != 0);
    *b = c.b;
    *h = c.h;
    *q_tile = c.qt;
    return FA_OK;
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M, int N,
           int D, float scale, int causal, int dtype, void *stream)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || N <= 0 || D <= 0) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    // element counts must fit in int64 (they do for any int sizes below 2^15 each; check anyway)
    const double nq = (double)B * Hq * M * D, nk = (double)B * Hkv * N * D;
    if (nq > 9.0e18 || nk > 9.0e18) return FA_ERR_INVALID_ARG;
    int BM, BN;
    if (fa::tile_shape(D, &BM, &BN) != FA_OK) return FA_ERR_UNSUPPORTED;
    const uintptr_t align = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
    if (align & 15u) return FA_ERR_UNSUPPORTED;

    fa::Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.M = M;
    p.N = N;
    p.n_qt = (M + BM - 1) / BM;
    p.total = (long long)B * Hq * p.n_qt;
    if (p.total > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;  // one-dimensional grid limit
    p.c = scale * 1.44269504088896340736f;                    // log2(e)

    hipStream_t s = (hipStream_t)stream;
    hipError_t err = dtype == FA_F16 ? fa::launch_t<_Float16>(p, D, causal != 0, s)
                                     : fa::launch_t<__bf16>(p, D, causal != 0, s);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
