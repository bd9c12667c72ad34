// gdn_fwd.hip -- Gated DeltaNet chunked prefill for MI355X (gfx950): the chunk recurrence of the
// page "lab3：GDN Prefill 前向优化", section "算法与数据依赖", and the per-chunk triangular solve
// that produces its A input.
//
// Per value head h (reading query/key head h / (Hv / Hqk)) and 64-token chunk c, with g the
// gate's cumulative log inside the chunk:
//     U' = K S_c;  W' = beta (V - exp(g) U');  V_new = A W';
//     O  = scale (exp(g) (Q S_c) + scores V_new),  scores_ts = (q_t . k_s) exp(g_t - g_s), s <= t;
//     S_{c+1} = exp(g_last) S_c + (K exp(g_last - g))^T V_new,
// with A = (I + L)^-1, L_ts = beta_t (k_t . k_s) exp(g_t - g_s) for s < t.
//
// chunk_kernel: one workgroup (4 waves) per (b, value head, 64 columns of the state), walking the
// chunks in order -- the state is the only thing carried from chunk to chunk, and each slice of
// it is independent, as the page's split of the state over (batch, V head, DV block) notes.
// The fp32 state lives in MFMA accumulators for the whole sequence; each chunk a bf16 copy
// goes to LDS as the operand of U' and Q S (operands bf16/fp16, accumulation and state fp32,
// as on the page).  The six products per chunk run on the 32x32x16 MFMA with every operand
// read from LDS; a result that feeds a later product as its B operand is written to LDS
// transposed (a lane's accumulator column holds 4 consecutive rows per register group, so the
// transposed write is 8 bytes).  Q and K tiles use the XOR-swizzled layout because K is also
// read transposed (K^T of the state update); the next chunk's Q, K, A, g and beta are copied
// HBM -> LDS by buffer loads while the current chunk computes.
//
// kkt_kernel: one workgroup per (b, value head, chunk): K K^T on MFMA, L, then the unit lower
// triangular inverse by forward substitution, one lane per column of A, in registers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_device.h"
#include "fa_swizzle.h"
#include "gdn.h"

namespace fa {
namespace gdn {

constexpr int C = 64;     // chunk length
constexpr int DK = 128;   // query/key head dim
constexpr int DVB = 64;   // state columns a workgroup owns
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float exp_(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Row order of a 32-row A operand that makes accumulator register r of lane half hh hold row
// 16 hh + r (the accumulator row of register r in half hh is 8 (r / 4) + 4 hh + r % 4).
__device__ __forceinline__ constexpr int perm32(int i) { return 16 * ((i >> 2) & 1) + ((i >> 3) << 2) + (i & 3); }

// one element rounded to T, as its 16 bits
template <typename T> __device__ __forceinline__ unsigned short bits16(float x)
{
    return (unsigned short)(Elem<T>::pack2(x, 0.f) & 0xffffu);
}

// 4-byte-per-lane buffer load into LDS: lane i writes dst + 4 i
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t rs, lds_void *dst, unsigned voffset)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voffset, 0, 0, 0);
#endif
}

typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// s_waitcnt vmcnt(0): every load (and store) this wave issued has completed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, long long bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)(bytes > 0 ? bytes : 0), 0x00020000);
}

// ----------------------------------------------------------------- KKT solve

struct KktParams {
    const void *k;
    const float *g, *beta;
    void *A;
    int B, T, Hqk, Hv, n_chunks;
};

template <typename T>
__global__ __launch_bounds__(256) void kkt_kernel(KktParams p)
{
    constexpr int KP = 17 * 16;  // K row pitch in bytes: odd units, conflict-free 16-byte row reads
    constexpr int LP = 68;       // L row pitch in floats
    __shared__ __attribute__((aligned(16))) unsigned char kt_raw[C * KP];
    __shared__ __attribute__((aligned(16))) float L[C * LP];
    __shared__ float X[C * (C + 1)];  // the inverse, X[t][j] at t * (C + 1) + j
    __shared__ float gs[C], bs[C];
    lds_u8 *kt = (lds_u8 *)kt_raw;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = (int)(blockIdx.x % p.n_chunks);
    const long long bh = blockIdx.x / p.n_chunks;
    const int b = (int)(bh / p.Hv), h = (int)(bh % p.Hv), hk = h / (p.Hv / p.Hqk);
    const int t0 = c * C, n = p.T - t0 < C ? p.T - t0 : C;

    for (int i = tid; i < C * (DK / 8); i += 256) {  // 64 rows x 16 units; rows past n are zero
        const int r = i >> 4, u = i & 15;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < n) v = *(const u32x4 *)((const T *)p.k + (((size_t)b * p.T + t0 + r) * p.Hqk + hk) * DK + u * 8);
        *(lds_u32x4 *)(kt + r * KP + u * 16) = v;
    }
    if (tid < C) {
        const size_t idx = ((size_t)b * p.T + t0 + tid) * p.Hv + h;
        gs[tid] = tid < n ? p.g[idx] : 0.f;
        bs[tid] = tid < n ? p.beta[idx] : 0.f;
    }
    __syncthreads();

    // K K^T: wave w computes the 32x32 block (rows t in 32 tb, columns s in 32 sb)
    {
        const int tb = wave >> 1, sb = wave & 1, ql = lane & 31, hh = lane >> 5;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) {
            const u32x4 a = *(const lds_u32x4 *)(kt + (32 * tb + ql) * KP + (2 * ks + hh) * 16);
            const u32x4 bb = *(const lds_u32x4 *)(kt + (32 * sb + ql) * KP + (2 * ks + hh) * 16);
            acc = Elem<T>::mfma(a, bb, acc);
        }
        const int s = 32 * sb + ql;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 32 * tb + 8 * (r >> 2) + 4 * hh + (r & 3);
            L[t * LP + s] = (s < t && t < n) ? bs[t] * acc[r] * exp_(gs[t] - gs[s]) : 0.f;
        }
    }
    __syncthreads();

    // (I + L) X = I, one lane per column j: X_tj = [t == j] - sum_{s < t} L_ts X_sj.  A lane reads
    // only its own column of X (and L rows broadcast), so one wave needs no barrier.  L's row t
    // is zero from column t on, so the sum runs over whole groups of 4.
    if (wave == 0) {
        const int j = lane;
        for (int t = 0; t < C; ++t) {
            float x = t == j ? 1.f : 0.f;
            for (int s4 = 0; s4 < t; s4 += 4) {
                const f32x4 l4 = *(const f32x4 *)(L + t * LP + s4);
#pragma unroll
                for (int e = 0; e < 4; ++e) x = __builtin_fmaf(-l4[e], X[(s4 + e) * (C + 1) + j], x);
            }
            X[t * (C + 1) + j] = x;
        }
        unsigned short *out = (unsigned short *)p.A;
        for (int t = 0; t < n; ++t) out[(((size_t)b * p.T + t0 + t) * p.Hv + h) * C + j] = bits16<T>(X[t * (C + 1) + j]);
    }
}

// ---------------------------------------------------------------- chunk kernel

struct ChunkParams {
    const void *q, *k, *v;
    const float *g, *beta;
    const void *A;
    const float *s0;  // may be null
    void *o;
    float *s_final;
    // two-kernel mode: the state at each chunk start, [B*Hv][chunks][DV][DK] (dtype), and
    // V_new, [B*Hv][chunks][DV][64] (dtype), both transposed (state column / value column major)
    void *ws_st, *ws_vn;
    // segmented mode: the chunks form runs of seg_chunks (the last may be shorter), n_seg of them
    // in the launch.  The transition walk's end state [M | Z] of each run but the last: ws_m
    // holds M, [B*Hv][runs - 1][DK / 4][DK][4] fp32 (4-column groups, each column group's rows
    // contiguous), ws_z holds Z, [B*Hv][runs - 1][DK][DV] fp32; ws_start the start state of each
    // run but the first, [B*Hv][runs - 1][DK][DV] fp32.
    float *ws_m, *ws_z, *ws_start;
    int B, T, Hqk, Hv, DV, n_chunks, dv_blocks, n_seg, seg_chunks;
    float scale;
};

// What a chunk walk computes.  WALK_FULL: state and outputs.  WALK_STATE: only the sequential
// part -- U', W', V_new and the state update -- storing each chunk's starting state and V_new
// for out_kernel.  WALK_TRANSITION: the state part over one run of chunks, with the state
// widened to DK + DV columns: the first DK start as the identity and see zero values, the
// others start at zero and see the run's values, so the end state is [M | Z] with M the run's
// linear map of the state and Z its end state from zero (the recurrence is linear in the state
// and each state column evolves on its own).
constexpr int WALK_FULL = 0, WALK_STATE = 1, WALK_TRANSITION = 2;

// One workgroup per (b, value head, run of chunks, 64 state columns) walks its run in order.
template <typename T, int MODE>
__global__ __launch_bounds__(256, 1) void chunk_kernel(ChunkParams p)
{
    constexpr bool SPLIT = MODE != WALK_FULL;  // no Q tile, no outputs
    // LDS: two input buffers [Q | K | A | g | beta | V] and the per-chunk work arrays
    constexpr int QK_TILE = C * DK * 2;        // swizzled, 256-byte rows
    constexpr int AP = 9 * 16;                 // A / work-array pitch in bytes (64 elements + pad)
    constexpr int A_TILE = C * AP;
    constexpr int OFF_V = 2 * QK_TILE + A_TILE + 2 * 256;  // the chunk's V block, laid out as A
    constexpr int BUF = OFF_V + A_TILE;
    constexpr int SP = 17 * 16;                // St pitch: 128 elements + pad
    constexpr int OFF_ST = 2 * BUF, OFF_WT = OFF_ST + DVB * SP, OFF_SC = OFF_WT + DVB * AP,
                  OFF_VN = OFF_SC + C * AP, OFF_VH = OFF_VN + DVB * AP, SMEM = OFF_VH + DVB * AP;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM];
    lds_u8 *smem = (lds_u8 *)smem_raw;
    lds_u8 *st = smem + OFF_ST, *wt = smem + OFF_WT, *sc = smem + OFF_SC, *vn = smem + OFF_VN,
           *vh = smem + OFF_VH;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ql = lane & 31, hh = lane >> 5;
    const int tb = wave >> 1, cb = wave & 1;  // this wave's 32x32 output block of the chunk products
    const int dvblk = (int)(blockIdx.x % p.dv_blocks);
    const long long rest = blockIdx.x / p.dv_blocks;
    const int seg = (int)(rest % p.n_seg);
    const long long bh = rest / p.n_seg;
    const int b = (int)(bh / p.Hv), h = (int)(bh % p.Hv), hk = h / (p.Hv / p.Hqk);
    // transition walk: column blocks below DK / DVB are the identity's columns (no values read)
    const bool ident = MODE == WALK_TRANSITION && dvblk < DK / DVB;
    const int dv0 = MODE == WALK_TRANSITION ? (ident ? 0 : dvblk * DVB - DK) : dvblk * DVB;
    const int c_begin = seg * p.seg_chunks, c_end = min(p.n_chunks, c_begin + p.seg_chunks);
    const int T_ = p.T, Hv = p.Hv, DV = p.DV;
    const long long qk_rs = (long long)p.Hqk * DK * sizeof(T);  // row stride of q / k in bytes
    const long long a_rs = (long long)Hv * C * sizeof(T);
    const T *qbase = (const T *)p.q + ((size_t)b * T_ * p.Hqk + hk) * DK;
    const T *kbase = (const T *)p.k + ((size_t)b * T_ * p.Hqk + hk) * DK;
    const T *abase = (const T *)p.A + ((size_t)b * T_ * Hv + h) * C;
    const float *gbase = p.g + (size_t)b * T_ * Hv + h, *bbase = p.beta + (size_t)b * T_ * Hv + h;

    // per-lane source offsets of the tile copies (see the 1 KiB-per-instruction layout notes in
    // the backward kernels): Q/K instruction j = wave + 4 i fills rows 4 j .. 4 j + 3
    const int qk_row = 4 * wave + (lane >> 4), qk_phys = lane & 15;
    const unsigned qk_src = (unsigned)(qk_row * qk_rs + ((qk_phys ^ swz<DK>(qk_row)) * 16));
    // V block of the chunk (its 64 tokens by this workgroup's 64 state columns): the same layout
    // and copy pattern as A, a token's row being v_rs bytes after the previous one
    const long long v_rs = (long long)Hv * DV * sizeof(T);
    unsigned a_src[3], v_src[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {  // A instruction j = wave + 4 i (< 9) fills units 64 j .. 64 j + 63
        const int u = (wave + 4 * i) * 64 + lane, row = u / 9, unit = u % 9;
        a_src[i] = unit < 8 && row < C ? (unsigned)(row * a_rs + unit * 16) : 0x7fffff00u;
        v_src[i] = unit < 8 && row < C ? (unsigned)(row * v_rs + unit * 16) : 0x7fffff00u;
    }
    auto issue = [&](int c, int buf) {
        const int t0 = c * C, n = T_ - t0 < C ? T_ - t0 : C;
        lds_u8 *dst = smem + buf * BUF;
        const __amdgpu_buffer_rsrc_t rq = rsrc(qbase + (size_t)t0 * p.Hqk * DK, (n - 1) * qk_rs + DK * sizeof(T));
        const __amdgpu_buffer_rsrc_t rk = rsrc(kbase + (size_t)t0 * p.Hqk * DK, (n - 1) * qk_rs + DK * sizeof(T));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned off = qk_src + (unsigned)(16 * i * qk_rs);
            if constexpr (!SPLIT) lds_load16(rq, (lds_void *)(dst + (wave + 4 * i) * 1024), off);
            lds_load16(rk, (lds_void *)(dst + QK_TILE + (wave + 4 * i) * 1024), off);
        }
        const __amdgpu_buffer_rsrc_t ra = rsrc(abase + (size_t)t0 * Hv * C, (n - 1) * a_rs + C * sizeof(T));
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (wave + 4 * i < 9) lds_load16(ra, (lds_void *)(dst + 2 * QK_TILE + (wave + 4 * i) * 1024), a_src[i]);
        // tokens past the sequence read as zero (the range ends at the chunk's last token)
        if (!ident) {
            const __amdgpu_buffer_rsrc_t rv = rsrc((const T *)p.v + (((size_t)b * T_ + t0) * Hv + h) * DV + dv0,
                                                   (n - 1) * v_rs + DVB * (long long)sizeof(T));
#pragma unroll
            for (int i = 0; i < 3; ++i)
                if (wave + 4 * i < 9) lds_load16(rv, (lds_void *)(dst + OFF_V + (wave + 4 * i) * 1024), v_src[i]);
        }
        if (wave < 2) {  // g (wave 0) and beta (wave 1): 64 floats, one per lane
            const float *src = (wave == 0 ? gbase : bbase) + (size_t)t0 * Hv;
            lds_load4(rsrc(src, (long long)(n - 1) * Hv * 4 + 4), (lds_void *)(dst + 2 * QK_TILE + A_TILE + wave * 256),
                      (unsigned)(lane * Hv * 4));
        }
    };
    // state: wave w owns state rows (key dims) 32 w .. 32 w + 31 for both 32-column blocks j;
    // accumulator register r of half hh is row 32 w + 16 hh + r (the transposing read's order).
    // It starts as s0 (or zero) for the first run of chunks and as the combined start state for
    // a later one; the transition walk starts from [I | 0].
    const float *s_in = seg == 0 ? (p.s0 ? p.s0 + (size_t)bh * DK * DV : nullptr)
                                 : p.ws_start + ((size_t)bh * (p.n_seg - 1) + seg - 1) * DK * DV;
    f32x16 S[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = 32 * wave + 16 * hh + r, e = dv0 + 32 * j + ql;
            if constexpr (MODE == WALK_TRANSITION)
                S[j][r] = ident && d == dvblk * DVB + 32 * j + ql ? 1.f : 0.f;
            else
                S[j][r] = s_in ? s_in[(size_t)d * DV + e] : 0.f;
        }
    // bf16 copy of the state, transposed: St[column][key dim], 16 consecutive key dims per lane
    auto write_st = [&]() {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 w0, w1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                w0[r] = Elem<T>::pack2(S[j][2 * r], S[j][2 * r + 1]);
                w1[r] = Elem<T>::pack2(S[j][8 + 2 * r], S[j][8 + 2 * r + 1]);
            }
            lds_u8 *dst = st + (32 * j + ql) * SP + (32 * wave + 16 * hh) * 2;
            *(lds_u32x4 *)dst = w0;
            *(lds_u32x4 *)(dst + 16) = w1;
        }
    };
    // Two-kernel mode: the chunk's starting state and V_new go to the workspace from their LDS
    // copies (St, and V_new staged in vn), each wave storing whole rows -- 16 bytes a lane, a
    // column's 256 (St) or 128 (V_new) contiguous bytes per 16 or 8 lanes -- rather than the
    // 16- and 8-byte pieces of many rows a lane holds in registers.  The state goes out at the
    // top of the chunk, once the next chunk's loads have been issued.
    auto store_st = [&](int cidx) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = 16 * wave + 4 * i + (lane >> 4), unit = lane & 15;
            const u32x4 x = *(const lds_u32x4 *)(st + col * SP + unit * 16);
            *(u32x4 *)((T *)p.ws_st + (((size_t)bh * p.n_chunks + cidx) * DV + dv0 + col) * DK + unit * 8) = x;
        }
    };
    auto store_vn = [&](int cidx) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int col = 16 * wave + 8 * i + (lane >> 3), unit = lane & 7;
            const u32x4 x = *(const lds_u32x4 *)(vn + col * AP + unit * 16);
            *(u32x4 *)((T *)p.ws_vn + (((size_t)bh * p.n_chunks + cidx) * DV + dv0 + col) * C + unit * 8) = x;
        }
    };
    // 8-byte transposed write: 4 accumulator rows (registers 4 q .. 4 q + 3) of column `col`
    auto put4 = [&](lds_u8 *arr, int pitch, int col, int row0, float x0, float x1, float x2, float x3) {
        u32x2 w;
        w[0] = Elem<T>::pack2(x0, x1);
        w[1] = Elem<T>::pack2(x2, x3);
        *(__attribute__((address_space(3))) u32x2 *)(arr + col * pitch + row0 * 2) = w;
    };
    auto row16 = [&](const lds_u8 *arr, int pitch, int row, int unit) {
        return *(const lds_u32x4 *)(arr + row * pitch + unit * 16);
    };

    // transposing-read offsets of K for this wave's 32 key dims (column block `wave`)
    const unsigned tr_lo = tr_off<DK>(lane, wave, 0), tr_hi = tr_off<DK>(lane, wave, 1);
    const float scale = p.scale;
    issue(c_begin, 0);
    write_st();
    wait_vm0();
    __syncthreads();

    for (int c = c_begin; c < c_end; ++c) {
        const int buf = (c - c_begin) & 1, t0 = c * C, n = T_ - t0 < C ? T_ - t0 : C;
        if (c + 1 < c_end) issue(c + 1, buf ^ 1);
        if constexpr (MODE == WALK_STATE) store_st(c);
        const lds_u8 *qt = smem + buf * BUF, *kt = qt + QK_TILE, *at = kt + QK_TILE;
        const lds_f32 *gl = (const lds_f32 *)(at + A_TILE), *bl = gl + C;
        const lds_u8 *vt = qt + OFF_V;

        // ---- U' = K S_c, Q S_c and K Q^T (this wave's blocks)
        // The output is computed transposed, O^T = S^T Q^T (+ V_new^T scores^T below), with the
        // state's rows read in perm32 order: lane (t = 32 tb + ql, hh) then holds the 16
        // consecutive columns 32 cb + 16 hh .. + 15 of its token and stores them as 32 bytes.
        f32x16 U, O, KQ;
#pragma unroll
        for (int r = 0; r < 16; ++r) U[r] = O[r] = KQ[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) {
            const int u = 2 * ks + hh;
            const u32x4 sb = row16(st, SP, 32 * cb + ql, u);
            const u32x4 ka = read_row<DK>(kt, 32 * tb + ql, u);
            U = Elem<T>::mfma(ka, sb, U);
            if constexpr (!SPLIT) {
                const u32x4 qa = read_row<DK>(qt, 32 * tb + ql, u);
                O = Elem<T>::mfma(row16(st, SP, 32 * cb + perm32(ql), u), qa, O);
                KQ = Elem<T>::mfma(ka, read_row<DK>(qt, 32 * cb + ql, u), KQ);
            }
        }
        if constexpr (!SPLIT) {
            const float eg = exp_(gl[32 * tb + ql]);  // O^T column t = 32 tb + ql
#pragma unroll
            for (int r = 0; r < 16; ++r) O[r] *= eg;
        }
        // rows t (or s) = 32 tb + 8 q + 4 hh + e; columns dv (or t) = 32 cb + ql
        const float g_col = gl[32 * cb + ql];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r0 = 32 * tb + 8 * q + 4 * hh;
            const f32x4 g4 = *(const lds_f32x4 *)(gl + r0), b4 = *(const lds_f32x4 *)(bl + r0);
            float w[4], s4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q + e;
                const float eg = exp_(g4[e]);
                const f32x2 vv = Elem<T>::unpack2(
                    *(const __attribute__((address_space(3))) unsigned short *)(vt + (r0 + e) * AP + (32 * cb + ql) * 2));
                w[e] = b4[e] * ((ident ? 0.f : vv[0]) - eg * U[r]);
                // scores[t][s] for t = column, s = row: causal and gate-decayed
                if constexpr (!SPLIT) s4[e] = r0 + e <= 32 * cb + ql ? KQ[r] * exp_(g_col - g4[e]) : 0.f;
            }
            put4(wt, AP, 32 * cb + ql, r0, w[0], w[1], w[2], w[3]);
            if constexpr (!SPLIT) put4(sc, AP, 32 * cb + ql, r0, s4[0], s4[1], s4[2], s4[3]);
        }
        __syncthreads();

        // ---- V_new = A W'
        f32x16 V;
#pragma unroll
        for (int r = 0; r < 16; ++r) V[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
            V = Elem<T>::mfma(row16(at, AP, 32 * tb + ql, 2 * ks + hh), row16(wt, AP, 32 * cb + ql, 2 * ks + hh), V);
        const float g_last = gl[n - 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r0 = 32 * tb + 8 * q + 4 * hh;
            const f32x4 g4 = *(const lds_f32x4 *)(gl + r0);
            if constexpr (MODE != WALK_TRANSITION)  // V_new^T, for the outputs
                put4(vn, AP, 32 * cb + ql, r0, V[4 * q], V[4 * q + 1], V[4 * q + 2], V[4 * q + 3]);
            // decayed copy for the state update, positions with bits 2 and 3 of s swapped so that
            // the 8 rows one transposing K read pairs with are 16 contiguous bytes
            const int p0 = 32 * tb + 16 * (q >> 1) + 8 * hh + 4 * (q & 1);
            put4(vh, AP, 32 * cb + ql, p0, V[4 * q] * exp_(g_last - g4[0]), V[4 * q + 1] * exp_(g_last - g4[1]),
                 V[4 * q + 2] * exp_(g_last - g4[2]), V[4 * q + 3] * exp_(g_last - g4[3]));
        }
        __syncthreads();

        if constexpr (MODE == WALK_STATE) store_vn(c);
        // ---- O = scale (exp(g) Q S_c + scores V_new)
        if constexpr (!SPLIT) {
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
            O = Elem<T>::mfma(row16(vn, AP, 32 * cb + perm32(ql), 2 * ks + hh), row16(sc, AP, 32 * tb + ql, 2 * ks + hh),
                              O);
        if (32 * tb + ql < n) {
            u32x4 w0, w1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                w0[r] = Elem<T>::pack2(O[2 * r] * scale, O[2 * r + 1] * scale);
                w1[r] = Elem<T>::pack2(O[8 + 2 * r] * scale, O[8 + 2 * r + 1] * scale);
            }
            u32x4 *dst = (u32x4 *)((T *)p.o + (((size_t)b * T_ + t0 + 32 * tb + ql) * Hv + h) * DV + dv0 + 32 * cb +
                                   16 * hh);
            dst[0] = w0;
            dst[1] = w1;
        }
        }
        // ---- S_{c+1} = exp(g_last) S_c + K^T (exp(g_last - g) V_new)
        const float decay = exp_(g_last);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) S[j][r] *= decay;
#pragma unroll
            for (int sblk = 0; sblk < 2; ++sblk)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const u32x4 a = read_tr_at<DK>(kt, 32 * sblk + 16 * tt, tr_lo, tr_hi);
                    const u32x4 bv = *(const lds_u32x4 *)(vh + (32 * j + ql) * AP + (32 * sblk + 16 * tt + 8 * hh) * 2);
                    S[j] = Elem<T>::mfma(a, bv, S[j]);
                }
        }
        // No barrier before the state's operand copy is rewritten: St is read only by the first
        // phase, which every wave finished before the first barrier of this chunk, and the work
        // arrays written in the next chunk are read here only before the barrier that ends it.
        write_st();
        wait_vm0();       // the next chunk's tiles (and this chunk's output stores) have landed
        __syncthreads();
    }
    if constexpr (MODE == WALK_TRANSITION) {
        if (ident) {
            float *dst = p.ws_m + ((size_t)bh * p.n_seg + seg) * DK * DK;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int col = dvblk * DVB + 32 * j + ql;
                    dst[((col >> 2) * DK + 32 * wave + 16 * hh + r) * 4 + (col & 3)] = S[j][r];
                }
        } else {
            float *dst = p.ws_z + ((size_t)bh * p.n_seg + seg) * DK * DV;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dst[(size_t)(32 * wave + 16 * hh + r) * DV + dv0 + 32 * j + ql] = S[j][r];
        }
    } else if (seg == p.n_seg - 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = 32 * wave + 16 * hh + r, e = dv0 + 32 * j + ql;
                p.s_final[((size_t)bh * DK + d) * DV + e] = S[j][r];
            }
    }
}

// Start states of the later runs of chunks in the segmented mode.  With run r's end state from
// the transition walk, [M_r | Z_r],
//     S_{r+1} = M_r S_r + Z_r,   S_0 = s0 (or zero),
// in fp32: Z first, then the products over the key dim in ascending order.  One workgroup (8
// waves) per (b, value head, 8 state columns); thread (d, quad) forms columns 2 quad and
// 2 quad + 1 of state row d.  Only S is carried from run to run: M_{r+1} (64 KiB) is copied into
// the other half of a double-buffered LDS area by buffer-to-LDS loads while run r's product
// reads M_r, and lane l of a wave then reads row 32 w + l / 2's 4-column group, 512 contiguous
// bytes a wave.
struct CombineParams {
    const float *m, *z, *s0;
    float *start;
    int n_runs;  // transition walks: the runs of chunks but the last
    int DV;
};

__global__ __launch_bounds__(512) void combine_kernel(CombineParams p)
{
    __shared__ __attribute__((aligned(16))) float m_raw[2 * DK * DK];
    __shared__ __attribute__((aligned(16))) float s_raw[DK * 8];
    lds_f32 *Ml = (lds_f32 *)m_raw, *Sl = (lds_f32 *)s_raw;
    typedef __attribute__((address_space(3))) f32x2 lds_f32x2;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int d = tid >> 2, e2 = 2 * (tid & 3);
    const int DV = p.DV, eblocks = DV / 8;
    const int e0 = (int)(blockIdx.x % eblocks) * 8 + e2;
    const long long bh = blockIdx.x / eblocks;
    auto issue = [&](int r, int buf) {  // instruction i = wave + 8 k copies bytes 1024 i .. 1024 i + 1023
        const __amdgpu_buffer_rsrc_t rs = rsrc(p.m + ((size_t)bh * p.n_runs + r) * DK * DK, DK * DK * 4);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = wave + 8 * k;
            lds_load16(rs, (lds_void *)(Ml + buf * DK * DK + i * 256), (unsigned)(i * 1024 + 16 * lane));
        }
    };
    auto load_z = [&](int r) { return *(const f32x2 *)(p.z + (((size_t)bh * p.n_runs + r) * DK + d) * DV + e0); };
#pragma unroll
    for (int i = 0; i < 2; ++i) Sl[d * 8 + e2 + i] = p.s0 ? p.s0[((size_t)bh * DK + d) * DV + e0 + i] : 0.f;
    issue(0, 0);
    f32x2 z = load_z(0);
    wait_vm0();
    __syncthreads();
    for (int r = 0; r < p.n_runs; ++r) {
        const int buf = r & 1;
        f32x2 zn = {0.f, 0.f};
        if (r + 1 < p.n_runs) {
            issue(r + 1, buf ^ 1);
            zn = load_z(r + 1);
        }
        const lds_f32 *mr = Ml + buf * DK * DK;
        f32x2 acc = z;
#pragma unroll
        for (int j = 0; j < DK / 4; ++j) {
            const f32x4 mv = *(const lds_f32x4 *)(mr + (j * DK + d) * 4);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x2 sv = *(const lds_f32x2 *)(Sl + (4 * j + jj) * 8 + e2);
                acc[0] = __builtin_fmaf(mv[jj], sv[0], acc[0]);
                acc[1] = __builtin_fmaf(mv[jj], sv[1], acc[1]);
            }
        }
        __syncthreads();  // every thread has read this run's S and M
        *(lds_f32x2 *)(Sl + d * 8 + e2) = acc;
        *(f32x2 *)(p.start + (((size_t)bh * p.n_runs + r) * DK + d) * DV + e0) = acc;
        wait_vm0();       // M_{r+1} and Z_{r+1} have landed
        __syncthreads();
        z = zn;
    }
}

// Outputs of the two-kernel mode: one workgroup per (b, value head, chunk, 64 value columns),
// all independent.  With the chunk's starting state S_c and V_new from chunk_kernel<T, WALK_STATE>,
//     O = scale (exp(g) (Q S_c) + scores V_new)
// by the same products, in the same order and on the same rounded operands as the fused
// kernel (so both modes give identical bits): O^T = S_c^T Q^T, scaled by exp(g) per token,
// then += V_new^T scores^T.
template <typename T>
__global__ __launch_bounds__(256, 2) void out_kernel(ChunkParams p)
{
    constexpr int TILE = C * DK * 2;  // Q, K and S_c^T tiles: swizzled 256-byte rows
    constexpr int AP = 9 * 16;        // V_new^T and scores pitch in bytes (64 elements + pad)
    constexpr int OFF_K = TILE, OFF_S = 2 * TILE, OFF_VN = 3 * TILE, OFF_SC = OFF_VN + DVB * AP,
                  OFF_G = OFF_SC + C * AP, SMEM = OFF_G + 256;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM];
    lds_u8 *smem = (lds_u8 *)smem_raw;
    const lds_u8 *qt = smem, *kt = smem + OFF_K, *stl = smem + OFF_S, *vnl = smem + OFF_VN;
    lds_u8 *sc = smem + OFF_SC;
    const lds_f32 *gl = (const lds_f32 *)(smem + OFF_G);

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ql = lane & 31, hh = lane >> 5;
    const int tb = wave >> 1, cb = wave & 1;  // this wave's 32x32 output block
    const int dvblk = (int)(blockIdx.x % p.dv_blocks);
    const long long rest = blockIdx.x / p.dv_blocks;
    const int c = (int)(rest % p.n_chunks);
    const long long bh = rest / p.n_chunks;
    const int b = (int)(bh / p.Hv), h = (int)(bh % p.Hv), hk = h / (p.Hv / p.Hqk);
    const int dv0 = dvblk * DVB, T_ = p.T, Hv = p.Hv, DV = p.DV;
    const int t0 = c * C, n = T_ - t0 < C ? T_ - t0 : C;

    // tile copies: Q, K and S_c^T (64 rows of 128 elements each, swizzled as the fused kernel's
    // Q/K tiles), V_new^T (64 rows of 64 elements, one pad unit per row) and g (64 floats)
    const long long qk_rs = (long long)p.Hqk * DK * sizeof(T);
    const int row = 4 * wave + (lane >> 4), phys = lane & 15;
    const unsigned src_qk = (unsigned)(row * qk_rs + ((phys ^ swz<DK>(row)) * 16));
    const unsigned src_st = (unsigned)(row * (DK * (int)sizeof(T)) + ((phys ^ swz<DK>(row)) * 16));
    const T *qb = (const T *)p.q + (((size_t)b * T_ + t0) * p.Hqk + hk) * DK;
    const T *kb = (const T *)p.k + (((size_t)b * T_ + t0) * p.Hqk + hk) * DK;
    const T *sb = (const T *)p.ws_st + (((size_t)bh * p.n_chunks + c) * DV + dv0) * DK;
    const T *vb = (const T *)p.ws_vn + (((size_t)bh * p.n_chunks + c) * DV + dv0) * C;
    const __amdgpu_buffer_rsrc_t rq = rsrc(qb, (n - 1) * qk_rs + DK * sizeof(T));
    const __amdgpu_buffer_rsrc_t rk = rsrc(kb, (n - 1) * qk_rs + DK * sizeof(T));
    const __amdgpu_buffer_rsrc_t rs = rsrc(sb, (long long)DVB * DK * sizeof(T));
    const __amdgpu_buffer_rsrc_t rv = rsrc(vb, (long long)DVB * C * sizeof(T));
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // instruction j = wave + 4 i fills rows 4 j .. 4 j + 3
        lds_load16(rq, (lds_void *)(smem + (wave + 4 * i) * 1024), src_qk + (unsigned)(16 * i * qk_rs));
        lds_load16(rk, (lds_void *)(smem + OFF_K + (wave + 4 * i) * 1024), src_qk + (unsigned)(16 * i * qk_rs));
        lds_load16(rs, (lds_void *)(smem + OFF_S + (wave + 4 * i) * 1024), src_st + (unsigned)(16 * i * DK * sizeof(T)));
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {  // instruction j = wave + 4 i (< 9) fills units 64 j .. 64 j + 63
        const int u = (wave + 4 * i) * 64 + lane, r = u / 9, unit = u % 9;
        const unsigned off = unit < 8 && r < DVB ? (unsigned)(r * C * sizeof(T) + unit * 16) : 0x7fffff00u;
        if (wave + 4 * i < 9) lds_load16(rv, (lds_void *)(smem + OFF_VN + (wave + 4 * i) * 1024), off);
    }
    if (wave == 0)
        lds_load4(rsrc(p.g + ((size_t)b * T_ + t0) * Hv + h, (long long)(n - 1) * Hv * 4 + 4),
                  (lds_void *)(smem + OFF_G), (unsigned)(lane * Hv * 4));
    wait_vm0();
    __syncthreads();

    auto row16 = [&](const lds_u8 *arr, int pitch, int r, int unit) {
        return *(const lds_u32x4 *)(arr + r * pitch + unit * 16);
    };
    // O^T = S_c^T Q^T and K Q^T, this wave's blocks (rows of S_c^T read in perm32 order, as in
    // the fused kernel, so that lane (t = 32 tb + ql, hh) holds 16 consecutive columns)
    f32x16 O, KQ;
#pragma unroll
    for (int r = 0; r < 16; ++r) O[r] = KQ[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) {
        const int u = 2 * ks + hh;
        const u32x4 ka = read_row<DK>(kt, 32 * tb + ql, u);
        const u32x4 qa = read_row<DK>(qt, 32 * tb + ql, u);
        O = Elem<T>::mfma(read_row<DK>(stl, 32 * cb + perm32(ql), u), qa, O);
        KQ = Elem<T>::mfma(ka, read_row<DK>(qt, 32 * cb + ql, u), KQ);
    }
    {
        const float eg = exp_(gl[32 * tb + ql]);
#pragma unroll
        for (int r = 0; r < 16; ++r) O[r] *= eg;
    }
    // scores, transposed into LDS: rows s = 32 tb + 8 q + 4 hh + e, column t = 32 cb + ql
    const float g_col = gl[32 * cb + ql];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r0 = 32 * tb + 8 * q + 4 * hh;
        const f32x4 g4 = *(const lds_f32x4 *)(gl + r0);
        float s4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s4[e] = r0 + e <= 32 * cb + ql ? KQ[4 * q + e] * exp_(g_col - g4[e]) : 0.f;
        u32x2 w;
        w[0] = Elem<T>::pack2(s4[0], s4[1]);
        w[1] = Elem<T>::pack2(s4[2], s4[3]);
        *(__attribute__((address_space(3))) u32x2 *)(sc + (32 * cb + ql) * AP + r0 * 2) = w;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks)
        O = Elem<T>::mfma(row16(vnl, AP, 32 * cb + perm32(ql), 2 * ks + hh), row16(sc, AP, 32 * tb + ql, 2 * ks + hh), O);
    if (32 * tb + ql < n) {
        const float scale = p.scale;
        u32x4 w0, w1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w0[r] = Elem<T>::pack2(O[2 * r] * scale, O[2 * r + 1] * scale);
            w1[r] = Elem<T>::pack2(O[8 + 2 * r] * scale, O[8 + 2 * r + 1] * scale);
        }
        u32x4 *dst = (u32x4 *)((T *)p.o + (((size_t)b * T_ + t0 + 32 * tb + ql) * Hv + h) * DV + dv0 + 32 * cb + 16 * hh);
        dst[0] = w0;
        dst[1] = w1;
    }
}

}  // namespace gdn
}  // namespace fa

extern "C" {

int gdn_kkt(const void *k, const float *g, const float *beta, void *A, int B, int T, int Hqk, int Hv, int DK,
            int dtype, void *stream)
{
    if (!k || !g || !beta || !A || B <= 0 || T <= 0 || Hqk <= 0 || Hv <= 0 || DK <= 0) return FA_ERR_INVALID_ARG;
    if (Hv % Hqk != 0 || (dtype != FA_F16 && dtype != FA_BF16)) return FA_ERR_INVALID_ARG;
    if (DK != fa::gdn::DK) return FA_ERR_UNSUPPORTED;
    if (((uintptr_t)k | (uintptr_t)A) & 15u) return FA_ERR_UNSUPPORTED;
    fa::gdn::KktParams p;
    p.k = k;
    p.g = g;
    p.beta = beta;
    p.A = A;
    p.B = B;
    p.T = T;
    p.Hqk = Hqk;
    p.Hv = Hv;
    p.n_chunks = (T + fa::gdn::C - 1) / fa::gdn::C;
    const long long grid = (long long)B * Hv * p.n_chunks;
    if (grid > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == FA_F16)
        hipLaunchKernelGGL((fa::gdn::kkt_kernel<_Float16>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((fa::gdn::kkt_kernel<__bf16>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// bytes of the two-kernel workspace: the chunk states (256-byte aligned end), then V_new
static size_t ws_states_bytes(int B, int T, int Hv, int DV)
{
    const size_t chunks = (size_t)B * Hv * ((T + fa::gdn::C - 1) / fa::gdn::C);
    return (chunks * DV * fa::gdn::DK * 2 + 255) & ~(size_t)255;
}

size_t gdn_chunk_workspace_size(int B, int T, int Hv, int DV)
{
    if (B <= 0 || T <= 0 || Hv <= 0 || DV <= 0) return 0;
    const size_t chunks = (size_t)B * Hv * ((T + fa::gdn::C - 1) / fa::gdn::C);
    return ws_states_bytes(B, T, Hv, DV) + chunks * DV * fa::gdn::C * 2;
}

// The two-kernel mode pays for a round trip of every chunk's state and V_new through HBM and
// an extra launch, and gains a shorter sequential step; it wins when the state walk leaves most
// CUs idle.  Rule: state-walk workgroups (B * Hv * DV / 64) at most a quarter of the 256 CUs
// (measured: 6 % faster to 8 % slower at 64 walkers, 34 % slower at 128).
int gdn_chunk_plan(int B, int T, int Hv, int DV, size_t *workspace_bytes)
{
    if (!workspace_bytes) return FA_ERR_INVALID_ARG;
    *workspace_bytes = 0;
    if (B <= 0 || T <= 0 || Hv <= 0 || DV <= 0) return FA_ERR_INVALID_ARG;
    if (DV % fa::gdn::DVB != 0) return FA_ERR_UNSUPPORTED;
    const long long walkers = (long long)B * Hv * (DV / fa::gdn::DVB);
    if (walkers <= 64) *workspace_bytes = gdn_chunk_workspace_size(B, T, Hv, DV);
    return FA_OK;
}

}  // extern "C"

// Argument checks shared by the chunk-recurrence entry points (before any HIP call).
static int check_chunk_args(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const void *A, const float *s0, const void *o, const float *s_final, int B, int T, int Hqk,
                            int Hv, int DK, int DV, float scale, int dtype)
{
    if (!q || !k || !v || !g || !beta || !A || !o || !s_final) return FA_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0 || Hqk <= 0 || Hv <= 0 || DK <= 0 || DV <= 0 || Hv % Hqk != 0) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale) || (dtype != FA_F16 && dtype != FA_BF16)) return FA_ERR_INVALID_ARG;
    if (DK != fa::gdn::DK || DV % fa::gdn::DVB != 0) return FA_ERR_UNSUPPORTED;
    // V is read with 32-bit offsets over one 64-token chunk of [B, T, Hv, DV] rows
    if ((long long)Hv * DV * 2 * fa::gdn::C > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)A | (uintptr_t)o |
                         (uintptr_t)s_final | (uintptr_t)s0 | (uintptr_t)g | (uintptr_t)beta;
    if (al & 15u) return FA_ERR_UNSUPPORTED;
    // tile copies use 32-bit offsets inside one chunk: 63 rows of q/k, A, g and beta
    if ((long long)Hqk * fa::gdn::DK * 2 * 64 > 0x7fff0000LL || (long long)Hv * 64 * 2 * 64 > 0x7fff0000LL)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

static fa::gdn::ChunkParams chunk_params(const void *q, const void *k, const void *v, const float *g,
                                         const float *beta, const void *A, const float *s0, void *o, float *s_final,
                                         int B, int T, int Hqk, int Hv, int DV, float scale)
{
    fa::gdn::ChunkParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.A = A;
    p.s0 = s0;
    p.o = o;
    p.s_final = s_final;
    p.B = B;
    p.T = T;
    p.Hqk = Hqk;
    p.Hv = Hv;
    p.DV = DV;
    p.n_chunks = (T + fa::gdn::C - 1) / fa::gdn::C;
    p.dv_blocks = DV / fa::gdn::DVB;
    p.n_seg = 1;
    p.seg_chunks = p.n_chunks;
    p.scale = scale;
    return p;
}

template <int MODE>
static void launch_walk(int dtype, long long grid, hipStream_t s, const fa::gdn::ChunkParams &p)
{
    if (dtype == FA_F16)
        hipLaunchKernelGGL((fa::gdn::chunk_kernel<_Float16, MODE>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((fa::gdn::chunk_kernel<__bf16, MODE>), dim3((unsigned)grid), dim3(256), 0, s, p);
}

extern "C" {

int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta, const void *A,
                  const float *s0, void *o, float *s_final, int B, int T, int Hqk, int Hv, int DK, int DV, float scale,
                  int dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    const int rc = check_chunk_args(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DK, DV, scale, dtype);
    if (rc != FA_OK) return rc;
    if (workspace) {
        if (workspace_bytes < gdn_chunk_workspace_size(B, T, Hv, DV)) return FA_ERR_INVALID_ARG;
        if ((uintptr_t)workspace & 255u) return FA_ERR_UNSUPPORTED;
    }
    fa::gdn::ChunkParams p = chunk_params(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DV, scale);
    p.ws_st = workspace;
    p.ws_vn = workspace ? (void *)((char *)workspace + ws_states_bytes(B, T, Hv, DV)) : nullptr;
    const long long grid = (long long)B * Hv * p.dv_blocks;
    const long long grid_out = grid * p.n_chunks;
    if (grid_out > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (!workspace) {
        launch_walk<fa::gdn::WALK_FULL>(dtype, grid, s, p);
        return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }
    launch_walk<fa::gdn::WALK_STATE>(dtype, grid, s, p);
    if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
    if (dtype == FA_F16)
        hipLaunchKernelGGL((fa::gdn::out_kernel<_Float16>), dim3((unsigned)grid_out), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((fa::gdn::out_kernel<__bf16>), dim3((unsigned)grid_out), dim3(256), 0, s, p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Runs of chunks of the segmented mode for `segments` requested: runs of ceil(chunks / segments)
// chunks (at most one per chunk), so that none is empty; returns their number.
static int seg_runs(int T, int segments, int *seg_chunks)
{
    const int n_chunks = (T + fa::gdn::C - 1) / fa::gdn::C;
    if (segments > n_chunks) segments = n_chunks;
    const int len = (n_chunks + segments - 1) / segments;
    *seg_chunks = len;
    return (n_chunks + len - 1) / len;
}

// workspace of the segmented mode: M, then Z, then the start states (each 256-byte aligned),
// per run but one
static size_t seg_part_bytes(int B, int Hv, int cols, int runs)
{
    return ((size_t)B * Hv * (runs - 1) * fa::gdn::DK * cols * 4 + 255) & ~(size_t)255;
}

size_t gdn_segmented_workspace_size(int B, int T, int Hv, int DV, int segments)
{
    if (B <= 0 || T <= 0 || Hv <= 0 || DV <= 0 || segments <= 0) return 0;
    int len;
    const int runs = seg_runs(T, segments, &len);
    if (runs == 1) return 0;
    return seg_part_bytes(B, Hv, fa::gdn::DK, runs) + 2 * seg_part_bytes(B, Hv, DV, runs);
}

// Cost model of the chunk walks (µs, measured on MI355X over long and small-grid shapes): a
// chunk step takes ~2.0 in the transition walk and ~3.0 in the output walk at one workgroup per
// CU, 2.1 in the two-kernel state walk; the two-kernel output kernel ~5.3 per 512 (chunk,
// 64-column) workgroups; a combine step ~3.5 (bound by fetching M_r); ~10 of launches.
static double seg_cost(long long walkers, long long tr_walkers, int runs, int len)
{
    const double tr_rounds = (double)((tr_walkers * (runs - 1) + 255) / 256);
    const double out_rounds = (double)((walkers * runs + 255) / 256);
    return tr_rounds * len * 2.0 + out_rounds * len * 3.0 + (runs - 1) * 3.5 + 10.0;
}

static double seq_cost(long long walkers, int n_chunks)
{
    if (walkers <= 64) return n_chunks * 2.1 + (double)((walkers * n_chunks + 511) / 512) * 5.3 + 5.0;
    return n_chunks * 3.0 * (double)((walkers + 255) / 256);
}

// The segmented mode walks runs of chunks in parallel at the price of a second (transition)
// walk over every run but the last with DK + DV state columns; it pays when the sequential walk
// leaves most CUs idle.  Picks the run count (at most 64) of least modelled time, and 1 (no
// segmentation) unless that beats the sequential pick of gdn_chunk_plan by a fifth; only for
// grids of at most 128 state walkers.
int gdn_segment_plan(int B, int T, int Hv, int DV, int *segments)
{
    if (!segments) return FA_ERR_INVALID_ARG;
    *segments = 1;
    if (B <= 0 || T <= 0 || Hv <= 0 || DV <= 0) return FA_ERR_INVALID_ARG;
    if (DV % fa::gdn::DVB != 0) return FA_ERR_UNSUPPORTED;
    const long long walkers = (long long)B * Hv * (DV / fa::gdn::DVB);
    const long long tr_walkers = (long long)B * Hv * ((fa::gdn::DK + DV) / fa::gdn::DVB);
    const int n_chunks = (T + fa::gdn::C - 1) / fa::gdn::C;
    if (walkers > 128 || n_chunks < 2) return FA_OK;
    double best = 0.8 * seq_cost(walkers, n_chunks);
    for (int want = 2; want <= 64 && want <= n_chunks; ++want) {
        int len;
        const int runs = seg_runs(T, want, &len);
        if (runs != want) continue;  // the same runs as a smaller request
        const double c = seg_cost(walkers, tr_walkers, runs, len);
        if (c < best) {
            best = c;
            *segments = runs;
        }
    }
    return FA_OK;
}

int gdn_chunk_fwd_segmented(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const void *A, const float *s0, void *o, float *s_final, int B, int T, int Hqk, int Hv,
                            int DK, int DV, float scale, int dtype, int segments, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    const int rc = check_chunk_args(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DK, DV, scale, dtype);
    if (rc != FA_OK) return rc;
    if (segments <= 0) return FA_ERR_INVALID_ARG;
    int len;
    const int runs = seg_runs(T, segments, &len);
    fa::gdn::ChunkParams p = chunk_params(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DV, scale);
    hipStream_t s = (hipStream_t)stream;
    if (runs == 1) {  // one run: the one-kernel mode
        launch_walk<fa::gdn::WALK_FULL>(dtype, (long long)B * Hv * p.dv_blocks, s, p);
        return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }
    if (!workspace || workspace_bytes < gdn_segmented_workspace_size(B, T, Hv, DV, segments)) return FA_ERR_INVALID_ARG;
    if ((uintptr_t)workspace & 255u) return FA_ERR_UNSUPPORTED;
    const long long bh = (long long)B * Hv;
    const long long grid_tr = bh * (runs - 1) * ((fa::gdn::DK + DV) / fa::gdn::DVB);
    const long long grid_out = bh * runs * p.dv_blocks;
    if (grid_tr > 0x7fffffffLL || grid_out > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    p.ws_m = (float *)workspace;
    p.ws_z = (float *)((char *)workspace + seg_part_bytes(B, Hv, fa::gdn::DK, runs));
    p.ws_start = (float *)((char *)p.ws_z + seg_part_bytes(B, Hv, DV, runs));
    p.seg_chunks = len;
    // transition walks of every run but the last
    fa::gdn::ChunkParams pt = p;
    pt.n_seg = runs - 1;
    pt.dv_blocks = (fa::gdn::DK + DV) / fa::gdn::DVB;
    launch_walk<fa::gdn::WALK_TRANSITION>(dtype, grid_tr, s, pt);
    if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
    fa::gdn::CombineParams pc;
    pc.m = p.ws_m;
    pc.z = p.ws_z;
    pc.s0 = s0;
    pc.start = p.ws_start;
    pc.n_runs = runs - 1;
    pc.DV = DV;
    hipLaunchKernelGGL(fa::gdn::combine_kernel, dim3((unsigned)(bh * (DV / 8))), dim3(512), 0, s, pc);
    if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
    // every run again from its start state, forming the outputs; the last run writes s_final
    p.n_seg = runs;
    launch_walk<fa::gdn::WALK_FULL>(dtype, grid_out, s, p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
