// fa_bwd.hip -- backward pass of the fused attention for MI355X (gfx950): the gradients of O
// with respect to q, k and v, recomputing the probabilities from the forward's logsumexp.
//
// With z_ij = scale q_i . k_j over the visible keys of row i, P_ij = exp(z_ij - lse_i) and an
// upstream gradient dO:
//     dv_j = sum_i P_ij dO_i          dP_ij = dO_i . v_j         Delta_i = dO_i . O_i
//     dS_ij = P_ij (dP_ij - Delta_i)   dq_i = scale sum_j dS_ij k_j   dk_j = scale sum_i dS_ij q_i
// (Delta_i = sum_j P_ij dP_ij, the softmax Jacobian's row term, taken from the forward output.)
// dk and dv of a KV head sum over the query heads of its group.
//
// Three kernels, all on the 32x32x16 MFMA with fp32 accumulation:
//   prep:  Delta_i and lse_i * log2(e) per row, into a small workspace.
//   dQ:    one workgroup per (b, h, 128 or 256 query rows), lane = query (as in the forward): per
//          64-key tile, S^T = K Q^T and dP^T = V dO^T with Q and dO resident in registers,
//          dS^T from them, then dQ^T += K^T dS^T with K^T read by the transposing LDS read.
//   dK/dV: one workgroup per (b, kv head, 128 keys), lane = key, K resident in registers and
//          the block's V rows in LDS: per 32-query tile of every query head of the group,
//          S = Q K^T and dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS (transposing
//          reads of dO and Q).  V in LDS rather than registers leaves room for the operand
//          read-ahead without spills; the 32-row query tiles keep two workgroups' LDS per CU.
// No atomics: every output element has one owner, so results are deterministic.
// Each wave raises its priority (s_setprio 1) while it issues a run of MFMAs and drops it for the
// exp / dS arithmetic between them, so that the other wave on the SIMD fills the VALU while the
// matrix pipe keeps taking this wave's products (3-4 % on the non-causal shapes).  Inside a run,
// the LDS operand of each MFMA is read a few MFMAs ahead (mfma_run) rather than just before it,
// so the LDS latency does not stall every product.
//
// LDS tiles here are read both row-wise (16-byte MFMA operand reads, 16 lanes = 16 rows of one
// unit) and transposed (8-byte transposing reads, 32 lanes = 4 rows x 4 units), so instead of
// padding they use an XOR swizzle of the 16-byte units that keeps both passes on distinct
// banks: unit u of row r is stored at u ^ swz(r).  The tiles are copied HBM -> LDS by buffer
// loads with LDS destination, each lane gathering the logical unit its LDS slot must hold.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_device.h"
#include "fa_mfma_run.h"
#include "fa_swizzle.h"
#include "fa_tiles.h"

namespace fa {
namespace bwd {

constexpr int kReadAhead = 3;  // LDS operand reads in flight ahead of the MFMA that uses them (mfma_run)

constexpr int kRows = 128;  // rows a 4-wave workgroup owns (4 waves x 32)
constexpr int kDqFullGrid = 256;  // 8-wave dQ workgroups that fill the MI355X's 256 CUs once
constexpr int kTile = 64;   // rows of the inner-loop tile
constexpr int kStats = 2 * kTile;  // floats per 64-row stats chunk: lse * log2(e), then Delta

struct Params {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *stats;  // [B*Hq][ceil(M/64)][128]
    int B, Hq, Hkv, M, N;
    int n_qt;           // query tiles of kRows per (b, h) (dQ) or key blocks of kRows per (b, kv head) (dK/dV)
    long long total;    // workgroups (< 2^31)
    GridMap gm;         // workgroup id -> work, for this grid
    float c;            // scale * log2(e)
    float scale;
};

// ------------------------------------------------------------------ prep
// 4 lanes per row, 64 rows per workgroup: Delta_i = dO_i . O_i (fp32) and lse_i * log2(e);
// rows past M get zeros (their chunk slots are read by the tile loads).
template <typename T, int D>
__global__ __launch_bounds__(256) void prep_kernel(Params p)
{
    const int chunks = (p.M + kTile - 1) / kTile;
    const long long chunk = blockIdx.x;  // over B * Hq * chunks
    const long long bh = chunk / chunks;
    const int i = (int)(chunk % chunks) * kTile + (threadIdx.x >> 2);
    const int part = threadIdx.x & 3;
    float acc = 0.f;
    if (i < p.M) {
        const size_t row = (size_t)bh * p.M + i;
        const u32x4 *o = (const u32x4 *)((const T *)p.o + row * D) + part * (D / 32);
        const u32x4 *g = (const u32x4 *)((const T *)p.dout + row * D) + part * (D / 32);
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
            const u32x4 a = o[u], b = g[u];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const auto x = Elem<T>::unpack2(a[w]), y = Elem<T>::unpack2(b[w]);
                acc = __builtin_fmaf(x[0], y[0], acc);
                acc = __builtin_fmaf(x[1], y[1], acc);
            }
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (part == 0) {
        float *st = p.stats + chunk * kStats + (threadIdx.x >> 2);
        const float l = i < p.M ? p.lse[(size_t)bh * p.M + i] : 0.f;
        st[0] = l * 1.44269504088896340736f;  // -inf stays -inf (a row that sees no key)
        st[kTile] = acc;
    }
}

// ------------------------------------------------------------ tile loads

// HBM -> LDS copy of ROWS rows of a contiguous [rows, D] slab into the swizzled layout:
// instruction j (of TI) fills LDS bytes [1 KiB j, 1 KiB (j+1)); of a workgroup of WV waves (4 or
// 8) the wave issues j = wave + WV i.  Lane l's slot is row j * RPK + l / UPR, physical unit
// l % UPR; it gathers the logical unit (l % UPR) ^ swz(row).  swz depends only on row bits that
// j = wave + WV i does not change, so one source offset per lane serves every i (plus i WV RPK
// rows).
template <int D, int ROWS, int WV = 4> struct TileLoad {
    static constexpr int RB = 2 * D;                // bytes per row
    static constexpr int UPR = RB / 16;             // units per row
    static constexpr int RPK = 1024 / RB;           // rows per 1 KiB instruction
    static constexpr int TI = ROWS * RB / 1024;     // instructions per tile
    static constexpr int PER_WAVE = TI / WV;
    static_assert(PER_WAVE * WV == TI, "tile instructions split evenly over the waves");
    unsigned src;
    __device__ TileLoad(int wave, int lane)
    {
        const int row = wave * RPK + lane / UPR, phys = lane % UPR;
        src = (unsigned)(row * RB + ((phys ^ swz<D>(row)) * 16));
    }
    // rows [r0, r0 + ROWS) of the slab at base, valid rows < rows_valid
    __device__ __forceinline__ void issue(const void *base, int r0, int rows_valid, lds_u8 *dst, int wave) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) issue_one(base, r0, rows_valid, dst, wave, i);
    }
    // instruction i (< PER_WAVE) of the above alone
    __device__ __forceinline__ void issue_one(const void *base, int r0, int rows_valid, lds_u8 *dst, int wave, int i) const
    {
        const int rows = rows_valid - r0 < ROWS ? rows_valid - r0 : ROWS;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const char *)base + (long long)r0 * RB), (short)0, rows > 0 ? rows * RB : 0, 0x00020000);
        lds_load16(rs, (lds_void *)(dst + (wave + WV * i) * 1024), src + i * WV * RPK * RB);
    }
};

// s_waitcnt vmcnt(0): every load this wave issued has landed (expcnt, lgkmcnt untouched)
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// B operand of a k-step from accumulator registers 8 tt .. 8 tt + 7 (rows {16 tt + 4 hh + e,
// 16 tt + 8 + 4 hh + e} of the natural accumulator layout), rounded to T
template <typename T> __device__ __forceinline__ u32x4 pack_b(const f32x16 &x, int tt)
{
    u32x4 b;
#pragma unroll
    for (int w = 0; w < 4; ++w) b[w] = Elem<T>::pack2(x[8 * tt + 2 * w], x[8 * tt + 2 * w + 1]);
    return b;
}

// stores 16 consecutive columns (accumulator registers 0..15 times `mul`) of one row as T
template <typename T> __device__ __forceinline__ void store16(T *dst, const f32x16 &x, float mul)
{
    u32x4 w0, w1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        w0[r] = Elem<T>::pack2(x[2 * r] * mul, x[2 * r + 1] * mul);
        w1[r] = Elem<T>::pack2(x[8 + 2 * r] * mul, x[8 + 2 * r + 1] * mul);
    }
    u32x4 *d = (u32x4 *)dst;
    d[0] = w0;
    d[1] = w1;
}

// -------------------------------------------------------------------- dQ

template <typename T, int D, bool CAUSAL, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void dq_kernel(Params p)
{
    constexpr int QR = 32 * W;  // query rows of the workgroup
    constexpr int KS = D / 16, DB = D / 32, TILE = kTile * 2 * D;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[4 * TILE];  // K0 K1 V0 V1
    lds_u8 *smem = (lds_u8 *)smem_raw;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ql = lane & 31, hh = lane >> 5;

    const TileCoord tc = logical_tile(xcd_remap(blockIdx.x, p.gm), p.gm, CAUSAL);
    const int g = p.Hq / p.Hkv, hk = tc.h / g;
    const int M = p.M, N = p.N;
    const int m0 = tc.qt * QR;
    const KvRange kr = kv_range(m0, QR, kTile, M, N, CAUSAL);
    const size_t bh = (size_t)tc.b * p.Hq + tc.h;
    const T *kg = (const T *)p.k + ((size_t)tc.b * p.Hkv + hk) * (size_t)N * D;
    const T *vg = (const T *)p.v + ((size_t)tc.b * p.Hkv + hk) * (size_t)N * D;
    const int qrow = m0 + wave * 32 + ql;
    const bool qvalid = qrow < M;

    // Q and dO of this lane's row: B operands of S^T = K Q^T and dP^T = V dO^T
    u32x4 qreg[KS], dreg[KS];
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const T *qr = (const T *)p.q + (bh * M + qrow) * D + hh * 8;
        const T *dr = (const T *)p.dout + (bh * M + qrow) * D + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qreg[ks] = qvalid ? *(const u32x4 *)(qr + ks * 16) : z;
            dreg[ks] = qvalid ? *(const u32x4 *)(dr + ks * 16) : z;
        }
    }
    float lse2 = 0.f, delta = 0.f;
    if (qvalid) {
        const float *st = p.stats + (bh * ((M + kTile - 1) / kTile) + qrow / kTile) * kStats + qrow % kTile;
        lse2 = st[0];
        delta = st[kTile];
    }
    const float c = p.c;
    const int causal_lim = qrow + (N - M);

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    const TileLoad<D, kTile, W> ld(wave, lane);
    const TrOffsets<D> tro(lane);
    const int n_tiles = kr.n_tiles;
    if (n_tiles > 0) {
        ld.issue(kg, 0, N, smem, wave);
        ld.issue(vg, 0, N, smem + 2 * TILE, wave);
    }
    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        wait_vm0();
        __syncthreads();  // tile t visible to all waves; every wave is done with tile t - 1
        // the copies of tile t + 1 go out one every few MFMAs of the S / dP run below rather than
        // all at once here; past the last tile they get an empty range (zeros into the spare buffer)
        const int n_next = t + 1 < n_tiles ? N : 0;
        auto copy = [&](auto cc) {
            constexpr int c = decltype(cc)::value, PW = TileLoad<D, kTile, W>::PER_WAVE;
            if constexpr (c < PW) ld.issue_one(kg, (t + 1) * kTile, n_next, smem + (buf ^ 1) * TILE, wave, c);
            else ld.issue_one(vg, (t + 1) * kTile, n_next, smem + (2 + (buf ^ 1)) * TILE, wave, c - PW);
        };
        const lds_u8 *kt = smem + buf * TILE, *vt = smem + (2 + buf) * TILE;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
        __builtin_amdgcn_s_setprio(1);
        // MFMA m: k-step m / 4 of key block (m / 2) % 2, of S (m even, K rows) or dP (m odd, V rows)
        mfma_run<4 * KS, kReadAhead>(
            [&](auto mc) {
                constexpr int m = decltype(mc)::value;
                return read_row<D>(m % 2 ? vt : kt, ((m / 2) % 2) * 32 + ql, 2 * (m / 4) + hh);
            },
            [&](auto mc, const u32x4 &a) {
                constexpr int m = decltype(mc)::value, kb = (m / 2) % 2;
                if constexpr (m % 2 == 0)
                    s[kb] = Elem<T>::mfma(a, qreg[m / 4], s[kb]);
                else
                    dp[kb] = Elem<T>::mfma(a, dreg[m / 4], dp[kb]);
                constexpr int NC = 2 * TileLoad<D, kTile, W>::PER_WAVE, ST = 4 * KS / NC;  // copies, MFMAs per copy
                static_assert(ST * NC == 4 * KS, "copies spread evenly over the run");
                if constexpr (m % ST == 1) copy(std::integral_constant<int, m / ST>{});
            });
        // dS^T = P^T (dP^T - Delta); register r of block kb is key n0 + 32 kb + 8 (r/4) + 4 hh + r%4
        __builtin_amdgcn_s_setprio(0);
        const int n0 = t * kTile;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -lse2));
                s[kb][r] = pr * (dp[kb][r] - delta);
            }
        // masked tiles (diagonal band, ragged tail): dS of the keys the row does not see is zero.
        // One uniform branch around the whole pass, so unmasked tiles run no per-element mask code.
        if (t >= kr.n_full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    s[kb][r] = key < N && (!CAUSAL || key <= causal_lim) ? s[kb][r] : 0.f;
                }
        }
        // dQ^T += K^T dS^T
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const u32x4 b = pack_b<T>(s[kb], tt);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = Elem<T>::mfma(read_tr<D>(kt, tro, kb * 32 + 16 * tt, db), b, acc[db]);
            }
        __builtin_amdgcn_s_setprio(0);
    }
    if (qvalid) {
        T *dst = (T *)p.dq + (bh * M + qrow) * D + hh * 16;
#pragma unroll
        for (int db = 0; db < DB; ++db) store16<T>(dst + db * 32, acc[db], p.scale);
    }
}

// ------------------------------------------------------------------ dK/dV

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void dkdv_kernel(Params p)
{
    constexpr int KS = D / 16, DB = D / 32, QT = 32;  // QT: query rows per step
    constexpr int TILE = QT * 2 * D;
    constexpr int BUF = 2 * TILE + 1024;  // Q tile, dO tile, stats (32 lse, 32 Delta; the
                                          // copy writes 16 bytes per lane of the wave: 1 KiB)
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * BUF];
    __shared__ __attribute__((aligned(16))) unsigned char vt_[kRows * 2 * D];  // V of the block
    lds_u8 *smem = (lds_u8 *)smem_raw, *vtile = (lds_u8 *)vt_;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kl = lane & 31, hh = lane >> 5;

    // (b, kv head) outer, key blocks inner (first blocks see the most queries when causal)
    const GridPos gp = grid_pos(xcd_remap(blockIdx.x, p.gm), p.gm);  // p.gm divides by the key blocks
    const int kblk = gp.inner;
    const int b = gp.b, hk = gp.hk;
    const long long bhk = (long long)b * p.Hkv + hk;
    const int g = p.Hq / p.Hkv;
    const int M = p.M, N = p.N;
    const int n0 = kblk * kRows;
    const int key = n0 + wave * 32 + kl;
    const bool kvalid = key < N;

    // K row of this lane's key: B operand of S = Q K^T (the V rows, B operands of dP = dO V^T,
    // are read from the block's V tile in LDS)
    u32x4 kreg[KS];
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const T *kr = (const T *)p.k + (bhk * N + key) * (size_t)D + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kreg[ks] = kvalid ? *(const u32x4 *)(kr + ks * 16) : z;
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.f;

    // query tiles that see some key of the block: i >= n0 - (N - M) when causal
    const int n_qtiles = (M + kTile - 1) / kTile;  // 64-row chunks of the statistics workspace
    const int n_q32 = (M + QT - 1) / QT;
    int qt_lo = 0;
    if (CAUSAL) {
        const long long first = (long long)n0 - (N - M);
        qt_lo = first <= 0 ? 0 : (first >= M ? n_q32 : (int)(first / QT));
    }
    const int nq = n_q32 - qt_lo;
    const int iters = g * nq;
    const float c = p.c;
    const long long diag = (long long)n0 + kRows - 1 - (N - M);  // rows >= diag see every key of the block

    const TileLoad<D, QT> ld(wave, lane);
    const TrOffsets<D> tro(lane);
    {  // the block's V rows, once (landed by the first step's wait)
        const TileLoad<D, kRows> vl(wave, lane);
        vl.issue((const T *)p.v + bhk * N * D, n0, N, vtile, wave);
    }
    auto issue = [&](int it, int buf) {
        const int h = hk * g + it / nq, qt = qt_lo + it % nq;
        const size_t bh = (size_t)b * p.Hq + h;
        lds_u8 *dst = smem + buf * BUF;
        ld.issue((const T *)p.q + bh * M * D, qt * QT, M, dst, wave);
        ld.issue((const T *)p.dout + bh * M * D, qt * QT, M, dst + TILE, wave);
        if (wave == 0) {  // 32 lse (lanes 0..7) and 32 Delta (lanes 8..15) of this 32-row tile
            const int i0 = qt * QT, ch = i0 / kTile, half = (i0 % kTile) / QT;
            const float *st = p.stats + (bh * n_qtiles + ch) * kStats + half * QT;
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void *)st, (short)0, (kTile + QT) * 4, 0x00020000);
            const unsigned off = lane < 8 ? (unsigned)(lane * 16) : lane < 16 ? (unsigned)(kTile * 4 + (lane - 8) * 16)
                                                                             : 0x7fffff00u;
            lds_load16(rs, (lds_void *)(dst + 2 * TILE), off);
        }
    };
    if (iters > 0) issue(0, 0);
    for (int it = 0; it < iters; ++it) {
        const int buf = it & 1;
        wait_vm0();
        __syncthreads();
        if (it + 1 < iters) issue(it + 1, buf ^ 1);
        const int qt = qt_lo + it % nq;
        const int i0 = qt * QT;
        const bool masked = n0 + kRows > N || i0 + QT > M || (CAUSAL && i0 < diag);
        const lds_u8 *qtile = smem + buf * BUF, *dtile = qtile + TILE;
        const float *stl = (const float *)(qtile + 2 * TILE);
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
        __builtin_amdgcn_s_setprio(1);
        // MFMA m: k-step m / 2 of S (m even: Q rows by the K registers) or of dP (m odd: dO rows
        // by this lane's V row, both from LDS); operands read kReadAhead MFMAs ahead
        mfma_run2<2 * KS, kReadAhead>(
            [&](auto mc, u32x4 &a, u32x4 &bo) {
                constexpr int m = decltype(mc)::value, ks = m / 2;
                if constexpr (m % 2 == 0) {
                    a = read_row<D>(qtile, kl, 2 * ks + hh);
                } else {
                    a = read_row<D>(dtile, kl, 2 * ks + hh);
                    bo = read_row<D>(vtile, wave * 32 + kl, 2 * ks + hh);
                }
            },
            [&](auto mc, const u32x4 &a, const u32x4 &bo) {
                constexpr int m = decltype(mc)::value;
                if constexpr (m % 2 == 0)
                    s = Elem<T>::mfma(a, kreg[m / 2], s);
                else
                    dp = Elem<T>::mfma(a, bo, dp);
            });
        __builtin_amdgcn_s_setprio(0);
        // register r is query i0 + 8 (r/4) + 4 hh + r%4 of this lane's key; P replaces S and dS
        // replaces dP in place
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int qi = 8 * gq + 4 * hh;
            const f32x4 l4 = *(const f32x4 *)(stl + qi);
            const f32x4 d4 = *(const f32x4 *)(stl + QT + qi);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * gq + e;
                const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l4[e]));
                s[r] = x;
                dp[r] = x * (dp[r] - d4[e]);
            }
        }
        // masked tiles (diagonal band, ragged ends): P and dS of the pairs the lane's key does not
        // see are zero.  One uniform branch around the whole pass, so unmasked tiles run no
        // per-element mask code (a second copy of the loop above made the compiler spill).
        if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool vis = kvalid && i < M && (!CAUSAL || key <= i + (N - M));
                s[r] = vis ? s[r] : 0.f;
                dp[r] = vis ? dp[r] : 0.f;
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the tile's 32 queries.  MFMA m: k-step
        // tt = m / (2 DB) of column block db = (m / 2) % DB, of dV (m even) or dK (m odd)
        __builtin_amdgcn_s_setprio(1);
        u32x4 bp = pack_b<T>(s, 0), bs = pack_b<T>(dp, 0);
        mfma_run<4 * DB, kReadAhead>(
            [&](auto mc) {
                constexpr int m = decltype(mc)::value;
                return read_tr<D>(m % 2 ? qtile : dtile, tro, 16 * (m / (2 * DB)), (m / 2) % DB);
            },
            [&](auto mc, const u32x4 &a) {
                constexpr int m = decltype(mc)::value, db = (m / 2) % DB;
                if constexpr (m == 2 * DB) {
                    bp = pack_b<T>(s, 1);
                    bs = pack_b<T>(dp, 1);
                }
                if constexpr (m % 2 == 0)
                    dv[db] = Elem<T>::mfma(a, bp, dv[db]);
                else
                    dk[db] = Elem<T>::mfma(a, bs, dk[db]);
            });
        __builtin_amdgcn_s_setprio(0);
    }
    if (kvalid) {
        T *dkr = (T *)p.dk + (bhk * N + key) * (size_t)D + hh * 16;
        T *dvr = (T *)p.dv + (bhk * N + key) * (size_t)D + hh * 16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            store16<T>(dkr + db * 32, dk[db], p.scale);
            store16<T>(dvr + db * 32, dv[db], 1.f);
        }
    }
}

// --------------------------------------------------------------------- host

size_t workspace_bytes(int B, int Hq, int M)
{
    return (size_t)B * Hq * ((M + kTile - 1) / kTile) * kStats * sizeof(float);
}

template <typename T, int D>
static hipError_t launch_d(Params p, bool causal, hipStream_t s)
{
    const long long chunks = (long long)p.B * p.Hq * ((p.M + kTile - 1) / kTile);
    hipLaunchKernelGGL((prep_kernel<T, D>), dim3((unsigned)chunks), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dQ: 8 waves over 256 rows (one K/V tile copy serves twice the rows) when those workgroups
    // alone fill every CU once at D = 128, else 4 waves over 128 rows
    const bool w8 = D == 128 && (long long)p.B * p.Hq * ((p.M + 255) / 256) >= kDqFullGrid;
    const int q_rows = w8 ? 256 : 128;
    Params pq = p;
    pq.n_qt = (p.M + q_rows - 1) / q_rows;
    pq.total = (long long)p.B * p.Hq * pq.n_qt;
    pq.gm = make_grid_map((unsigned)pq.total, p.Hq / p.Hkv, pq.n_qt, p.Hkv);
    if (w8) {
        if (causal)
            hipLaunchKernelGGL((dq_kernel<T, D, true, 8>), dim3((unsigned)pq.total), dim3(512), 0, s, pq);
        else
            hipLaunchKernelGGL((dq_kernel<T, D, false, 8>), dim3((unsigned)pq.total), dim3(512), 0, s, pq);
    } else {
        if (causal)
            hipLaunchKernelGGL((dq_kernel<T, D, true, 4>), dim3((unsigned)pq.total), dim3(256), 0, s, pq);
        else
            hipLaunchKernelGGL((dq_kernel<T, D, false, 4>), dim3((unsigned)pq.total), dim3(256), 0, s, pq);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    Params pk = p;
    pk.n_qt = (p.N + kRows - 1) / kRows;
    pk.total = (long long)p.B * p.Hkv * pk.n_qt;
    pk.gm = make_grid_map((unsigned)pk.total, pk.n_qt, 1, p.Hkv);  // logical index: (b, kv head), key block
    if (causal)
        hipLaunchKernelGGL((dkdv_kernel<T, D, true>), dim3((unsigned)pk.total), dim3(256), 0, s, pk);
    else
        hipLaunchKernelGGL((dkdv_kernel<T, D, false>), dim3((unsigned)pk.total), dim3(256), 0, s, pk);
    return hipGetLastError();
}

}  // namespace bwd
}  // namespace fa

extern "C" {

size_t fa_bwd_workspace_size(int B, int Hq, int M)
{
    if (B <= 0 || Hq <= 0 || M <= 0) return 0;
    return fa::bwd::workspace_bytes(B, Hq, M);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse, void *dq,
           void *dk, void *dv, int B, int Hq, int Hkv, int M, int N, int D, float scale, int causal, int dtype,
           void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || N <= 0 || D <= 0) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    const double nq = (double)B * Hq * M * D, nk = (double)B * Hkv * N * D;
    if (nq > 9.0e18 || nk > 9.0e18) return FA_ERR_INVALID_ARG;
    if (workspace_bytes < fa::bwd::workspace_bytes(B, Hq, M)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    const uintptr_t align = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
                            (uintptr_t)lse | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace;
    if (align & 15u) return FA_ERR_UNSUPPORTED;
    const long long wg_q = (long long)B * Hq * ((M + fa::bwd::kRows - 1) / fa::bwd::kRows);
    const long long wg_k = (long long)B * Hkv * ((N + fa::bwd::kRows - 1) / fa::bwd::kRows);
    const long long wg_p = (long long)B * Hq * ((M + fa::bwd::kTile - 1) / fa::bwd::kTile);
    if (wg_q > 0x7fffffffLL || wg_k > 0x7fffffffLL || wg_p > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;

    fa::bwd::Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.stats = (float *)workspace;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.M = M;
    p.N = N;
    p.n_qt = 0;
    p.total = 0;
    p.c = scale * 1.44269504088896340736f;
    p.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    if (dtype == FA_F16)
        err = D == 128 ? fa::bwd::launch_d<_Float16, 128>(p, causal != 0, s)
                       : fa::bwd::launch_d<_Float16, 64>(p, causal != 0, s);
    else
        err = D == 128 ? fa::bwd::launch_d<__bf16, 128>(p, causal != 0, s)
                       : fa::bwd::launch_d<__bf16, 64>(p, causal != 0, s);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
