// fa_fwd.hip -- fused attention forward for MI355X (gfx950, CDNA4), and its C ABI.
//
// One workgroup computes one (batch b, query head h, query tile of BM rows): 8 waves over 256
// rows on large grids, 4 waves over 128 rows on small ones, or -- small grids with long key
// ranges -- 8 waves over 128 rows in two key groups of 4 that share the key tiles out
// between them and merge their softmax states at the end.  Each wave of a group owns 32
// query rows.  The key/value sequence is the inner loop, in tiles of BN = 64 keys
// ("从零开始写Qwen3", FlashAttention derivation article, section "FlashAttention" and its
// variant note: Q tiles in parallel, KV as the inner loop).  K and V tiles are staged through
// LDS, double-buffered; Q stays in registers for the whole loop.  The key-split mode (further
// down) gives one query tile's key tiles to several workgroups and merges their results.
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

#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_mfma_run.h"
#include "fa_tiles.h"

namespace fa {

constexpr int kBN = 64;  // keys per tile; a workgroup of W waves owns 32 W query rows

// ------------------------------------------------------------------- layouts

// Row permutation of a 32-row MFMA operand block: A-operand row i holds key (or output
// column) pi(i), chosen so that accumulator register r of a lane in half hh maps to
// 16*hh + r.  (The accumulator row of register r in half hh is 8*(r/4) + 4*hh + r%4.)
// pi_inv is that accumulator-row formula itself.
__host__ __device__ constexpr int pi32(int i) { return 16 * ((i >> 2) & 1) + ((i >> 3) << 2) + (i & 3); }
__host__ __device__ constexpr int pi32_inv(int k) { return ((k & 15) >> 2) * 8 + 4 * (k >> 4) + (k & 3); }

// LDS tiles.  gfx950 LDS has 64 banks of 4 bytes; a 16-byte read serves 16 lanes per pass,
// the 8-byte transposing read 32 lanes per pass.  Rows are padded so that every pass of
// the MFMA operand reads and of the tile writes touches distinct banks, and so that every
// read address is a per-lane base plus a compile-time offset:
//   K tile: the rows of each 32-key block are stored in pi order (slot i holds key pi(i)), so
//     the 16 lanes of a pass read 16 consecutive slots; a pitch of (odd) 16-byte units spreads
//     them over all 16 bank groups.
//   V tile: row-major in key order; a transposing pass reads 4 consecutive rows x 4 units, so
//     the pitch shifts consecutive rows by 4 bank groups.
//   At D = 128 the rows are instead exactly 256 bytes (one pass over the 64 banks) and the
//   16-byte units are XOR-swizzled, which is conflict-free for the same passes without pad
//   bytes: no pad lanes in the tile copies and 16 whole 1 KiB copy instructions per tile.
//   K: unit u of slot r at u ^ (4 (r mod 4) + (r / 4) mod 4), which spreads the 16 slots of a
//   read pass over all 16 bank groups; V: unit u of row r at u ^ 4 (r mod 4), which spreads the
//   4 rows x 4 units of a transposing pass.  A read address is then a per-lane offset chosen by
//   the k-step (K) or column block (V) plus a compile-time row offset.
template <int D> struct Lds {
    static constexpr bool SWZ = D == 128;
    static constexpr int K_PITCH = D == 128 ? 16 * 16 : 9 * 16;   // bytes
    static constexpr int V_PITCH = D == 128 ? 16 * 16 : 12 * 16;  // bytes
    static __device__ __forceinline__ constexpr int k_swz(int r) { return SWZ ? 4 * (r & 3) + ((r >> 2) & 3) : 0; }
    static __device__ __forceinline__ constexpr int v_swz(int r) { return SWZ ? 4 * (r & 3) : 0; }
};

struct Params {
    const void *q, *k, *v;
    void *o;
    float *lse;
    // element strides of the batch, head and row axes (the head-dim axis has unit stride)
    long long q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, v_sb, v_sh, v_ss, o_sb, o_sh, o_ss;
    int B, Hq, Hkv, M, N;
    int n_qt;           // query tiles per (b, h)
    long long total;    // workgroups in the grid (< 2^31)
    GridMap gm;         // workgroup id -> work, for this grid
    float c;            // scale * log2(e)
};

// Key-split mode.  The key tiles a query tile visits are divided over n_split workgroups (an
// even share each); each writes the normalised output and natural-log lse of its share to the
// workspace, and a merge kernel combines them.  A query tile with one share writes O and lse
// directly.  Query tiles are taken in rank order (longest first when causal), so the shares
// per tile never grow with the rank and the split tiles are the ranks [0, n_split_ranks).
// Rows come in units of R = pack * M: with pack = 1 a unit is one query head; with pack = g
// (short queries, M < 128) a unit stacks the g query heads of one KV group, row r being query
// r % M of head r / M, so that one tile's MFMA rows are not mostly empty.
constexpr int kMaxSplitQt = 128;  // query tiles per (b, h) the split plan can describe
struct SplitParams : Params {
    int wg_per_head;    // workgroups per (b, h): prefix[n_qt]
    int slots;          // partial slots per (b, h): prefix[n_split_ranks]
    int n_split_ranks;
    int causal;
    int pack;           // 1, or Hq / Hkv
    int slot_rows;      // rows a slot holds: min(BM, R)
    float *ws_lse;      // [units][slots][slot_rows], units = B * Hq / pack
    float *ws_o;        // [units][slots][slot_rows][D]
    int prefix[kMaxSplitQt + 1];  // workgroups of the query-tile ranks below r
};


// --------------------------------------------------------------------- kernel

// W waves per workgroup (KG = 1: BM = 32 W query rows).  W = 4: two workgroups share a CU.
// W = 8: one workgroup per CU (still two waves per SIMD).  K and V tiles are double-buffered:
// the copies issued at the top of a step land before the step's closing barrier (whose
// workgroup fence waits for them in any case, so a third buffer would buy no extra lead).
//
// KG = 2 (small grids): the W waves form two key groups of W / 2 waves over the same BM =
// 16 W rows; group k takes the query tile's key tiles k, k + 2, ... with buffers of its own,
// both groups walk the same number of tiles (the second one's last tile, when the count is
// odd, lies past the visible range and is masked out entirely), and the two groups' running
// maxima, partial sums and output accumulators are merged through LDS before the epilogue,
// each group merging and storing half of the output columns: half the sequential key loop per
// workgroup, and two waves per SIMD instead of one.
template <typename T, int D, bool CAUSAL, int W, bool SPLIT, int KG, typename P>
__device__ __forceinline__ void fa_fwd_body(const P &p)
{
    static_assert(KG == 1 || (KG == 2 && !SPLIT), "key groups only in the plain kernel");
    constexpr int WG = W / KG;  // waves of one key group
    constexpr int kBM = 32 * WG, kWaves = WG;
    constexpr int NBUF = 2;  // K and V tile buffers of a key group
    constexpr int UNITS = D / 8;                       // 16-byte units per row
    constexpr int KS = D / 16;                         // MFMA k-steps over the head dimension
    constexpr int KB = kBN / 32;                       // 32-key blocks per tile
    constexpr int DB = D / 32;                         // 32-column blocks of the output
    constexpr int KP = Lds<D>::K_PITCH, VP = Lds<D>::V_PITCH;
    constexpr bool SWZ = Lds<D>::SWZ;
    constexpr int K_TILE = kBN * KP, V_TILE = kBN * VP;

    // LDS tile buffers.  KG = 1: one LDS object per K buffer, per V buffer and for the 1 KiB
    // sink of padding loads, so that the compiler can tell a read of one buffer from a copy in
    // flight into another and does not make the read wait for every copy (with one shared
    // array it must, the first transposing V read of each step then waiting for the copies
    // issued at the top of that step).  KG = 2: one array, [K buf 0 .. NBUF-1 | V buf 0 ..
    // NBUF-1] per key group, then the sink -- separate objects measured slower there.
    constexpr int GROUP_BYTES = NBUF * (K_TILE + V_TILE);
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[KG == 2 ? KG * GROUP_BYTES + 1024 : 16];
    __shared__ __attribute__((aligned(16))) unsigned char k0_[K_TILE], k1_[K_TILE];
    __shared__ __attribute__((aligned(16))) unsigned char v0_[V_TILE], v1_[V_TILE];
    __shared__ __attribute__((aligned(16))) unsigned char sink_[1024];
    lds_u8 *smem = (lds_u8 *)smem_raw;

    // Request every 64-byte line of the launch parameters at entry, behind one wait: left to
    // itself the compiler loads each field where it is first used, behind its own wait, and each
    // cold line of the argument segment then costs one more memory round trip before the first
    // tile load is issued.  The parameters are the kernel's only argument (offset 0); later field
    // loads hit the scalar cache.
    {
        typedef const __attribute__((address_space(4))) unsigned karg_u32;
        karg_u32 *ka = (karg_u32 *)__builtin_amdgcn_kernarg_segment_ptr();
        static_assert(sizeof(Params) <= 4 * 64 && sizeof(SplitParams) > 4 * 64, "argument lines touched below");
        if constexpr (SPLIT)  // the fifth line holds the first share-table entries
            asm volatile("" ::"s"(ka[0]), "s"(ka[16]), "s"(ka[32]), "s"(ka[48]), "s"(ka[64]));
        else
            asm volatile("" ::"s"(ka[0]), "s"(ka[16]), "s"(ka[32]), "s"(ka[48]));
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane((tid >> 6) / WG);  // key group
    const int wave = (tid >> 6) % WG;  // wave inside the key group
    lds_u8 *const gsmem = smem + grp * GROUP_BYTES;  // this group's tile buffers (KG = 2)
    // K and V buffer i (i a compile-time constant wherever a copy may be in flight)
    auto kb_ptr = [&](int i) -> lds_u8 * {
        if constexpr (KG == 1) return i == 0 ? (lds_u8 *)k0_ : (lds_u8 *)k1_;
        return gsmem + i * K_TILE;
    };
    auto vb_ptr = [&](int i) -> lds_u8 * {
        if constexpr (KG == 1) return i == 0 ? (lds_u8 *)v0_ : (lds_u8 *)v1_;
        return gsmem + NBUF * K_TILE + i * V_TILE;
    };
    const int ql = lane & 31;   // query column of this lane inside the wave's 32 rows
    const int hh = lane >> 5;   // which half of each 32-key block this lane holds

    // ---- A1: which (b, h, query tile) this workgroup computes
    const unsigned L = xcd_remap(blockIdx.x, p.gm);
    TileCoord tc;  // tc.h: the (first) query head of the workgroup's unit
    int rank = 0, split = 0, n_split = 1;
    int R = p.M;           // rows of the unit
    long long unit = 0;    // unit index (key-split mode)
    if constexpr (SPLIT) {
        // logical order: (b, kv head), then query-tile rank with its shares, then the group's
        // units (p.gm divides by the units per KV group and by the workgroups per unit)
        const GridPos gp = grid_pos(L, p.gm);
        const int hg = gp.inner;
        const int j = gp.mid;
        int lo = 0, hi = p.n_qt;  // prefix[lo] <= j < prefix[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.prefix[mid] <= j) lo = mid; else hi = mid;
        }
        rank = lo;
        split = j - p.prefix[lo];
        n_split = p.prefix[lo + 1] - p.prefix[lo];
        tc.b = gp.b;
        tc.h = (gp.hk * (int)p.gm.inner.d + hg) * p.pack;  // g = inner.d * pack heads per KV head
        tc.hk = gp.hk;
        tc.qt = CAUSAL ? p.n_qt - 1 - rank : rank;
        unit = ((long long)gp.b * p.Hkv + gp.hk) * p.gm.inner.d + hg;
        R = p.pack * p.M;
    } else {
        tc = logical_tile(L, p.gm, CAUSAL);
    }
    const int hk = tc.hk;
    const int m0 = tc.qt * kBM;
    const int M = p.M, N = p.N;
    const KvRange kr = SPLIT ? unit_kv_range(m0, kBM, kBN, M, N, R, CAUSAL) : kv_range(m0, kBM, kBN, M, N, CAUSAL);
    // key tiles [t0, t0 + n_tiles) of the query tile's visible range are this workgroup's; its
    // key group grp walks n_loc of them: t0 + KG i + grp for i < n_loc
    const int t0 = split * kr.n_tiles / n_split;
    const int n_tiles = (split + 1) * kr.n_tiles / n_split - t0;
    const int n_loc = (n_tiles + KG - 1) / KG;

    const T *kg = (const T *)p.k + tc.b * p.k_sb + hk * p.k_sh;
    const T *vg = (const T *)p.v + tc.b * p.v_sb + hk * p.v_sh;

    const int qrow = m0 + wave * 32 + ql;  // this lane's row of the unit
    const bool qvalid = qrow < R;
    int qpos = qrow, qhead = tc.h;           // its query position and head
    if constexpr (SPLIT) {
        qpos = qrow % M;
        qhead = tc.h + qrow / M;
    }
    const T *qg = (const T *)p.q + tc.b * p.q_sb + qhead * p.q_sh + qpos * p.q_ss;  // read only if qvalid

    // ---- A2: the Q operand, resident in registers (B operand of S^T = K Q^T)
    u32x4 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qreg[ks] = qvalid ? *(const u32x4 *)(qg + ks * 16 + hh * 8) : z;
    }

    // ---- A3: K and V tiles go from HBM straight into LDS: buffer loads whose destination is
    // LDS, 16 bytes per lane, lane i of one instruction filling bytes [16 i, 16 i + 16) of a
    // 1 KiB block.  Instruction j of a tile fills block j of that tile's LDS buffer; the wave
    // issues j = wave, wave + W, ...  Each tile gets its own buffer resource whose size ends at
    // N, so key rows past N -- and the lanes that land on pad units, given an offset past any
    // size -- read as zero without touching memory.  Every wave issues the same number of
    // loads per tile (a wave short of blocks loads nothing into a sink block), so that one
    // constant wait count covers every wave.
    constexpr int K_INSTR = K_TILE / 1024, V_INSTR = V_TILE / 1024;
    static_assert(K_INSTR * 1024 == K_TILE && V_INSTR * 1024 == V_TILE, "tiles are whole 1 KiB blocks");
    constexpr int KI = (K_INSTR + kWaves - 1) / kWaves, VI = (V_INSTR + kWaves - 1) / kWaves;
    constexpr int LOADS_PER_TILE = KI + VI;  // per wave
    static_assert(LOADS_PER_TILE < 16, "wait count encoding");
    constexpr unsigned kPad = 0x7fffff00u;  // an offset past the end of every tile resource
    lds_u8 *const sink = KG == 1 ? (lds_u8 *)sink_ : smem + KG * GROUP_BYTES;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    __builtin_assume(wave_u >= 0 && wave_u < kWaves);
    // key rows at or past kv_end read as zero: the end of the keys, or of this workgroup's share
    // (the pipeline's look-ahead loads run past it)
    const int kv_end = (t0 + n_tiles) * kBN < N ? (t0 + n_tiles) * kBN : N;
    const int k_rs = (int)(p.k_ss * (long long)sizeof(T)), v_rs = (int)(p.v_ss * (long long)sizeof(T));  // row bytes
    unsigned k_src[KI], v_src[VI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        // (unsigned arithmetic and the wave's range let the compiler fold the divisions into
        // shifts and drop the bound test when every wave's blocks exist)
        const unsigned u = (unsigned)(wave_u + kWaves * i) * 64u + (unsigned)lane;  // 16-byte unit of the K tile
        const unsigned slot = u / (KP / 16), unit = u % (KP / 16);  // LDS slot and physical unit
        const unsigned key = (slot & ~31u) | (unsigned)pi32((int)(slot & 31u));  // slot order pi in each 32-key block
        k_src[i] = unit < UNITS && u < K_INSTR * 64 ? key * (unsigned)k_rs + (unit ^ (unsigned)Lds<D>::k_swz((int)slot)) * 16u : kPad;
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
        const unsigned u = (unsigned)(wave_u + kWaves * i) * 64u + (unsigned)lane;
        const unsigned row = u / (VP / 16), unit = u % (VP / 16);
        v_src[i] = unit < UNITS && u < V_INSTR * 64 ? row * (unsigned)v_rs + (unit ^ (unsigned)Lds<D>::v_swz((int)row)) * 16u : kPad;
    }
    // buffer resource of key tile t: its rows up to kv_end, so a row past it (every byte of which
    // lies at or beyond (rows - 1) * row_bytes + D * sizeof(T)) reads as zero
    auto tile_rsrc = [&](const T *base, int row_bytes, int t) {
        const int r0 = t * kBN;
        const int rows = kv_end - r0 < kBN ? kv_end - r0 : kBN;
        const int bytes = rows > 0 ? (rows - 1) * row_bytes + D * (int)sizeof(T) : 0;
        return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + (long long)r0 * row_bytes), (short)0,
                                                 bytes, 0x00020000);
    };
    // copy instruction i of the group's K (or V) tile t into buffer buf
    auto load_k_one = [&](int t, int buf, int i) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(kg, k_rs, t0 + KG * t + grp);
        const int j = wave_u + kWaves * i;
        lds_load16(rs, (lds_void *)(K_INSTR % kWaves == 0 || j < K_INSTR ? kb_ptr(buf) + j * 1024 : sink), k_src[i]);
    };
    auto load_v_one = [&](int t, int buf, int i) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(vg, v_rs, t0 + KG * t + grp);
        const int j = wave_u + kWaves * i;
        lds_load16(rs, (lds_void *)(V_INSTR % kWaves == 0 || j < V_INSTR ? vb_ptr(buf) + j * 1024 : sink), v_src[i]);
    };
    auto load_k = [&](int t, int buf) {  // the group's tile t
#pragma unroll
        for (int i = 0; i < KI; ++i) load_k_one(t, buf, i);
    };
    auto load_v = [&](int t, int buf) {
#pragma unroll
        for (int i = 0; i < VI; ++i) load_v_one(t, buf, i);
    };
    // every load into LDS this wave issued has landed; a barrier then publishes them
    // (s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maximum)
    auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };

    // ---- online-softmax state (A6) and output accumulator
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY;  // running max of the raw scores s (not scaled)
    float l_part = 0.f;       // running sum over this half's keys, relative to m_run
    const float c = p.c;
    const int causal_lim = qpos + (N - M);  // last visible key of this row (causal)

    // per-lane read bases: K slot ql of each 32-key block, unit hh of each 32-byte k-step
    const int k_rd = SWZ ? 0 : ql * KP + hh * 16;
    // transposing V read: in each 16-lane group, source lane 4*e + j reads row (4-row group base + e)
    // at column chunk dcol(j); the result gives lane l the 4 keys of column pi(l % 32)
    const int tr_g = (lane >> 4) & 1, tr_s = lane & 15, tr_e = tr_s >> 2, tr_j = tr_s & 3;
    const int tr_dcol = 16 * (tr_j & 1) + 8 * tr_g + 4 * (tr_j >> 1);
    const int v_rd = SWZ ? 0 : (hh * 16 + tr_e) * VP + tr_dcol * 2;
    // swizzled tiles: per-lane offsets of K k-step ks (slot ql, unit 2 ks + hh) and of the V column
    // block db (row 16 hh + tr_e; the swizzle only flips the block bits, by tr_e)
    unsigned koff[SWZ ? KS : 1], voff[SWZ ? DB : 1];
    if constexpr (SWZ) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) koff[ks] = (unsigned)(ql * KP + (((2 * ks + hh) ^ Lds<D>::k_swz(ql)) * 16));
#pragma unroll
        for (int db = 0; db < DB; ++db)
            voff[db] = (unsigned)((hh * 16 + tr_e) * VP + (4 * (db ^ tr_e) + 2 * (tr_j & 1) + tr_g) * 16 + 8 * (tr_j >> 1));
    }

    // ---- A5: visibility of key `key` to this lane's row (diagonal band / ragged last tile)
    auto visible = [&](int key) { return key < N && (!CAUSAL || key <= causal_lim); };

    // mask (unless `none`) the scores of tile t, then return their in-lane max
    auto mask_max = [&](int t, f32x16 (&sc)[KB], bool none = false) {
        const int n0 = (t0 + KG * t + grp) * kBN;
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (!none) sc[kb][r] = visible(n0 + kb * 32 + hh * 16 + r) ? sc[kb][r] : -INFINITY;
                mt = fmaxf(mt, sc[kb][r]);
            }
        return mt;
    };

    // ---- A6: cross-half row max and running-max update.  O and the partial sum are rescaled only
    // when some row's max grew (alpha = exp2((m_old - m_new) * c) is exactly 1 otherwise);
    // returns m * c for the exp2 of the tile
    auto update_max = [&](float mt) {
        auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mt), __builtin_bit_cast(unsigned, mt),
                                                   false, false);
        mt = fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
        const float m_new = fmaxf(m_run, mt);
        const bool grew = m_new > m_run;
        if (__any(grew)) {
            const float alpha = grew ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.f;  // 0 from -inf
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_run = m_new;
        }
        return (m_run == -INFINITY ? 0.f : m_run) * c;  // no visible key yet: keep exp2 finite
    };

    // The loop body is one straight-line sequence of 2 NM MFMAs whose issue is interleaved
    // with the VALU work of the softmax (the MFMA pipe runs while the wave issues VALU work):
    //   MFMA j <  NM: S_{t+1} += K_{t+1} Q^T      ||  p = exp2(fma(s, c, -m c)) of tile t, in place
    //   MFMA j >= NM: O^T += V_t^T P_t^T          ||  rounding of p to T and row sums of tile t,
    //                                                  in-lane row max of tile t+1
    // followed, only when some row's running max grew, by the rescale of O.  Scheduling
    // barriers fix the order: MFMA j, then its share of VALU work; the LDS operand of MFMA
    // j + RA is read while MFMA j issues.
    constexpr int NM = KS * KB;                 // MFMAs per half step
    constexpr int VALS = KB * 16;               // score values per lane per tile
    constexpr int VPM = VALS / NM;              // values handled per MFMA in each half
    constexpr int NG = 2 * KB;                  // key octets per tile
    constexpr int CPM = 4 / DB;                 // P dwords rounded per value MFMA
    constexpr int RA = 3;                       // operand read-ahead, in MFMAs
    constexpr int NPRE = 2;                     // score MFMAs issued before the running-max update
    static_assert(VPM * NM == VALS && VPM % 2 == 0, "each half must split evenly");
    static_assert(NM == KB * 2 * DB && CPM * DB == 4, "value MFMAs: key block x octet x column block");

    // LDS operand of MFMA j: a K fragment (j < NM) or two transposing V reads (j >= NM).
    // Value MFMA i = j - NM: key block kb = i / (2 DB), key octet tt = (i / DB) % 2, column block i % DB.
    auto read_op = [&](int j, const lds_u8 *kp, const lds_u8 *vp) {
        if (j < NM) {
            if constexpr (SWZ) return *(const lds_u32x4 *)(kp + koff[j / KB] + (j % KB) * 32 * KP);
            return *(const lds_u32x4 *)(kp + (j % KB) * 32 * KP + (j / KB) * 32);
        }
        const int i = j - NM, kb = i / (2 * DB), tt = (i / DB) % 2, db = i % DB;
        // rows k0.., columns of block db
        const int off = SWZ ? (kb * 32 + tt * 8) * VP + (int)voff[SWZ ? db : 0] : (kb * 32 + tt * 8) * VP + db * 64;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp + off));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp + off + 4 * VP));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 v = {lo2[0], lo2[1], hi2[0], hi2[1]};
        return v;
    };
    // dword w of key octet g of P: keys 8 (g % 2) + 2 w, +1 of key block g / 2, rounded to T
    auto cvt = [&](const f32x16 (&pr)[KB], int g, int w) {
        const int kb = g / 2, r = 8 * (g % 2) + 2 * w;
        return Elem<T>::pack2(pr[kb][r], pr[kb][r + 1]);
    };

    // One step.  QK: also compute the scores s_next of the next tile (from kbuf) and the
    // probabilities of s_cur (overwritten in place); otherwise s_cur already holds them.
    // Returns the in-lane max of s_next (unmasked); sets psum to this tile's row sum (psum is 0 on entry).
    // copy(integral_constant<i>) is called after score MFMA 2 i + 1 for each of the step's copy
    // instructions (a no-op where the caller issues the copies itself).
    auto step = [&](auto qk_tag, int kbuf, int vbuf, f32x16 (&s_next)[KB], f32x16 (&s_cur)[KB], float mt_cur,
                    float &psum, auto &&copy) {
        constexpr bool QK = decltype(qk_tag)::value;
        float mc = 0.f;  // m * c of tile t, set by the running-max update inside the sequence
        constexpr int J0 = QK ? 0 : NM;  // first MFMA of the sequence
        const lds_u8 *kp = kb_ptr(kbuf) + k_rd;
        const lds_u8 *vp = vb_ptr(vbuf) + v_rd;
        if constexpr (QK) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s_next[kb][r] = 0.f;
        }
        u32x4 a[RA + 1];
#pragma unroll
        for (int j = J0; j < J0 + RA; ++j) a[j % (RA + 1)] = read_op(j, kp, vp);
        // the wave issuing the score half of a step (its exp2 work) takes issue priority over
        // a wave in its value half, which keeps the two waves of a SIMD half a step apart
        if constexpr (QK) __builtin_amdgcn_s_setprio(1);
        float mt = -INFINITY;
        u32x4 bop[2];
        static_for<J0, 2 * NM>([&](auto jc) {  // every MFMA index a compile-time constant
            constexpr int j = decltype(jc)::value;
            if constexpr (j == NM) __builtin_amdgcn_s_setprio(0);
            if constexpr (j + RA < 2 * NM) a[(j + RA) % (RA + 1)] = read_op(j + RA, kp, vp);
            if constexpr (j < NM) {
                s_next[j % KB] = Elem<T>::mfma(a[j % (RA + 1)], qreg[j / KB], s_next[j % KB]);
                if constexpr (j % 2 == 1 && j / 2 < LOADS_PER_TILE)  // next tiles' copies, when spread
                    copy(std::integral_constant<int, j / 2>{});
                // the running-max update of tile t (and the rare rescale of O) runs while the
                // first score MFMAs of tile t+1 execute; the probabilities follow
                if constexpr (j == NPRE - 1) mc = update_max(mt_cur);
                if constexpr (j >= NPRE) {
                    constexpr int SLOTS = NM - NPRE;
#pragma unroll
                    for (int pr = (j - NPRE) * (VALS / 2) / SLOTS; pr < (j - NPRE + 1) * (VALS / 2) / SLOTS; ++pr) {
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int v = 2 * pr + e;
                            s_cur[v / 16][v % 16] =
                                __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[v / 16][v % 16], c, -mc));
                        }
                    }
                }
                if constexpr (j == NM - 1) {  // P octet 0 is needed by the first value MFMA
#pragma unroll
                    for (int w = 0; w < 4; ++w) bop[0][w] = cvt(s_cur, 0, w);
                }
            } else {
                constexpr int i = j - NM, g = i / DB;
                if constexpr (!QK && i == 0) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) bop[0][w] = cvt(s_cur, 0, w);
                }
                oacc[i % DB] = Elem<T>::mfma(a[j % (RA + 1)], bop[g % 2], oacc[i % DB]);
                if constexpr (g + 1 < NG) {
#pragma unroll
                    for (int w = (i % DB) * CPM; w < (i % DB + 1) * CPM; ++w) bop[(g + 1) % 2][w] = cvt(s_cur, g + 1, w);
                }
#pragma unroll
                for (int e = 0; e < VPM; ++e) {
                    const int v = i * VPM + e;
                    if (i == 0 && e == 0) psum = s_cur[v / 16][v % 16];  // (saves the add to 0)
                    else psum += s_cur[v / 16][v % 16];
                }
                if constexpr (QK) {
#pragma unroll
                    for (int e = 0; e < VPM; e += 2) {
                        const int v = i * VPM + e;
                        mt = fmaxf(mt, fmaxf(s_next[v / 16][v % 16], s_next[v / 16][v % 16 + 1]));
                    }
                }
                asm volatile("" : "+v"(mt), "+v"(psum));  // keep both chains in place
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        return mt;
    };

    // probabilities of the last tile, with no next tile to overlap
    auto probs = [&](f32x16 (&s_cur)[KB], float mc) {
#pragma unroll
        for (int v = 0; v < VALS; ++v)
            s_cur[v / 16][v % 16] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[v / 16][v % 16], c, -mc));
    };

    // scores of one tile only (the first one)
    auto scores = [&](int kbuf, f32x16 (&s)[KB]) {
        const lds_u8 *kp = kb_ptr(kbuf) + k_rd;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int j = 0; j < NM; ++j) s[j % KB] = Elem<T>::mfma(read_op(j, kp, kp), qreg[j / KB], s[j % KB]);
    };


    // Software pipeline over key tiles.  Step t reads K_{t+1} (scores of the next tile) and
    // V_t from LDS, and issues the loads of K_{t+2} and V_{t+1} into the buffers that step t-1
    // finished reading; the one barrier per tile publishes them.
    f32x16 s_cur[KB], s_nxt[KB];
    float mt_pending = -INFINITY;  // in-lane max of the scores whose running-max update is pending
    if (n_loc > 0) {
        load_k(0, 0);
        load_v(0, 0);
        load_k(1, 1);
        wait_loads();
        __syncthreads();
        scores(0, s_cur);
        mt_pending = mask_max(0, s_cur, t0 + grp < kr.n_full);
        __syncthreads();  // every wave has read K_0 before its buffer is refilled
    }
    // one full step t: probabilities and P V of tile t (scores in cur), scores of tile t+1 into
    // nxt.  With ph = t % 2, K_{t+1} and V_t are read from buffers 1 - ph and ph, and the copies
    // of K_{t+2} and V_{t+1} go to buffers ph and 1 - ph.  ph is a compile-time constant (the
    // loop below runs steps in pairs), so every buffer is a fixed LDS object.
    //
    // On the full-grid shape (one 8-wave workgroup per CU) the step's copy instructions go out one
    // after every other score MFMA rather than all at the top of the step, where the eight waves'
    // copies would queue behind each other in the CU's address unit while the matrix core idles.
    // Small grids (two key groups, the key-split mode) keep them at the top, where the copies'
    // lead matters more than their issue cost.
    constexpr bool SPREAD = W == 8 && KG == 1 && !SPLIT;
    static_assert(!SPREAD || LOADS_PER_TILE <= NM / 2, "one copy after every other score MFMA covers the tile");
    auto body = [&](auto ph_c, int t, f32x16 (&cur)[KB], f32x16 (&nxt)[KB]) {
        constexpr int ph = decltype(ph_c)::value;
        auto copy = [&](auto ic) {  // copy instruction i of K_{t+2} (i < KI) or V_{t+1}
            constexpr int i = decltype(ic)::value;
            if constexpr (i < KI) load_k_one(t + 2, ph, i);
            else load_v_one(t + 1, 1 - ph, i - KI);
        };
        if constexpr (!SPREAD) {
            load_k(t + 2, ph);  // rows past N (or a tile past the end) read as zero
            load_v(t + 1, 1 - ph);
        }
        float psum = 0.f;
        float mt = SPREAD ? step(std::true_type{}, 1 - ph, ph, nxt, cur, mt_pending, psum, copy)
                          : step(std::true_type{}, 1 - ph, ph, nxt, cur, mt_pending, psum, [](auto) {});
        l_part += psum;
        if (t0 + KG * (t + 1) + grp >= kr.n_full) mt = mask_max(t + 1, nxt);  // diagonal band / ragged tail
        mt_pending = mt;
        wait_loads();
        __syncthreads();
    };
    // Steps run in pairs, the two score arrays swapping roles (no copies) as the buffers do;
    // the second step of a pair sits behind a uniform exit test.
    const int n_steps = n_loc - 1;
    for (int t = 0; t < n_steps; t += 2) {
        body(std::integral_constant<int, 0>{}, t, s_cur, s_nxt);
        if (t + 1 < n_steps) body(std::integral_constant<int, 1>{}, t + 1, s_nxt, s_cur);
    }
    if (n_steps > 0 && (n_steps & 1)) {  // the last tile's scores are in s_nxt
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s_cur[kb] = s_nxt[kb];
    }
    const int vb_cur = n_steps > 0 ? n_steps % 2 : 0;  // buffer of the last V tile
    if (n_loc > 0) {  // last tile: no scores to prefetch
        const float mc = update_max(mt_pending);
        probs(s_cur, mc);
        float psum = 0.f;
        step(std::false_type{}, 0, vb_cur, s_nxt, s_cur, -INFINITY, psum, [](auto) {});
        l_part += psum;
    }

    if constexpr (KG == 2) {
        // Merge of the two key groups' states, lane by lane (both groups hold the same rows in the
        // same layout).  Group k keeps the output column blocks [k DB/2, (k+1) DB/2): it hands the
        // other half of its O accumulators, its running max and its partial sum to the other group
        // through LDS, and both groups form the merged state of their own half with the same
        // arithmetic (R12's rescale-and-add, group 0's term as the product inside the FMA).  Each
        // group then stores its half of every row.
        __attribute__((address_space(3))) float *xf = (__attribute__((address_space(3))) float *)smem;
        constexpr int HB = DB / 2, NVH = HB * 16, REG = NVH + 2;  // floats per lane a group hands over
        static_assert(2 * REG * 64 * WG * 4 <= KG * GROUP_BYTES, "merge area inside the tile buffers");
        const int slot = wave * 64 + lane;
        __attribute__((address_space(3))) float *mine = xf + grp * REG * 64 * WG;
        const __attribute__((address_space(3))) float *other = xf + (1 - grp) * REG * 64 * WG;
        wait_loads();         // no load into LDS still in flight (the look-ahead ones included)
        __syncthreads();      // and every wave is done with the tile buffers
        if (grp == 0) {
#pragma unroll
            for (int db = 0; db < HB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[(db * 16 + r) * 64 * WG + slot] = oacc[HB + db][r];
        } else {
#pragma unroll
            for (int db = 0; db < HB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[(db * 16 + r) * 64 * WG + slot] = oacc[db][r];
        }
        mine[NVH * 64 * WG + slot] = m_run;
        mine[(NVH + 1) * 64 * WG + slot] = l_part;
        __syncthreads();
        const float m_o = other[NVH * 64 * WG + slot], l_o = other[(NVH + 1) * 64 * WG + slot];
        const float m0 = grp == 0 ? m_run : m_o, m1 = grp == 0 ? m_o : m_run;  // group 0's, group 1's
        const float l0 = grp == 0 ? l_part : l_o, l1 = grp == 0 ? l_o : l_part;
        const float m = fmaxf(m0, m1);
        const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m0 - m) * c);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * c);
        l_part = __builtin_fmaf(a1, l1, a0 * l0);
        if (grp == 0) {
#pragma unroll
            for (int db = 0; db < HB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[db][r] = __builtin_fmaf(a1, other[(db * 16 + r) * 64 * WG + slot], a0 * oacc[db][r]);
        } else {
#pragma unroll
            for (int db = 0; db < HB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[HB + db][r] = __builtin_fmaf(a1, oacc[HB + db][r], a0 * other[(db * 16 + r) * 64 * WG + slot]);
        }
        m_run = m;
    }

    // ---- A8: epilogue -- normalise once, write O and the logsumexp
    float l_tot;
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, l_part),
                                                   __builtin_bit_cast(unsigned, l_part), false, false);
        l_tot = __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
    }
    if (qvalid) {  // with two key groups each stores its half of the row's columns
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float lse = l_tot > 0.f ? (m_run * c + __builtin_log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
        const size_t row = ((size_t)tc.b * p.Hq + qhead) * (size_t)M + qpos;
        bool partial = false;
        if constexpr (SPLIT) partial = n_split > 1;
        if (partial) {  // this share's normalised fp32 output and lse, for the merge
            if constexpr (SPLIT) {
                const size_t slot = ((size_t)unit * p.slots + p.prefix[rank] + split) * p.slot_rows + (qrow - m0);
                f32x4 *dst = (f32x4 *)(p.ws_o + slot * D);
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const f32x4 w4 = {oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv,
                                          oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv};
                        dst[(db * 32 + hh * 16) / 4 + r4] = w4;
                    }
                if (hh == 0) p.ws_lse[slot] = lse;
            }
        } else {
            T *og = (T *)p.o + tc.b * p.o_sb + qhead * p.o_sh + qpos * p.o_ss;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if (KG == 2 && (db < DB / 2) != (grp == 0)) continue;
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
            if (hh == 0 && grp == 0) p.lse[row] = lse;
        }
    }
}

template <typename T, int D, bool CAUSAL, int W, int KG>
__global__ __launch_bounds__(64 * W, 2) void fa_fwd_kernel(Params p)
{
    fa_fwd_body<T, D, CAUSAL, W, false, KG>(p);
}

// one share of a query tile's keys (key-split mode)
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa_fwd_split_kernel(SplitParams p)
{
    fa_fwd_body<T, D, CAUSAL, 4, true, 1>(p);
}

// Merge of the key shares of the split query tiles: with share lse_s (natural log) and
// normalised share output O_s, lse = log sum_s exp(lse_s) and O = sum_s exp(lse_s - lse) O_s.
// A share that saw no key of a row has lse_s = -inf and weight 0; a row no share saw gets
// O = 0 and lse = -inf.  D/4 lanes per row, 4 columns each.
constexpr int kMergeRegShares = 16;  // shares a merge thread holds in registers
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(SplitParams p)
{
    constexpr int BM = 128, LPR = D / 4, RPB = 256 / LPR;
    {  // every line of the launch parameters requested at once (as in the forward kernels)
        typedef const __attribute__((address_space(4))) unsigned karg_u32;
        karg_u32 *ka = (karg_u32 *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" ::"s"(ka[0]), "s"(ka[16]), "s"(ka[32]), "s"(ka[48]), "s"(ka[64]));
    }
    const int SR = p.slot_rows, units_per_b = p.Hq / p.pack;
    // blockIdx.y is the query-tile rank, so the share table is read with scalar loads (a per-lane
    // index would make it a vector load from the argument segment: one more memory round trip
    // before any partial result can be addressed); blockIdx.x covers (unit, row of the slot)
    const int rank = blockIdx.y;
    const long long r = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    if (r >= (long long)p.B * units_per_b * SR) return;
    const int col = (threadIdx.x % LPR) * 4;
    const long long unit = r / SR;
    const int ri = (int)(r % SR);
    const int rl = (p.causal ? p.n_qt - 1 - rank : rank) * BM + ri;  // row of the unit
    if (rl >= p.pack * p.M) return;
    const int b = (int)(unit / units_per_b), h = (int)(unit % units_per_b) * p.pack + rl / p.M, i = rl % p.M;
    const int base = p.prefix[rank], ns = p.prefix[rank + 1] - base;
    const size_t s0 = ((size_t)unit * p.slots + base) * SR + ri;  // share s is slot s0 + s * SR
    float m = -INFINITY;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (ns <= kMergeRegShares) {
        // every partial lse and output row loaded at once (one memory round trip instead of two),
        // then the same arithmetic in the same order as the general path below
        float ls[kMergeRegShares];
        f32x4 os[kMergeRegShares];
#pragma unroll
        for (int s = 0; s < kMergeRegShares; ++s) {
            if (s < ns) {
                const size_t slot = s0 + (size_t)s * SR;
                ls[s] = p.ws_lse[slot];
                os[s] = *(const f32x4 *)(p.ws_o + slot * D + col);
            }
        }
#pragma unroll
        for (int s = 0; s < kMergeRegShares; ++s)
            if (s < ns) m = fmaxf(m, ls[s]);
        if (m != -INFINITY) {
#pragma unroll
            for (int s = 0; s < kMergeRegShares; ++s) {
                if (s < ns) {
                    const float w = __expf(ls[s] - m);
                    wsum += w;
                    acc += w * os[s];
                }
            }
        }
    } else {
        for (int s = 0; s < ns; ++s) m = fmaxf(m, p.ws_lse[s0 + (size_t)s * SR]);
        if (m != -INFINITY) {
            for (int s = 0; s < ns; ++s) {
                const size_t slot = s0 + (size_t)s * SR;
                const float w = __expf(p.ws_lse[slot] - m);
                wsum += w;
                const f32x4 os = *(const f32x4 *)(p.ws_o + slot * D + col);
                acc += w * os;
            }
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const size_t row = ((size_t)b * p.Hq + h) * p.M + i;
    u32x2 w;
    w[0] = Elem<T>::pack2(acc[0] * inv, acc[1] * inv);
    w[1] = Elem<T>::pack2(acc[2] * inv, acc[3] * inv);
    *(u32x2 *)((T *)p.o + b * p.o_sb + h * p.o_sh + i * p.o_ss + col) = w;
    if (col == 0) p.lse[row] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

// ------------------------------------------------------------------ host side

// Launch plan: at D = 128, 8-wave workgroups over 256 query rows when they alone fill every
// CU once; 128-row query tiles otherwise -- small grids need the larger workgroup count, and
// at D = 64 two independent 4-wave workgroups per CU measured 7-8 % faster than one 8-wave
// workgroup.  A 128-row grid that leaves CUs with one workgroup at most runs 8-wave
// workgroups with two key groups when the longest key range has kMinKgTiles tiles or more:
// with a single 4-wave workgroup on a CU each SIMD runs one wave, and the second group's wave
// adds throughput (measured about 8 % per key tile with every CU busy, 17 % with 32
// workgroups), while the merge and the larger workgroup add a fixed cost (about 2 us) that
// short key ranges do not win back.
constexpr int kNumCUs = 256;      // compute units of an MI355X
constexpr int kMinKgTiles = 16;   // key tiles of the longest range for two key groups
struct LaunchShape {
    int W;   // waves per workgroup
    int KG;  // key groups
};
static bool tiles_256(int B, int Hq, int M, int D)
{
    return D == 128 && (long long)B * Hq * ((M + 255) / 256) >= kNumCUs;
}
static LaunchShape launch_shape(int B, int Hq, int M, int N, int D)
{
    if (tiles_256(B, Hq, M, D)) return {8, 1};
    const long long wg128 = (long long)B * Hq * ((M + 127) / 128);
    // the longest key range of any query tile is the whole key sequence (the last tile's, when causal)
    if (wg128 <= kNumCUs && (N + kBN - 1) / kBN >= kMinKgTiles) return {8, 2};
    return {4, 1};
}

static int tile_shape(int B, int Hq, int M, int D, int *BM, int *BN)
{
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    *BM = tiles_256(B, Hq, M, D) ? 256 : 128;
    *BN = kBN;
    return FA_OK;
}

template <typename T, int D, int W, int KG>
static hipError_t launch_w(const Params &p, bool causal, hipStream_t stream)
{
    dim3 grid((unsigned)p.total), block(64 * W);
    if (causal)
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, true, W, KG>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, false, W, KG>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const Params &p, LaunchShape ls, bool causal, hipStream_t stream)
{
    if (ls.KG == 2) return launch_w<T, D, 8, 2>(p, causal, stream);
    return ls.W == 8 ? launch_w<T, D, 8, 1>(p, causal, stream) : launch_w<T, D, 4, 1>(p, causal, stream);
}

template <typename T>
static hipError_t launch_t(const Params &p, int D, LaunchShape ls, bool causal, hipStream_t stream)
{
    return D == 128 ? launch_d<T, 128>(p, ls, causal, stream) : launch_d<T, 64>(p, ls, causal, stream);
}

// ---- key-split mode (4-wave workgroups, 128-row query tiles)

constexpr int kSplitBM = 128;
// largest K/V row stride (elements): a key tile's 32-bit buffer range must hold 63 rows plus one
constexpr long long kMaxKvRowStride = ((0x7fff0000LL / 2) - 128) / 63;
constexpr int kSplitTargetWgs = 512;  // two 4-wave workgroups per CU
constexpr int kSplitMinWgs = 256;     // one per CU
constexpr int kSplitMinTiles = 8;     // smallest share the automatic plan hands one workgroup
constexpr int kSplitMinRange = 32;    // the automatic plan splits only query tiles this long or longer

struct SplitPlan {
    SplitParams sp;
    int tiles;          // key tiles per share (the largest a workgroup gets)
    size_t ws_bytes;    // workspace the partial results need (0: no tile is split)
    size_t ws_o_offset; // byte offset of the partial outputs inside the workspace
};

// Shares per query tile: with at most `tiles` key tiles a share, a tile visiting n key tiles
// gets ceil(n / tiles) shares.  tiles <= 0 asks for the automatic choice: no split when the
// plain 4-wave grid already has kSplitTargetWgs workgroups or no query tile visits
// kSplitMinRange key tiles (the partial results' round trip and the merge launch would cost
// more than the balance gains), else the total key-tile work spread over about
// kSplitTargetWgs workgroups, at least kSplitMinTiles tiles each.  A share's partial output
// (slot_rows fp32 rows, written once and read once by the merge) costs slot_rows / 32 key
// tiles of K/V bytes, so shares are also made at least slot_rows / 4 tiles long (that round
// trip then adds at most 1/8 to the share's traffic), as long as the grid keeps one
// workgroup per CU.
static int split_plan(int B, int Hq, int Hkv, int M, int N, int D, bool causal, int tiles, SplitPlan *pl)
{
    // short queries: stack the query heads of a KV group into the rows of one unit
    const int g = Hq / Hkv;
    int pack = M < kSplitBM && g > 1 && ((long long)g * M + kSplitBM - 1) / kSplitBM <= kMaxSplitQt ? g : 1;
    const int R = pack * M;
    const int n_qt = (R + kSplitBM - 1) / kSplitBM;
    if (n_qt > kMaxSplitQt) return FA_ERR_UNSUPPORTED;
    int nt[kMaxSplitQt];
    long long total_tiles = 0;
    int max_tiles = 1;
    for (int r = 0; r < n_qt; ++r) {
        const int qt = causal ? n_qt - 1 - r : r;
        nt[r] = unit_kv_range(qt * kSplitBM, kSplitBM, kBN, M, N, R, causal).n_tiles;
        total_tiles += nt[r];
        if (nt[r] > max_tiles) max_tiles = nt[r];
    }
    const long long heads = (long long)B * Hq / pack;  // units
    const int slot_rows = R < kSplitBM ? R : kSplitBM;
    if (tiles <= 0) {
        if (heads * n_qt >= kSplitTargetWgs || max_tiles < kSplitMinRange) {
            tiles = max_tiles;
        } else {
            const long long work = heads * total_tiles;
            const long long t_target = (work + kSplitTargetWgs - 1) / kSplitTargetWgs;
            const long long t_cus = (work + kSplitMinWgs - 1) / kSplitMinWgs;
            const long long t_rows = (slot_rows + 3) / 4;
            long long t = t_rows < t_cus ? t_rows : t_cus;
            if (t < t_target) t = t_target;
            tiles = (int)(t < kSplitMinTiles ? kSplitMinTiles : (t > max_tiles ? max_tiles : t));
        }
    }
    SplitParams &sp = pl->sp;
    sp.prefix[0] = 0;
    sp.n_split_ranks = 0;
    for (int r = 0; r < n_qt; ++r) {
        const int ns = nt[r] > tiles ? (nt[r] + tiles - 1) / tiles : 1;
        sp.prefix[r + 1] = sp.prefix[r] + ns;
        if (ns > 1) {
            if (sp.n_split_ranks != r) return FA_ERR_INVALID_ARG;  // shares must not grow with the rank
            sp.n_split_ranks = r + 1;
        }
    }
    sp.n_qt = n_qt;
    sp.wg_per_head = sp.prefix[n_qt];
    sp.slots = sp.prefix[sp.n_split_ranks];
    sp.causal = causal ? 1 : 0;
    sp.pack = pack;
    sp.slot_rows = slot_rows;
    sp.total = heads * sp.wg_per_head;
    if (sp.slots && heads * slot_rows > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;  // the merge grid's x extent
    if (sp.total <= 0x7fffffffLL) sp.gm = make_grid_map((unsigned)sp.total, g / pack, sp.wg_per_head, Hkv);
    pl->tiles = tiles;
    const size_t rows = (size_t)heads * sp.slots * sp.slot_rows;
    pl->ws_o_offset = (rows * sizeof(float) + 255) & ~(size_t)255;
    pl->ws_bytes = sp.slots ? pl->ws_o_offset + rows * D * sizeof(float) : 0;
    return FA_OK;
}

// Scratch of the no-allocation key-split entry point: the partial results live in this
// file-scope device array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each GPU's copy is looked up
// once per device with hipGetSymbolAddress and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void *scratch_ptr[kMaxDevices];

// Device address of the scratch of the current device, which must be the stream's device (it is
// looked up on the first use on that device, with that device current).
static int scratch_for_stream(hipStream_t stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_LAUNCH;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_INVALID_ARG;
        if ((int)sdev != dev) return FA_ERR_INVALID_ARG;  // another device's scratch would be the wrong memory
    }
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_LAUNCH;
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return FA_OK;
}

template <typename T, int D>
static hipError_t launch_split_d(const SplitParams &p, bool causal, hipStream_t stream)
{
    dim3 grid((unsigned)p.total), block(256);
    if (causal)
        hipLaunchKernelGGL((fa_fwd_split_kernel<T, D, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fa_fwd_split_kernel<T, D, false>), grid, block, 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.slots == 0) return e;
    constexpr int RPB = 256 / (D / 4);
    const long long rows = (long long)p.B * (p.Hq / p.pack) * p.slot_rows;  // merge rows per split rank
    hipLaunchKernelGGL((fa_merge_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB), (unsigned)p.n_split_ranks),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_split(const SplitParams &p, int D, bool causal, hipStream_t stream)
{
    return D == 128 ? launch_split_d<T, 128>(p, causal, stream) : launch_split_d<T, 64>(p, causal, stream);
}

// Strides (in elements) of one [B, H, S, D] tensor: the caller's, or the contiguous ones for
// NULL.  Every row must start 16-byte aligned (strides multiples of 8 elements), strides are
// non-negative, and the largest element offset must fit in int64.  K and V rows are addressed
// with 32-bit offsets inside one key tile, which bounds their row stride.
static int strides_of(const fa_strides *st, int B, int H, int S, int D, bool kv, long long *sb, long long *sh,
                      long long *ss)
{
    if (!st) {
        *ss = D;
        *sh = (long long)S * D;
        *sb = (long long)H * S * D;
        return FA_OK;
    }
    if (st->batch < 0 || st->head < 0 || st->row < 0) return FA_ERR_INVALID_ARG;
    if ((st->batch | st->head | st->row) & 7) return FA_ERR_UNSUPPORTED;
    const double last = (double)(B - 1) * st->batch + (double)(H - 1) * st->head + (double)(S - 1) * st->row + D;
    if (last > 9.0e18) return FA_ERR_INVALID_ARG;
    if (kv && st->row > kMaxKvRowStride) return FA_ERR_UNSUPPORTED;
    *sb = st->batch;
    *sh = st->head;
    *ss = st->row;
    return FA_OK;
}

// argument checks shared by the entry points; fills the sizes and strides of p
static int check_args(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M,
                      int N, int D, const fa_strides *qs, const fa_strides *ks, const fa_strides *vs,
                      const fa_strides *os, float scale, int dtype, Params *p)
{
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || N <= 0 || D <= 0) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
    // element counts must fit in int64 (they do for any int sizes below 2^15 each; check anyway)
    const double nq = (double)B * Hq * M * D, nk = (double)B * Hkv * N * D;
    if (nq > 9.0e18 || nk > 9.0e18) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    int rc;
    if ((rc = strides_of(qs, B, Hq, M, D, false, &p->q_sb, &p->q_sh, &p->q_ss)) != FA_OK) return rc;
    if ((rc = strides_of(ks, B, Hkv, N, D, true, &p->k_sb, &p->k_sh, &p->k_ss)) != FA_OK) return rc;
    if ((rc = strides_of(vs, B, Hkv, N, D, true, &p->v_sb, &p->v_sh, &p->v_ss)) != FA_OK) return rc;
    if ((rc = strides_of(os, B, Hq, M, D, false, &p->o_sb, &p->o_sh, &p->o_ss)) != FA_OK) return rc;
    const uintptr_t align = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse;
    if (align & 15u) return FA_ERR_UNSUPPORTED;
    p->q = q;
    p->k = k;
    p->v = v;
    p->o = o;
    p->lse = lse;
    p->B = B;
    p->Hq = Hq;
    p->Hkv = Hkv;
    p->M = M;
    p->N = N;
    p->c = scale * 1.44269504088896340736f;  // log2(e)
    return FA_OK;
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
    case FA_ERR_SCRATCH_TOO_SMALL:
        return "the partial results need more than the no-allocation entry point's scratch (FA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
    }
}

int fa_tile_shape(int B, int Hq, int M, int D, int *BM, int *BN)
{
    if (!BM || !BN || B <= 0 || Hq <= 0 || M <= 0) return FA_ERR_INVALID_ARG;
    return fa::tile_shape(B, Hq, M, D, BM, BN);
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
    if (fa::tile_shape(B, Hq, M, D, &BM, &BN) != FA_OK) return FA_ERR_INVALID_ARG;
    const int n_qt = (M + BM - 1) / BM;
    const long long total = (long long)B * Hq * n_qt;
    if (wg < 0 || wg >= total) return FA_ERR_INVALID_ARG;
    if (total > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;  // the kernels' grid limit
    const fa::GridMap gm = fa::make_grid_map((unsigned)total, Hq / Hkv, n_qt, Hkv);  // the kernel's mapping
    fa::TileCoord c = fa::logical_tile(fa::xcd_remap((unsigned)wg, gm), gm, causal != 0);
    *b = c.b;
    *h = c.h;
    *q_tile = c.qt;
    return FA_OK;
}

int fa_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M,
                   int N, int D, const fa_strides *q_strides, const fa_strides *k_strides,
                   const fa_strides *v_strides, const fa_strides *o_strides, float scale, int causal, int dtype,
                   void *stream)
{
    fa::Params p;
    int rc = fa::check_args(q, k, v, o, lse, B, Hq, Hkv, M, N, D, q_strides, k_strides, v_strides, o_strides, scale,
                            dtype, &p);
    if (rc != FA_OK) return rc;
    int BM, BN;
    if (fa::tile_shape(B, Hq, M, D, &BM, &BN) != FA_OK) return FA_ERR_UNSUPPORTED;
    p.n_qt = (M + BM - 1) / BM;
    p.total = (long long)B * Hq * p.n_qt;
    if (p.total > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;  // one-dimensional grid limit
    p.gm = fa::make_grid_map((unsigned)p.total, Hq / Hkv, p.n_qt, Hkv);

    hipStream_t s = (hipStream_t)stream;
    const fa::LaunchShape ls = fa::launch_shape(B, Hq, M, N, D);
    hipError_t err = dtype == FA_F16 ? fa::launch_t<_Float16>(p, D, ls, causal != 0, s)
                                     : fa::launch_t<__bf16>(p, D, ls, causal != 0, s);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M, int N,
           int D, float scale, int causal, int dtype, void *stream)
{
    return fa_fwd_strided(q, k, v, o, lse, B, Hq, Hkv, M, N, D, nullptr, nullptr, nullptr, nullptr, scale, causal,
                          dtype, stream);
}

int fa_splitkv_plan(int B, int Hq, int Hkv, int M, int N, int D, int causal, int tiles_per_split, int *tiles_used,
                    long long *workgroups, size_t *workspace_bytes)
{
    if (!tiles_used || !workgroups || !workspace_bytes) return FA_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || N <= 0 || D <= 0 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    fa::SplitPlan pl;
    const int rc = fa::split_plan(B, Hq, Hkv, M, N, D, causal != 0, tiles_per_split, &pl);
    if (rc != FA_OK) return rc;
    *tiles_used = pl.tiles;
    *workgroups = pl.sp.total;
    *workspace_bytes = pl.ws_bytes;
    return FA_OK;
}

int fa_fwd_splitkv_strided(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv,
                           int M, int N, int D, const fa_strides *q_strides, const fa_strides *k_strides,
                           const fa_strides *v_strides, const fa_strides *o_strides, float scale, int causal,
                           int dtype, int tiles_per_split, void *workspace, size_t workspace_bytes, void *stream)
{
    fa::SplitPlan pl;
    int rc = fa::check_args(q, k, v, o, lse, B, Hq, Hkv, M, N, D, q_strides, k_strides, v_strides, o_strides, scale,
                            dtype, &pl.sp);
    if (rc != FA_OK) return rc;
    rc = fa::split_plan(B, Hq, Hkv, M, N, D, causal != 0, tiles_per_split, &pl);
    if (rc != FA_OK) return rc;
    if (pl.sp.total > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (pl.ws_bytes) {
        if (!workspace || workspace_bytes < pl.ws_bytes) return FA_ERR_INVALID_ARG;
        if ((uintptr_t)workspace & 255u) return FA_ERR_UNSUPPORTED;
        pl.sp.ws_lse = (float *)workspace;
        pl.sp.ws_o = (float *)((char *)workspace + pl.ws_o_offset);
    } else {
        pl.sp.ws_lse = nullptr;
        pl.sp.ws_o = nullptr;
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t err = dtype == FA_F16 ? fa::launch_split<_Float16>(pl.sp, D, causal != 0, s)
                                     : fa::launch_split<__bf16>(pl.sp, D, causal != 0, s);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M,
                   int N, int D, float scale, int causal, int dtype, int tiles_per_split, void *workspace,
                   size_t workspace_bytes, void *stream)
{
    return fa_fwd_splitkv_strided(q, k, v, o, lse, B, Hq, Hkv, M, N, D, nullptr, nullptr, nullptr, nullptr, scale,
                                  causal, dtype, tiles_per_split, workspace, workspace_bytes, stream);
}

int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv,
                           int M, int N, int D, float scale, int causal, int dtype, int tiles_per_split, void *stream)
{
    // every check that needs no device first, so that a bad call never touches the GPU
    fa::SplitPlan pl;
    int rc = fa::check_args(q, k, v, o, lse, B, Hq, Hkv, M, N, D, nullptr, nullptr, nullptr, nullptr, scale, dtype,
                            &pl.sp);
    if (rc != FA_OK) return rc;
    rc = fa::split_plan(B, Hq, Hkv, M, N, D, causal != 0, tiles_per_split, &pl);
    if (rc != FA_OK) return rc;
    if (pl.sp.total > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (pl.ws_bytes > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH_TOO_SMALL;
    hipStream_t s = (hipStream_t)stream;
    void *ws = nullptr;
    if (pl.ws_bytes) {
        if ((rc = fa::scratch_for_stream(s, &ws)) != FA_OK) return rc;
        pl.sp.ws_lse = (float *)ws;
        pl.sp.ws_o = (float *)((char *)ws + pl.ws_o_offset);
    } else {
        pl.sp.ws_lse = nullptr;
        pl.sp.ws_o = nullptr;
    }
    hipError_t err = dtype == FA_F16 ? fa::launch_split<_Float16>(pl.sp, D, causal != 0, s)
                                     : fa::launch_split<__bf16>(pl.sp, D, causal != 0, s);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
