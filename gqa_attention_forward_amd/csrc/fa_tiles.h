// fa_tiles.h -- integer tile math of the attention forward, shared by the gfx950 kernel
// and the host-side launch/introspection code.  No floating point here.
//
// Key-tile classification per query tile ("从零开始写Qwen3", FlashAttention speed-up
// article, sections "改进2-KV只读取下三角" and "改进3-两阶段计算"): tiles that no row of the
// query tile can see are never visited; tiles every row sees entirely run without mask
// code; the remaining band (the diagonal, plus a ragged last key tile) runs masked.
// With the bottom-right causal alignment key j is visible to query i iff j <= i + (N - M).
//
// Grid order ("改进1-使用正确的grid" on the same page): the query-tile index varies fastest
// inside one KV group, so every workgroup that reads the same K/V runs close together in
// time; on MI355X the linear workgroup id is first remapped so that such workgroups land
// on the same XCD (each XCD has its own L2), and causal query tiles are issued longest-first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin across them

struct KvRange {
    int n_tiles;  // key tiles [0, n_tiles) are visited
    int n_full;   // of which [0, n_full) need no mask
};

__host__ __device__ inline int clampi(long long x, long long lo, long long hi)
{
    return (int)(x < lo ? lo : (x > hi ? hi : x));
}

// Key tiles for a query tile whose rows have query positions first .. last (first <= last).
__host__ __device__ inline KvRange kv_range_rows(int first, int last, int BN, int M, int N, bool causal)
{
    KvRange r;
    int n_whole = N / BN;  // key tiles with no ragged tail
    if (!causal) {
        r.n_tiles = (N + BN - 1) / BN;
        r.n_full = n_whole;
        return r;
    }
    long long off = (long long)N - M;
    // keys [0, hi) are visible to at least the last row of the tile
    int hi = clampi((long long)last + 1 + off, 0, N);
    r.n_tiles = (hi + BN - 1) / BN;
    // a tile [n0, n0+BN) needs no mask iff its last key is visible to the first row
    int lo_keys = clampi((long long)first + 1 + off, 0, N);  // keys visible to the first row
    int nf = lo_keys / BN;
    r.n_full = nf < n_whole ? nf : n_whole;
    if (r.n_full > r.n_tiles) r.n_full = r.n_tiles;
    return r;
}

// Key tiles for the query tile whose first row is m0 (rows m0 .. m0+BM-1, clipped to M).
__host__ __device__ inline KvRange kv_range(int m0, int BM, int BN, int M, int N, bool causal)
{
    return kv_range_rows(m0, (m0 + BM < M ? m0 + BM : M) - 1, BN, M, N, causal);
}

// Key tiles for rows m0 .. m0+BM-1 (clipped to R) of a unit of R = pack * M rows in which row r
// is query position r % M of the unit's head r / M (pack query heads of one KV group stacked).
// A tile that crosses from one head into the next holds both the last and the first position.
__host__ __device__ inline KvRange unit_kv_range(int m0, int BM, int BN, int M, int N, int R, bool causal)
{
    const int r1 = (m0 + BM < R ? m0 + BM : R) - 1;
    if (m0 / M == r1 / M) return kv_range_rows(m0 % M, r1 % M, BN, M, N, causal);
    return kv_range_rows(0, M - 1, BN, M, N, causal);
}

// Division of an unsigned n < 2^31 by a divisor d >= 1 known at launch time, as a multiply-high,
// an add and a shift: with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1,
// floor(n / d) = (mulhi(n, m) + n) >> s (Granlund and Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, section 4; mulhi(n, m) <= n, so the sum fits 32 bits).  A
// workgroup's tile coordinates then cost a handful of scalar instructions instead of the long
// expansion of an integer division by a runtime value.
struct FastDiv {
    unsigned d, m, s;
};

inline FastDiv make_fastdiv(unsigned d)  // d >= 1
{
    unsigned s = 0;
    while ((1ull << s) < d) ++s;
    FastDiv f;
    f.d = d;
    f.m = (unsigned)((((1ull << s) - d) << 32) / d + 1);
    f.s = s;
    return f;
}

__host__ __device__ inline unsigned fdiv(unsigned n, const FastDiv &f)
{
    const unsigned t = (unsigned)(((unsigned long long)n * f.m) >> 32);
    return (t + n) >> f.s;
}

// Everything a workgroup needs to find its work, computed once per launch on the host.  The grid
// has total < 2^31 workgroups.  Logical index L = ((bhk * n_mid) + mid) * n_inner + inner, with
// bhk = b * Hkv + kv head.
struct GridMap {
    unsigned xcd_q, xcd_rem;  // total / kNumXcd and total % kNumXcd
    FastDiv inner;            // query heads of a KV group (per workgroup unit, in key-split mode)
    FastDiv mid;              // query-tile ranks (workgroups per unit, in key-split mode)
    FastDiv hkv;              // KV heads
};

inline GridMap make_grid_map(unsigned total, unsigned n_inner, unsigned n_mid, unsigned hkv)
{
    GridMap gm;
    gm.xcd_q = total / kNumXcd;
    gm.xcd_rem = total % kNumXcd;
    gm.inner = make_fastdiv(n_inner);
    gm.mid = make_fastdiv(n_mid);
    gm.hkv = make_fastdiv(hkv);
    return gm;
}

// Linear workgroup id -> logical work index, so that logical indices that are contiguous
// run on one XCD: XCD x receives the logical block [start_x, start_x + count_x).
static_assert((kNumXcd & (kNumXcd - 1)) == 0, "XCD count is a power of two");
__host__ __device__ inline unsigned xcd_remap(unsigned wg, const GridMap &gm)
{
    const unsigned xcd = wg % kNumXcd, slot = wg / kNumXcd;
    const unsigned start = xcd < gm.xcd_rem ? xcd * (gm.xcd_q + 1) : gm.xcd_rem * (gm.xcd_q + 1) + (xcd - gm.xcd_rem) * gm.xcd_q;
    return start + slot;
}

// Logical index -> (inner, mid, b, kv head).
struct GridPos {
    int inner, mid, b, hk;
};
__host__ __device__ inline GridPos grid_pos(unsigned L, const GridMap &gm)
{
    GridPos g;
    const unsigned rest = fdiv(L, gm.inner);
    g.inner = (int)(L - rest * gm.inner.d);
    const unsigned bhk = fdiv(rest, gm.mid);
    g.mid = (int)(rest - bhk * gm.mid.d);
    g.b = (int)fdiv(bhk, gm.hkv);
    g.hk = (int)(bhk - (unsigned)g.b * gm.hkv.d);
    return g;
}

struct TileCoord {
    int b, h, qt;
    int hk;  // KV head of query head h
};

// Logical work index -> (b, h, query tile).  Logical order: (b, kv head) outermost, then the
// query-tile rank (longest-first when causal), then the query heads of the KV group, so the
// g heads that share one K/V stream and the same key range are adjacent.  gm.inner divides by
// g = Hq / Hkv and gm.mid by the query tiles per head.
__host__ __device__ inline TileCoord logical_tile(unsigned L, const GridMap &gm, bool causal)
{
    const GridPos gp = grid_pos(L, gm);
    TileCoord c;
    c.b = gp.b;
    c.h = gp.hk * (int)gm.inner.d + gp.inner;
    c.qt = causal ? (int)gm.mid.d - 1 - gp.mid : gp.mid;
    c.hk = gp.hk;
    return c;
}

}  // namespace fa
