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

// Linear workgroup id -> logical work index, so that logical indices that are contiguous
// run on one XCD: XCD x receives the logical block [start_x, start_x + count_x).
__host__ __device__ inline long long xcd_remap(long long wg, long long total)
{
    long long xcd = wg % kNumXcd, slot = wg / kNumXcd;
    long long q = total / kNumXcd, rem = total % kNumXcd;
    long long start = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
    return start + slot;
}

struct TileCoord {
    int b, h, qt;
};

// Logical work index -> (b, h, query tile).  Logical order: (b, kv head) outermost, then the
// query-tile rank (longest-first when causal), then the query heads of the KV group, so the
// g heads that share one K/V stream and the same key range are adjacent.
__host__ __device__ inline TileCoord logical_tile(long long L, int Hq, int Hkv, int n_qt, bool causal)
{
    int g = Hq / Hkv;
    int hg = (int)(L % g);
    long long rest = L / g;
    int rank = (int)(rest % n_qt);
    long long bhk = rest / n_qt;
    TileCoord c;
    c.b = (int)(bhk / Hkv);
    int hk = (int)(bhk % Hkv);
    c.h = hk * g + hg;
    c.qt = causal ? n_qt - 1 - rank : rank;
    return c;
}

}  // namespace fa
