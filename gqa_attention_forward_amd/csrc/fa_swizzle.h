// fa_swizzle.h -- the XOR-swizzled LDS tile layout used where one tile is read both row-wise
// (16-byte MFMA operand reads: 16 lanes = 16 rows of one unit) and transposed (8-byte
// transposing reads: 32 lanes = 4 rows x 4 units).  No padded pitch serves both patterns
// without bank conflicts; storing unit u of row r at unit u ^ swz(r) does.
#pragma once

#include "fa_device.h"

namespace fa {

// unit swizzle of row r (rows of D / 8 units of 16 bytes)
template <int D> __device__ __forceinline__ constexpr int swz(int r)
{
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// ---- operand reads from a swizzled tile (base points at the tile)

// Row-wise 16-byte A operand: row `row` (lane-dependent part included), logical unit u.
template <int D> __device__ __forceinline__ u32x4 read_row(const lds_u8 *tile, int row, int u)
{
    return *(const lds_u32x4 *)(tile + row * (2 * D) + ((u ^ swz<D>(row)) * 16));
}

// Per-lane byte offsets of the transposing reads that give the A operand X^T for a k-step of 16
// rows {16 tt + 4 hh + e, 16 tt + 8 + 4 hh + e} (e = 0..3: the "lo" and "hi" reads) and the 32
// columns of block db.  Source lane 4 e + j of each 16-lane group G reads 8 bytes of row
// (base + e) at column 16 (j & 1) + 8 G + 4 (j >> 1) of the block; the hardware hands lane l
// the 4 rows of column pi(l % 32), so the accumulator register r of half hh is column
// 32 db + 16 hh + r.  Rows differ from the base by multiples of 16 (tt, 32-row blocks), which
// leave swz unchanged, so the offsets depend on (db, lo/hi) only.
template <int D> __device__ __forceinline__ unsigned tr_off(int lane, int db, int hi)
{
    const int hh = lane >> 5, G = (lane >> 4) & 1, s = lane & 15, e = s >> 2, j = s & 3;
    const int row = 8 * hi + 4 * hh + e;
    const int u = 4 * db + 2 * (j & 1) + G;
    return (unsigned)(row * (2 * D) + ((u ^ swz<D>(row)) * 16) + 8 * (j >> 1));
}

template <int D> struct TrOffsets {
    static constexpr int DB = D / 32;
    unsigned off[DB][2];
    __device__ TrOffsets(int lane)
    {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) off[db][hi] = tr_off<D>(lane, db, hi);
    }
};

// X^T operand for k-step row0 (32-row block + 16 tt), from the lane's two offsets of one column
// block (tr_off with hi = 0 and 1)
template <int D>
__device__ __forceinline__ u32x4 read_tr_at(const lds_u8 *tile, int row0, unsigned off_lo, unsigned off_hi)
{
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + row0 * (2 * D) + off_lo));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + row0 * (2 * D) + off_hi));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 v = {lo2[0], lo2[1], hi2[0], hi2[1]};
    return v;
}

// X^T operand for k-step row0 and column block db (a compile-time index wherever the offsets
// should stay in registers)
template <int D>
__device__ __forceinline__ u32x4 read_tr(const lds_u8 *tile, const TrOffsets<D> &to, int row0, int db)
{
    return read_tr_at<D>(tile, row0, to.off[db][0], to.off[db][1]);
}

}  // namespace fa
