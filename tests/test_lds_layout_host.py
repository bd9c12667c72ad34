"""Host model of the forward kernel's D = 128 LDS tiles (256-byte rows, XOR-swizzled 16-byte units).

The forward copies K and V tiles from HBM into LDS with one 16-byte unit per lane and reads them
back as MFMA operands: K with plain 16-byte reads (16-lane passes), V with the transposing 8-byte
read (32-lane passes).  This test replays, in Python, the unit each copy lane writes and the
address each reading lane uses, for both wave counts, and checks that

* every read finds the element of K or V that the MFMA operand layout asks for, and
* every read pass touches distinct LDS banks (gfx950: 64 banks of 4 bytes).

It mirrors the index formulas of `fa_fwd.hip` (the swizzle functions, the copy-lane source
offsets and the per-lane read offsets); a change there that is not made here fails it.
"""
import pytest

KP = VP = 256          # row pitch in bytes
UNITS = 16             # 16-byte units per row
K_INSTR = 16           # 1 KiB copy instructions per 64-row tile


def pi32(i):
    """Slot order inside a 32-key block: slot i holds key pi32(i)."""
    return 16 * ((i >> 2) & 1) + ((i >> 3) << 2) + (i & 3)


def k_swz(r):
    return 4 * (r & 3) + ((r >> 2) & 3)


def v_swz(r):
    return 4 * (r & 3)


def k_tile_map(waves):
    """(LDS slot, physical unit) -> (key, logical unit) written by the copy lanes."""
    m = {}
    for wave in range(waves):
        for i in range(K_INSTR // waves):
            for lane in range(64):
                u = (wave + waves * i) * 64 + lane
                slot, unit = u // UNITS, u % UNITS
                key = (slot & ~31) | pi32(slot & 31)
                m[(slot, unit)] = (key, unit ^ k_swz(slot))
    return m


def v_tile_map(waves):
    m = {}
    for wave in range(waves):
        for i in range(K_INSTR // waves):
            for lane in range(64):
                u = (wave + waves * i) * 64 + lane
                row, unit = u // UNITS, u % UNITS
                m[(row, unit)] = (row, unit ^ v_swz(row))
    return m


def k_read_off(lane, ks, kb):
    ql, hh = lane & 31, lane >> 5
    return ql * KP + (((2 * ks + hh) ^ k_swz(ql)) * 16) + kb * 32 * KP


def v_read_off(lane, db):
    hh, g, s = lane >> 5, (lane >> 4) & 1, lane & 15
    e, j = s >> 2, s & 3
    return (hh * 16 + e) * VP + (4 * (db ^ e) + 2 * (j & 1) + g) * 16 + 8 * (j >> 1)


@pytest.mark.parametrize("waves", [4, 8])
def test_copies_fill_every_unit_once(waves):
    km, vm = k_tile_map(waves), v_tile_map(waves)
    assert len(km) == 64 * UNITS and len(vm) == 64 * UNITS
    assert sorted(km.values()) == [(k, u) for k in range(64) for u in range(UNITS)]
    assert sorted(vm.values()) == [(r, u) for r in range(64) for u in range(UNITS)]


@pytest.mark.parametrize("waves", [4, 8])
def test_k_reads_find_operand(waves):
    # lane (ql, hh) of k-step ks in key block kb wants K[kb*32 + pi32(ql)][16 ks + 8 hh .. +8]
    km = k_tile_map(waves)
    for lane in range(64):
        ql, hh = lane & 31, lane >> 5
        for ks in range(8):
            for kb in range(2):
                off = k_read_off(lane, ks, kb)
                assert off % 16 == 0
                key, unit = km[(off // KP, (off % KP) // 16)]
                assert key == kb * 32 + pi32(ql) and unit == 2 * ks + hh


@pytest.mark.parametrize("waves", [4, 8])
def test_v_transposed_reads_find_operand(waves):
    # the transposing read of lane (hh, g, e, j) covers row kb*32 + 16 hh + 8 tt + 4 hi + e at
    # the 4-column chunk 16 (j & 1) + 8 g + 4 (j >> 1) of column block db
    vm = v_tile_map(waves)
    for lane in range(64):
        hh, g, s = lane >> 5, (lane >> 4) & 1, lane & 15
        e, j = s >> 2, s & 3
        for db in range(4):
            for kb in range(2):
                for tt in range(2):
                    for hi in range(2):
                        off = (kb * 32 + tt * 8) * VP + v_read_off(lane, db) + hi * 4 * VP
                        assert off % 8 == 0
                        row, unit = vm[(off // VP, (off % VP) // 16)]
                        assert row == kb * 32 + 16 * hh + 8 * tt + 4 * hi + e
                        col = unit * 8 + (off % 16) // 2
                        assert col == 32 * db + 16 * (j & 1) + 8 * g + 4 * (j >> 1)


def test_k_read_passes_conflict_free():
    # a 16-byte read runs in passes of 16 lanes; each must cover all 16 four-bank groups
    for ks in range(8):
        for kb in range(2):
            for first in (0, 16, 32, 48):
                groups = {(k_read_off(first + q, ks, kb) // 16) % 16 for q in range(16)}
                assert len(groups) == 16


def test_v_read_passes_conflict_free():
    # a transposing 8-byte read runs in passes of 32 lanes; each must cover all 64 banks
    for db in range(4):
        for first in (0, 32):
            banks = set()
            for q in range(32):
                b = (v_read_off(first + q, db) // 4) % 64
                banks.update((b, b + 1))
            assert len(banks) == 64


def test_copy_writes_conflict_free():
    # a copy instruction writes 1 KiB contiguously: 64 lanes x 16 bytes, 4 full bank sweeps
    for j in range(K_INSTR):
        for first in (0, 16, 32, 48):
            groups = {((j * 64 + first + q) * 16 // 16) % 16 for q in range(16)}
            assert len(groups) == 16
