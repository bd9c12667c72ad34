"""The C-ABI library loads, exports every symbol include/fa.h declares, and rejects bad
arguments before touching the GPU (no compute calls here: this runs without a GPU)."""
import ctypes
import os
import re

import pytest

import gqa_attention_forward_amd as fa

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def _declared():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names.update(re.findall(r"\b((?:fa|gdn)_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared()
    assert {"fa_fwd", "fa_strerror", "fa_bwd", "gdn_kkt", "gdn_chunk_fwd"} <= set(names)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_strerror_texts():
    assert fa.fa_strerror(0) == "success"
    for code in (-1, -2, -3, -4, 12345):
        assert isinstance(fa.fa_strerror(code), str) and fa.fa_strerror(code)


GOOD = dict(q=0x1000, k=0x2000, v=0x3000, o=0x4000, lse=0x5000, B=1, Hq=2, Hkv=1, M=16, N=16, D=64,
            scale=0.125, causal=1, dtype=0, stream=None)


def _call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["M"], a["N"], a["D"],
                     a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(B=0), dict(Hq=0), dict(Hkv=0), dict(M=0), dict(N=-1), dict(D=0),
    dict(Hq=3, Hkv=2), dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(dtype=2), dict(dtype=-1),
])
def test_invalid_arguments(bad):
    assert _call(**bad) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(D=96), dict(D=256), dict(D=32), dict(q=0x1008), dict(lse=0x5004)])
def test_unsupported(bad):
    assert _call(**bad) == fa.FA_ERR_UNSUPPORTED


# ------------------------------------------------------------ key-split forward plan

def _brute_key_tiles(M, N, BM, BN, causal, pack):
    """Key tiles each 128-row query tile of a unit visits, from the mask definition itself: a unit
    stacks `pack` query heads, its row r being query position r % M (rank order: longest first
    when causal)."""
    R = pack * M
    tiles = []
    for qt in range((R + BM - 1) // BM):
        rows = range(qt * BM, min(R, (qt + 1) * BM))
        seen = max(N if not causal else max(0, min(N, r % M + 1 + N - M)) for r in rows)
        tiles.append((seen + BN - 1) // BN)
    return tiles[::-1] if causal else tiles


@pytest.mark.parametrize("shape", [
    (2, 16, 8, 1024, 1024, 128, True, 5), (1, 32, 8, 1, 8192, 128, True, 8), (1, 4, 1, 300, 77, 64, True, 1),
    (1, 2, 2, 200, 333, 128, False, 2), (3, 2, 1, 1000, 1000, 64, True, 3), (1, 1, 1, 16384, 16384, 128, True, 40),
    (4, 32, 8, 64, 8192, 128, True, 16), (1, 12, 1, 100, 700, 64, True, 2), (2, 8, 1, 33, 64, 128, True, 1),
    (1, 16, 2, 127, 3000, 128, False, 5),
])
def test_splitkv_plan_matches_brute_force(shape):
    B, Hq, Hkv, M, N, D, causal, tiles = shape
    used, wgs, ws = fa.fa_splitkv_plan(B, Hq, Hkv, M, N, D, causal, tiles)
    assert used == tiles
    pack = Hq // Hkv if M < 128 else 1  # short queries: the heads of a KV group share tiles
    units = B * Hq // pack
    shares = [(n + tiles - 1) // tiles if n > tiles else 1 for n in _brute_key_tiles(M, N, 128, 64, causal, pack)]
    assert wgs == units * sum(shares)
    slots = sum(s for s in shares if s > 1)
    rows = units * slots * min(128, pack * M)
    assert ws == (0 if slots == 0 else ((rows * 4 + 255) // 256) * 256 + rows * D * 4)


def test_splitkv_auto_policy():
    # the 4-wave grid already has 512 workgroups: no split
    for B, Hq, M in [(4, 32, 512), (1, 32, 16384), (8, 64, 128)]:
        used, wgs, ws = fa.fa_splitkv_plan(B, Hq, Hq, M, 4096, 128, True, 0)
        assert ws == 0 and wgs == B * Hq * ((M + 127) // 128)
    # no query tile visits 32 key tiles: no split (the 1k causal workload)
    used, wgs, ws = fa.fa_splitkv_plan(2, 16, 8, 1024, 1024, 128, True, 0)
    assert ws == 0 and wgs == 2 * 16 * 8
    # decode-like: one query row per head, 8192 keys -> 128 key tiles; the 4 heads of each KV group
    # share one tile, and the 8 groups' tiles are spread over 512 workgroups (but >= 8 tiles a share)
    used, wgs, ws = fa.fa_splitkv_plan(1, 32, 8, 1, 8192, 128, True, 0)
    assert used == 8 and wgs == 8 * 16 and ws > 0
    # never below 8 key tiles a share (the two heads of the group stacked in one 128-row tile)
    used, wgs, ws = fa.fa_splitkv_plan(1, 2, 1, 64, 2048, 64, False, 0)
    assert used == 8 and wgs == 4
    used, wgs, ws = fa.fa_splitkv_plan(1, 2, 2, 64, 2048, 64, False, 0)  # no grouping: one tile per head
    assert used == 8 and wgs == 2 * 4
    # full 128-row tiles (64-row chunk x 4 stacked heads): a share's fp32 partial output weighs as
    # much as 4 key tiles, so shares grow to 32 tiles while the grid keeps 256 workgroups
    used, wgs, ws = fa.fa_splitkv_plan(4, 32, 8, 64, 8192, 128, True, 0)
    assert used == 32 and wgs == 4 * 8 * 2 * 4
    # decode with few rows per tile keeps the 512-workgroup spread
    used, wgs, ws = fa.fa_splitkv_plan(8, 32, 8, 1, 8192, 128, True, 0)
    assert used == 16 and wgs == 8 * 8 * 8
    # one 128-row tile on a small grid: the CU bound wins over the partial-output bound
    used, wgs, ws = fa.fa_splitkv_plan(1, 8, 8, 128, 8192, 128, False, 0)
    assert used == 8 and wgs == 8 * 16


def test_splitkv_plan_merge_grid_limit():
    """The merge kernel's grid has one row of workgroups per split query-tile rank, covering
    B * Hq * min(128, M) rows (heads not stacked): a plan beyond 2^31 - 1 such rows is refused,
    one just below the limit is planned."""
    per_b = 8 * 128  # Hq = Hkv = 8, M = 128: one 128-row tile per head, 4 key tiles, shares of 1
    with pytest.raises(fa.FaError) as e:
        fa.fa_splitkv_plan(2 ** 31 // per_b + 1, 8, 8, 128, 256, 128, True, 1)
    assert e.value.code == fa.FA_ERR_UNSUPPORTED
    used, wgs, ws = fa.fa_splitkv_plan((2 ** 31 - 1) // per_b, 8, 8, 128, 256, 128, True, 1)
    assert used == 1 and ws > 0


SPLIT_GOOD = dict(GOOD, tiles=1, ws=0x100000, ws_bytes=1 << 30)


def _call_split(**kw):
    a = dict(SPLIT_GOOD)
    a.update(kw)
    return fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["M"], a["N"],
                             a["D"], a["scale"], a["causal"], a["dtype"], a["tiles"], a["ws"], a["ws_bytes"],
                             a["stream"])


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(lse=None), dict(B=0), dict(Hq=3, Hkv=2), dict(scale=0.0), dict(dtype=2),
    dict(M=200, N=1000, ws=None), dict(M=200, N=1000, ws_bytes=1024),
])
def test_splitkv_invalid_arguments(bad):
    assert _call_split(**bad) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(D=96), dict(q=0x1008), dict(M=200, N=1000, ws=0x100080),
                                 dict(M=16385, N=64)])
def test_splitkv_unsupported(bad):
    assert _call_split(**bad) == fa.FA_ERR_UNSUPPORTED


def test_splitkv_plan_invalid():
    with pytest.raises(fa.FaError):
        fa.fa_splitkv_plan(1, 3, 2, 16, 16, 64, True)
    with pytest.raises(fa.FaError):
        fa.fa_splitkv_plan(1, 2, 1, 16385, 16, 64, True)


# ------------------------------------------------------------ strided entry points

def _call_strided(qs=None, ks=None, vs=None, os_=None, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["M"], a["N"],
                             a["D"], qs, ks, vs, os_, a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("bad", [dict(qs=(-64, 1024, 64)), dict(ks=(0, -8, 64)), dict(os_=(1024, 64, -64)),
                                 dict(B=0, qs=(1024, 512, 64))])
def test_strided_invalid(bad):
    assert _call_strided(**bad) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(qs=(2048, 1024, 68)), dict(vs=(2048, 1028, 64)), dict(os_=(2052, 1024, 64)),
                                 dict(ks=(1 << 40, 1 << 30, 1 << 25)), dict(D=96, ks=(4096, 2048, 128))])
def test_strided_unsupported(bad):
    assert _call_strided(**bad) == fa.FA_ERR_UNSUPPORTED


def test_strided_split_invalid():
    st = fa.fa_strides(-8, 0, 64)
    rc = fa.fa_fwd_splitkv_strided(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 1, 2, 1, 16, 16, 64, None, st, None, None,
                                   0.125, 1, 0, 1, None, 0, None)
    assert rc == fa.FA_ERR_INVALID_ARG


# ------------------------------------------------------------ Gated DeltaNet entry points

GDN = dict(q=0x1000, k=0x2000, v=0x3000, g=0x4000, beta=0x5000, A=0x6000, s0=None, o=0x7000, sf=0x8000,
           B=1, T=64, Hqk=1, Hv=2, DK=128, DV=128, scale=0.1, dtype=1, ws=None, ws_bytes=0)


def _gdn(**kw):
    a = dict(GDN)
    a.update(kw)
    return fa.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A"], a["s0"], a["o"], a["sf"], a["B"],
                            a["T"], a["Hqk"], a["Hv"], a["DK"], a["DV"], a["scale"], a["dtype"], a["ws"], a["ws_bytes"],
                            None)


@pytest.mark.parametrize("bad", [dict(q=None), dict(A=None), dict(sf=None), dict(T=0), dict(Hqk=2, Hv=3),
                                 dict(scale=0.0), dict(dtype=5)])
def test_gdn_invalid(bad):
    assert _gdn(**bad) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(DK=64), dict(DV=96), dict(v=0x3008), dict(s0=0x9004),
                                 dict(ws=0x10080, ws_bytes=1 << 20)])
def test_gdn_unsupported(bad):
    assert _gdn(**bad) == fa.FA_ERR_UNSUPPORTED


def test_gdn_workspace_size_and_check():
    # chunk states (DV x 128 per chunk, 2-byte elements, end rounded up to 256 bytes), then V_new
    # (DV x 64 per chunk)
    for B, T, Hv, DV in [(1, 64, 2, 128), (2, 200, 4, 64), (1, 32768, 16, 128), (3, 1, 1, 64)]:
        chunks = B * Hv * ((T + 63) // 64)
        st = (chunks * DV * 128 * 2 + 255) // 256 * 256
        assert fa.gdn_chunk_workspace_size(B, T, Hv, DV) == st + chunks * DV * 64 * 2
    assert fa.gdn_chunk_workspace_size(0, 64, 2, 128) == 0
    need = fa.gdn_chunk_workspace_size(1, 64, 2, 128)
    assert _gdn(ws=0x100000, ws_bytes=need - 1) == fa.FA_ERR_INVALID_ARG


def test_gdn_chunk_plan():
    # two-kernel mode while the state walk (B * Hv * DV / 64 workgroups) fills at most 64 CUs
    assert fa.gdn_chunk_plan(1, 32768, 16, 128) == fa.gdn_chunk_workspace_size(1, 32768, 16, 128)  # 32 walkers
    assert fa.gdn_chunk_plan(1, 4096, 32, 128) == fa.gdn_chunk_workspace_size(1, 4096, 32, 128)    # 64
    assert fa.gdn_chunk_plan(2, 4096, 32, 128) == 0                                                # 128
    assert fa.gdn_chunk_plan(8, 4096, 32, 128) == 0                                                # 512
    assert fa.gdn_chunk_plan(1, 100, 65, 64) == 0                                                  # 65
    with pytest.raises(fa.FaError):
        fa.gdn_chunk_plan(1, 64, 2, 96)
    with pytest.raises(fa.FaError):
        fa.gdn_chunk_plan(0, 64, 2, 128)


def _gdn_seg(segments=8, **kw):
    a = dict(GDN, T=1000)
    a.update(kw)
    return fa.gdn_chunk_fwd_segmented(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A"], a["s0"], a["o"], a["sf"],
                                      a["B"], a["T"], a["Hqk"], a["Hv"], a["DK"], a["DV"], a["scale"], a["dtype"],
                                      segments, a["ws"], a["ws_bytes"], None)


def _seg_runs(T, segments):
    chunks = (T + 63) // 64
    length = -(-chunks // min(segments, chunks))
    return -(-chunks // length), length


@pytest.mark.parametrize("bad", [dict(q=None), dict(A=None), dict(sf=None), dict(T=0), dict(Hqk=2, Hv=3),
                                 dict(scale=0.0), dict(dtype=5), dict(segments=0), dict(segments=-2)])
def test_gdn_segmented_invalid(bad):
    assert _gdn_seg(**bad) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(DK=64), dict(DV=96), dict(v=0x3008), dict(s0=0x9004)])
def test_gdn_segmented_unsupported(bad):
    assert _gdn_seg(**bad) == fa.FA_ERR_UNSUPPORTED


def test_gdn_segmented_workspace_size_and_check():
    # runs of ceil(chunks / segments) chunks; per (b, value head) and run but the last: M (128 x 128),
    # Z and a start state (128 x DV), fp32, each of the three parts' ends rounded up to 256 bytes
    for B, T, Hv, DV, seg in [(1, 32768, 16, 128, 8), (2, 700, 3, 64, 5), (1, 200, 4, 128, 9), (1, 64, 2, 128, 4),
                              (1, 1000, 4, 128, 1), (3, 1000, 1, 64, 6)]:
        runs, _ = _seg_runs(T, seg)
        part = lambda cols: -(-(B * Hv * (runs - 1) * 128 * cols * 4) // 256) * 256  # noqa: E731
        want = 0 if runs == 1 else part(128) + 2 * part(DV)
        assert fa.gdn_segmented_workspace_size(B, T, Hv, DV, seg) == want, (B, T, Hv, DV, seg)
    for bad in [(0, 64, 2, 128, 2), (1, 0, 2, 128, 2), (1, 640, 2, 128, 0)]:
        assert fa.gdn_segmented_workspace_size(*bad) == 0
    need = fa.gdn_segmented_workspace_size(1, 1000, 2, 128, 8)
    assert need > 0
    assert _gdn_seg(ws=None, ws_bytes=0) == fa.FA_ERR_INVALID_ARG
    assert _gdn_seg(ws=0x100000, ws_bytes=need - 1) == fa.FA_ERR_INVALID_ARG
    assert _gdn_seg(ws=0x100080, ws_bytes=need) == fa.FA_ERR_UNSUPPORTED


def test_gdn_segment_plan():
    # segmented only for grids of at most 128 state walkers (B * Hv * DV / 64) with two or more
    # chunks, and only when the cost model gives it a clear gain
    assert fa.gdn_segment_plan(1, 32768, 16, 128) > 1      # 32 walkers, 512 chunks
    assert fa.gdn_segment_plan(1, 65536, 4, 64) > 1        # 4 walkers, 1024 chunks
    assert fa.gdn_segment_plan(8, 4096, 32, 128) == 1      # 512 walkers
    assert fa.gdn_segment_plan(1, 100, 129, 64) == 1       # 129 walkers
    assert fa.gdn_segment_plan(1, 64, 2, 128) == 1         # one chunk
    for shape in [(1, 32768, 16, 128), (1, 8192, 4, 128), (2, 8192, 16, 128), (1, 16384, 8, 128),
                  (1, 65536, 4, 64), (4, 4096, 8, 128), (1, 3000, 1, 64)]:
        runs = fa.gdn_segment_plan(*shape)
        assert 1 <= runs <= 64
        if runs > 1:  # a run count the segmented mode really forms, with a workspace
            assert _seg_runs(shape[1], runs)[0] == runs
            assert fa.gdn_segmented_workspace_size(*shape, runs) > 0
    with pytest.raises(fa.FaError):
        fa.gdn_segment_plan(1, 64, 2, 96)
    with pytest.raises(fa.FaError):
        fa.gdn_segment_plan(0, 64, 2, 128)


def test_gdn_kkt_invalid():
    assert fa.gdn_kkt(None, 0x4000, 0x5000, 0x6000, 1, 64, 1, 2, 128, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.gdn_kkt(0x2000, 0x4000, 0x5000, 0x6000, 1, 64, 1, 2, 64, 1, None) == fa.FA_ERR_UNSUPPORTED


def test_headers_are_plain_c(tmp_path):
    # include/*.h must compile as strict C99 and as C++ (no C++ or HIP types in the ABI)
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "use.c"
    src.write_text("".join(f'#include "{h}"\n' for h in sorted(os.listdir(inc)) if h.endswith(".h")) +
                   "int main(void) { return 0; }\n")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-I", inc, str(src)],
                   check=True)
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", "c++", "-I", inc,
                    str(src)], check=True)


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(INCLUDE, "fa.h")).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_plans_beyond_its_scratch_before_touching_the_gpu():
    """A plan whose partial results exceed the scratch is refused on the host (no GPU here: the
    call must return before any HIP call)."""
    args = (1, 64, 64, 4096, 8192, 128, 1)  # 64 heads x 32 query tiles, shares of 8 key tiles
    _, _, ws = fa.fa_splitkv_plan(*args, 8)
    assert ws > fa.FA_NOALLOC_SCRATCH_BYTES
    B, Hq, Hkv, M, N, D, causal = args
    rc = fa.fa_fwd_splitkv_noalloc(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, B, Hq, Hkv, M, N, D, 0.088, causal,
                                   fa.FA_BF16, 8, None)
    assert rc == fa.FA_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in fa.fa_strerror(rc)
    # and the ordinary argument checks come first
    assert fa.fa_fwd_splitkv_noalloc(None, 0x2000, 0x3000, 0x4000, 0x5000, B, Hq, Hkv, M, N, D, 0.088, causal,
                                     fa.FA_BF16, 8, None) == fa.FA_ERR_INVALID_ARG
