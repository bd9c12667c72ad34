"""Host-side tile math and scheduling of the HIP path (no GPU needed): the library's own
classification functions, checked against the pages' worked numbers and brute force."""
import itertools
import json
import os

import pytest

import gqa_attention_forward_amd as fa
from gqa_attention_forward_amd import accounting

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_worked_numbers.json")))


def test_pages_visited_tile_count_bm32():
    full, masked, skipped = fa.fa_tile_counts(1024, 1024, 32, 32, True)
    assert full + masked == GOLDEN["visited_tiles_bm32"]["value"] == 528
    assert masked == GOLDEN["masked_tiles_bm32"]["value"]
    assert skipped / (32 * 32) == GOLDEN["saved_fraction_bm32"]["value"]


def test_pages_stage_counts_bm64():
    full, masked, skipped = fa.fa_tile_counts(1024, 1024, 64, 64, True)
    g = GOLDEN["stage_counts_bm64"]
    assert (full, masked) == (g["full"], g["masked"])
    e = GOLDEN["executions_bm64"]
    outside = e["B"] * e["H"] * (1024 // 64) * e["warps"]
    assert outside == e["outside_loop"]
    # every (b, h) runs `full` unmasked tiles, each executed by all warps
    assert e["B"] * e["H"] * full * e["warps"] == e["unmasked_loop"]


def test_pages_bytes_model():
    g = GOLDEN["bytes_model_bm32"]
    BM, M, N, D = 32, 1024, 1024, 128
    blocks = 32 * (M // BM)  # B*H = 32 blocks per query-tile position
    assert blocks * (BM * D + 2 * N * D) * 2 == g["read_bytes"]
    assert blocks * BM * D * 2 == g["write_bytes"]
    # compulsory Q+K+V bytes of the shape, which the measured 17.1 MB approaches
    qkv = 2 * 16 * 1024 * 128 * 2 + 2 * 2 * 8 * 1024 * 128 * 2
    assert abs(qkv / 1e6 - GOLDEN["compulsory_read_bytes"]["value_mb_measured"]) < 0.5


def _brute(M, N, BM, BN, causal):
    """Classify every (query tile, key tile) by enumerating its (i, j) pairs."""
    full = masked = skipped = 0
    for q0 in range(0, M, BM):
        rows = range(q0, min(q0 + BM, M))
        for k0 in range(0, N, BN):
            keys = range(k0, k0 + BN)  # a ragged last tile still spans BN key slots
            vis = [[j < N and (not causal or j <= i + N - M) for j in keys] for i in rows]
            if not any(any(r) for r in vis):
                skipped += 1
            elif all(all(r) for r in vis):
                full += 1
            else:
                masked += 1
    return full, masked, skipped


@pytest.mark.parametrize("M,N,BM,BN,causal", [
    (128, 128, 128, 64, True), (1000, 1000, 128, 64, True), (77, 300, 128, 64, True),
    (300, 77, 128, 64, True), (5, 3, 128, 64, True), (130, 250, 32, 48, True),
    (512, 8192, 128, 64, True), (256, 200, 64, 64, False), (9, 1, 128, 64, False),
])
def test_classification_matches_brute_force(M, N, BM, BN, causal):
    assert fa.fa_tile_counts(M, N, BM, BN, causal) == _brute(M, N, BM, BN, causal)


def test_tile_shape():
    # 8-wave workgroups (256 rows) at D = 128 once they alone fill the 256 CUs, 4-wave ones
    # (128 rows) below that and at D = 64
    assert fa.fa_tile_shape(1, 32, 16384, 128) == (256, 64)
    assert fa.fa_tile_shape(8, 32, 4096, 128) == (256, 64)
    assert fa.fa_tile_shape(4, 32, 512, 128) == (256, 64)
    assert fa.fa_tile_shape(2, 16, 1024, 128) == (128, 64)
    assert fa.fa_tile_shape(1, 2, 128, 64) == (128, 64)
    assert fa.fa_tile_shape(1, 32, 16384, 64) == (128, 64)  # D = 64: 4-wave workgroups on any grid
    with pytest.raises(fa.FaError):
        fa.fa_tile_shape(1, 2, 128, 96)
    with pytest.raises(fa.FaError):
        fa.fa_tile_shape(0, 2, 128, 64)


@pytest.mark.parametrize("B,Hq,Hkv,M,causal", [
    (1, 2, 1, 128, True), (2, 16, 8, 1024, True), (3, 6, 2, 300, False), (1, 32, 8, 2048, True),
    (2, 5, 5, 129, False), (1, 3, 1, 1, True),
])
def test_schedule_is_a_bijection(B, Hq, Hkv, M, causal):
    BM, _ = fa.fa_tile_shape(B, Hq, M, 128)
    n_qt = (M + BM - 1) // BM
    total = B * Hq * n_qt
    seen = set(fa.fa_schedule(B, Hq, Hkv, M, 128, causal, w) for w in range(total))
    assert seen == set(itertools.product(range(B), range(Hq), range(n_qt)))
    with pytest.raises(fa.FaError):
        fa.fa_schedule(B, Hq, Hkv, M, 128, causal, total)


def test_schedule_keeps_kv_groups_on_one_xcd():
    """For the long causal GQA prefill shape, each of the 8 XCDs (wg % 8) serves exactly one
    KV head, and issues its query tiles longest-first."""
    B, Hq, Hkv, M = 1, 32, 8, 16384
    BM, _ = fa.fa_tile_shape(B, Hq, M, 128)
    total = B * Hq * (M // BM)
    per_xcd = {x: [] for x in range(8)}
    for w in range(total):
        b, h, qt = fa.fa_schedule(B, Hq, Hkv, M, 128, True, w)
        per_xcd[w % 8].append((h // (Hq // Hkv), qt))
    for x, items in per_xcd.items():
        assert {hk for hk, _ in items} == {x}
        qts = [qt for _, qt in items]
        assert qts == sorted(qts, reverse=True)


def test_accounting_visible_pairs_closed_forms():
    assert accounting.visible_pairs_per_head(1024, 1024, True) == 1024 * 1025 // 2
    assert accounting.visible_pairs_per_head(512, 8192, True) == sum(min(8192, i + 1 + 7680) for i in range(512))
    assert accounting.visible_pairs_per_head(3, 1, True) == 1
    assert accounting.visible_pairs_per_head(7, 9, False) == 63


def _exact_schedule(B, Hq, Hkv, n_qt, causal, wg):
    """The schedule written with exact integer division: XCD x = wg % 8 owns the x-th block of
    consecutive logical indices; logical order (b, kv head), query-tile rank, query head."""
    total = B * Hq * n_qt
    q, rem = divmod(total, 8)
    xcd, slot = wg % 8, wg // 8
    L = (xcd * (q + 1) if xcd < rem else rem * (q + 1) + (xcd - rem) * q) + slot
    g = Hq // Hkv
    rest, hg = divmod(L, g)
    bhk, rank = divmod(rest, n_qt)
    b, hk = divmod(bhk, Hkv)
    return b, hk * g + hg, (n_qt - 1 - rank) if causal else rank


@pytest.mark.parametrize("B,Hq,Hkv,M,causal", [
    (3, 21, 7, 1000, False),          # g = 3, 8 query tiles
    (5, 15, 3, 777, True),            # g = 5
    (7, 56, 8, 70000, True),          # g = 7, 274 query tiles
    (64, 96, 32, 65536, False),       # 1.5 M workgroups
    (8191, 32, 4, 8191 * 256, True),  # 2.147e9 workgroups, just under the 2^31 grid limit
])
def test_schedule_matches_exact_division(B, Hq, Hkv, M, causal):
    """The kernels find their tile with multiply-high division by divisors fixed at launch; the
    library's schedule (the same code) equals exact division on sampled and boundary workgroups."""
    import numpy as np

    BM, _ = fa.fa_tile_shape(B, Hq, M, 128)
    n_qt = (M + BM - 1) // BM
    total = B * Hq * n_qt
    assert total < 2 ** 31
    rng = np.random.default_rng(total % 1000)
    wgs = set(range(min(total, 64))) | set(range(max(0, total - 64), total))
    wgs |= set(int(x) for x in rng.integers(0, total, 3000))
    for wg in sorted(wgs):
        assert fa.fa_schedule(B, Hq, Hkv, M, 128, causal, wg) == _exact_schedule(B, Hq, Hkv, n_qt, causal, wg), wg
