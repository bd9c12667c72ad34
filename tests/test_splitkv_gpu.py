"""Parity of the key-split forward (split kernel + lse merge, through the C ABI) against the
fp64 CPU oracle, with the same tolerances as fa_fwd: max-abs error of O <= 4e-3 (fp16) /
1.6e-2 (bf16), logsumexp within 1e-3; rows that see no key give O = 0 and lse = -inf."""
import math

import numpy as np
import pytest
import torch

import gqa_attention_forward_amd as fa
import oracle
from gqa_attention_forward_amd.inputs import SMALL_GRID_WORKLOADS, WORKLOADS, make_custom, make_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
LSE_TOL = 1e-3


def _run(q, k, v, causal, scale, split_kv):
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.attention_forward(dq, dk, dv, causal=causal, scale=scale, split_kv=split_kv)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what):
    o_gpu = o_gpu.double().numpy()
    lse_gpu = lse_gpu.double().numpy()
    fin = np.isfinite(lse_ref)
    err = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    lerr = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    print(f"{what}: max|dO| = {err:.3e} (tol {TOL[dtype]:.1e}), max|dlse| = {lerr:.3e}", flush=True)
    assert np.all(np.isfinite(o_gpu)), what
    assert err <= TOL[dtype], what
    assert lerr <= LSE_TOL, what
    assert np.all(np.isneginf(lse_gpu[~fin])), what
    assert np.all(o_gpu[~fin] == 0.0), what


SHAPES = [
    # B, Hq, Hkv, M, N, D, causal, dtype, key tiles per share
    (1, 2, 1, 128, 128, 64, True, torch.float16, 1),
    (2, 4, 2, 300, 300, 128, True, torch.bfloat16, 1),     # ragged, shares of one tile
    (2, 4, 2, 300, 300, 128, True, torch.float16, 3),      # shares of uneven length
    (1, 8, 2, 77, 300, 128, True, torch.float16, 2),
    (1, 4, 1, 300, 77, 128, True, torch.bfloat16, 1),      # first 223 rows see no key
    (2, 2, 2, 200, 333, 128, False, torch.float16, 2),
    (1, 4, 4, 129, 65, 64, False, torch.bfloat16, 1),
    (1, 6, 3, 256, 1000, 64, True, torch.bfloat16, 4),
    (3, 2, 1, 1, 1, 128, True, torch.float16, 1),           # one query, one key
    (1, 2, 1, 1, 500, 128, True, torch.float16, 1),         # decode-like, 8 shares
    (1, 32, 8, 1, 4096, 128, True, torch.bfloat16, 0),      # decode-like, automatic plan
    (2, 8, 2, 16, 3000, 64, True, torch.float16, 0),        # short M, automatic plan
    (1, 8, 8, 64, 2048, 128, False, torch.float16, 0),
    (1, 2, 1, 1000, 600, 128, True, torch.bfloat16, 2),     # M > N: early rows empty, later rows split
    # M < 128 with grouped KV heads: the group's query heads are stacked in one tile's rows
    (1, 12, 1, 100, 700, 64, True, torch.bfloat16, 2),      # tiles straddle head boundaries, causal
    (2, 8, 1, 33, 64, 128, True, torch.float16, 1),
    (1, 6, 2, 50, 40, 128, True, torch.bfloat16, 1),        # M > N: the first 10 rows of every head empty
    # the merge holds up to 16 shares of a row in registers and loops over more
    (1, 2, 1, 64, 1024, 64, False, torch.bfloat16, 1),      # 16 shares
    (1, 2, 1, 64, 1088, 64, False, torch.float16, 1),       # 17 shares
    (1, 4, 2, 200, 1500, 128, True, torch.float16, 1),      # up to 24 shares, two split query-tile ranks
    (1, 16, 2, 127, 3000, 128, False, torch.float16, 5),
    (16, 32, 8, 64, 512, 128, True, torch.float16, 0),      # automatic: stacked heads, no split
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(str(x) for x in s[:7]) + str(s[7]).split(".")[-1] + f"t{s[8]}")
def test_splitkv_small_shapes(shape):
    B, Hq, Hkv, M, N, D, causal, dtype, tiles = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=M * 13 + N)
    scale = 1.0 / math.sqrt(D)
    used, wgs, ws = fa.fa_splitkv_plan(B, Hq, Hkv, M, N, D, causal, tiles)
    print(f"plan: {used} tiles a share, {wgs} workgroups, workspace {ws} B", flush=True)
    o, lse = _run(q, k, v, causal, scale, tiles if tiles > 0 else "auto")
    ro, rlse = oracle.attn_fwd(q, k, v, scale, causal)
    _check(o, lse, ro, rlse, dtype, f"split {shape}")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_splitkv_peaky(dtype):
    """Peaky logits: the shares' maxima differ widely, so the merge weights span many decades."""
    q, k, v = make_custom(1, 4, 1, 256, 2048, 128, dtype, seed=7, peak_rate=0.02)
    scale = 1.0 / math.sqrt(128)
    o, lse = _run(q, k, v, True, scale, 2)
    ro, rlse = oracle.attn_fwd(q, k, v, scale, True)
    _check(o, lse, ro, rlse, dtype, "split peaky")


def test_splitkv_pages_workload():
    """The pages' 1k causal GQA workload with shares of 5 key tiles (the longer query tiles split)."""
    w = WORKLOADS["pages_causal_gqa_1k"]
    used, wgs, ws = fa.fa_splitkv_plan(w.B, w.Hq, w.Hkv, w.M, w.N, w.D, w.causal, 5)
    assert ws > 0
    q, k, v, _ = make_inputs(w)
    o, lse = _run(q, k, v, w.causal, w.scale, 5)
    ro, rlse = oracle.attn_fwd(q, k, v, w.scale, w.causal)
    _check(o, lse, ro, rlse, w.dtype, f"{w.name} split ({used} tiles a share, {wgs} workgroups)")


def test_splitkv_deterministic_and_close_to_plain():
    q, k, v = make_custom(2, 8, 2, 300, 2000, 128, torch.bfloat16, seed=5)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = fa.attention_forward(dq, dk, dv, causal=True, split_kv=3)
    o2, l2 = fa.attention_forward(dq, dk, dv, causal=True, split_kv=3)
    op, lp = fa.attention_forward(dq, dk, dv, causal=True, split_kv=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # two roundings of the same fp32 result to bf16 differ by at most one unit in the last place
    assert (o1.float() - op.float()).abs().max().item() <= 2 * TOL[torch.bfloat16]
    assert (l1 - lp).abs().max().item() <= 1e-4


def test_splitkv_workspace_reuse_across_shapes():
    """One workspace serves successive calls of different plans (every slot a merge reads is rewritten)."""
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for (M, N, tiles) in [(600, 1200, 2), (100, 900, 1), (600, 1200, 3)]:
        q, k, v = make_custom(1, 4, 2, M, N, 64, torch.float16, seed=M + N + tiles)
        dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
        o = torch.empty_like(dq)
        lse = torch.empty((1, 4, M), dtype=torch.float32, device="cuda")
        used, wgs, need = fa.fa_splitkv_plan(1, 4, 2, M, N, 64, True, tiles)
        assert 0 < need <= ws.numel()
        rc = fa.fa_fwd_splitkv(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 4, 2, M,
                               N, 64, 0.125, 1, fa.FA_F16, tiles, ws.data_ptr(), ws.numel(),
                               torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        ro, rlse = oracle.attn_fwd(q, k, v, 0.125, True)
        _check(o.cpu(), lse.cpu(), ro, rlse, torch.float16, f"reuse M={M} N={N} tiles={tiles}")


@pytest.mark.parametrize("name", list(SMALL_GRID_WORKLOADS))
def test_small_grid_workloads_auto(name):
    """The decode and short-query workloads at full size through the automatic plan (which splits
    them), in the launch configuration the benchmark times: in full when the oracle finishes in
    seconds, else the first and last 64 rows of every head plus random rows."""
    w = SMALL_GRID_WORKLOADS[name]
    used, wgs, ws = fa.fa_splitkv_plan(w.B, w.Hq, w.Hkv, w.M, w.N, w.D, w.causal, 0)
    assert ws > 0, "the automatic plan is expected to split this workload"
    q, k, v, _ = make_inputs(w)
    o, lse = _run(q, k, v, w.causal, w.scale, "auto")
    what = f"{name} ({used} tiles a share, {wgs} workgroups)"
    if w.B * w.Hq * w.M * w.N <= 16 * 1024 * 1024:
        ro, rlse = oracle.attn_fwd(q, k, v, w.scale, w.causal)
        _check(o, lse, ro, rlse, w.dtype, what)
        return
    rows = []
    for bh in range(w.B * w.Hq):
        rows.extend(range(bh * w.M, bh * w.M + min(16, w.M)))
        rows.extend(range(bh * w.M + max(0, w.M - 16), (bh + 1) * w.M))
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([np.array(rows), rng.integers(0, w.B * w.Hq * w.M, size=256)])).astype(np.int64)
    ro, rlse = oracle.attn_fwd_rows(q, k, v, w.scale, w.causal, rows)
    og = o.reshape(-1, w.D)[torch.from_numpy(rows)]
    lg = lse.reshape(-1)[torch.from_numpy(rows)]
    _check(og, lg, ro, rlse, w.dtype, what + f", {rows.size} sampled rows")


def test_splitkv_many_split_tiles_merge_kernel():
    """A plan with 18432 single-row query tiles, each split in two (36864 split work-groups and as
    many merge rows): checked on sampled rows against the oracle, and every row against the
    unsplit forward."""
    B, Hq, Hkv, M, N, D = 64, 288, 288, 1, 128, 64
    _, wgs, need = fa.fa_splitkv_plan(B, Hq, Hkv, M, N, D, True, 1)
    assert wgs == 2 * B * Hq and need > 0
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=808)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.attention_forward(dq, dk, dv, causal=True, split_kv=1)
    op, lp = fa.attention_forward(dq, dk, dv, causal=True, split_kv=False)
    torch.cuda.synchronize()
    assert (o.float() - op.float()).abs().max().item() <= 2 * TOL[torch.bfloat16]
    assert (lse - lp).abs().max().item() <= 1e-4
    rows = np.random.default_rng(3).choice(B * Hq * M, 400, replace=False)
    ro, rlse = oracle.attn_fwd_rows(q, k, v, 1.0 / math.sqrt(D), True, rows)
    og = o.reshape(-1, D)[torch.from_numpy(rows).cuda()].cpu()
    lg = lse.reshape(-1)[torch.from_numpy(rows).cuda()].cpu()
    _check(og, lg, ro, rlse, torch.bfloat16, "merge-kernel plan, 400 sampled rows")
