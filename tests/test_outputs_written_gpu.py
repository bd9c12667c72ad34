"""Every output element is written by every launch shape of the forward (O, lse), the backward (dq,
dk, dv) and the Gated DeltaNet prefill (O, final state; all three modes): the outputs are pre-filled with NaN (and,
in a second call, with zeros), and the two results must be identical bit for bit and free of
NaN.  The parity tests compare against the oracle, but a buffer that happens to hold an earlier
call's correct values would hide an element a kernel never stores (one key group's half of the
columns, a merged row, a ragged row)."""
import math

import pytest
import torch

import gqa_attention_forward_amd as fa
from gqa_attention_forward_amd.inputs import make_custom

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, M, N, D, causal, dtype, split_kv; the comment names the launch shape it reaches
CASES = [
    (8, 32, 8, 300, 333, 128, True, torch.bfloat16, False),     # 8-wave 256-row workgroups
    (1, 4, 2, 300, 700, 128, True, torch.float16, False),       # 4-wave 128-row workgroups
    (2, 4, 2, 200, 1030, 64, False, torch.float16, False),      # two key groups, D = 64, odd tile count
    (1, 4, 2, 300, 1500, 128, True, torch.bfloat16, False),     # two key groups, D = 128, ragged rows
    (1, 2, 1, 1200, 1000, 128, True, torch.float16, False),     # two key groups, rows with no key
    (1, 8, 2, 77, 3000, 128, True, torch.float16, "auto"),      # key split, stacked heads, merge
    (2, 4, 2, 300, 1200, 64, True, torch.bfloat16, 3),          # key split, shares of 3 tiles
    (1, 4, 1, 300, 77, 128, True, torch.bfloat16, 1),           # key split, rows with no key
]


def _call(q, k, v, causal, split_kv, fill):
    o = torch.full_like(q, fill)
    lse = torch.full(q.shape[:3], fill, dtype=torch.float32, device=q.device)
    fa.attention_forward(q, k, v, causal=causal, scale=1.0 / math.sqrt(q.shape[-1]), out=o, lse=lse,
                         split_kv=split_kv)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(x) for x in c[:7]) + f"-{c[8]}")
def test_every_output_element_written(case):
    B, Hq, Hkv, M, N, D, causal, dtype, split_kv = case
    q, k, v = (t.cuda() for t in make_custom(B, Hq, Hkv, M, N, D, dtype, seed=M + 3 * N))
    o_nan, lse_nan = _call(q, k, v, causal, split_kv, float("nan"))
    o_zero, lse_zero = _call(q, k, v, causal, split_kv, 0.0)
    print(f"{case}: NaN in O {int(torch.isnan(o_nan).sum())}, in lse {int(torch.isnan(lse_nan).sum())}", flush=True)
    assert not torch.isnan(o_nan).any()
    assert not torch.isnan(lse_nan).any()
    assert torch.equal(o_nan, o_zero)
    assert torch.equal(lse_nan, lse_zero)
    # rows that see no key: O = 0 and lse = -inf; every other lse is finite
    empty = torch.isneginf(lse_nan)
    assert torch.all(o_nan[empty] == 0)
    assert torch.isfinite(lse_nan[~empty]).all()
    if causal:
        rows = torch.arange(M, device=q.device)
        assert torch.equal(empty[0, 0], rows + (N - M) < 0)


def _bwd(q, k, v, o, lse, do, causal, fill):
    B, Hq, M, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    dq, dk, dv = (torch.full_like(t, fill) for t in (q, k, v))
    ws_bytes = fa.fa_bwd_workspace_size(B, Hq, M)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, M, N, D, 1.0 / math.sqrt(D), causal,
                   fa.FA_F16 if q.dtype == torch.float16 else fa.FA_BF16, ws.data_ptr(), ws_bytes,
                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return dq, dk, dv


# B, Hq, Hkv, M, N, D, causal, dtype: ragged query and key blocks, grouped heads, rows with no key
BWD_CASES = [
    (1, 4, 2, 300, 333, 128, True, torch.bfloat16),
    (2, 2, 2, 200, 130, 64, False, torch.float16),
    (1, 2, 1, 300, 100, 128, True, torch.float16),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(str(x) for x in c[:7]))
def test_backward_writes_every_gradient(case):
    B, Hq, Hkv, M, N, D, causal, dtype = case
    q, k, v = (t.cuda() for t in make_custom(B, Hq, Hkv, M, N, D, dtype, seed=M + N))
    o, lse = fa.attention_forward(q, k, v, causal=causal, split_kv=False)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(M), dtype=torch.float32).to(dtype).cuda()
    g_nan = _bwd(q, k, v, o, lse, do, causal, float("nan"))
    g_zero = _bwd(q, k, v, o, lse, do, causal, 0.0)
    for name, a, b in zip(("dq", "dk", "dv"), g_nan, g_zero):
        print(f"{case} {name}: NaN {int(torch.isnan(a).sum())}", flush=True)
        assert not torch.isnan(a).any(), name
        assert torch.equal(a, b), name


@pytest.mark.parametrize("two_kernel", [False, True])
def test_gdn_writes_every_output(two_kernel):
    from gqa_attention_forward_amd.inputs import GdnWorkload, make_gdn_inputs

    w = GdnWorkload("t", 2, 200, 2, 4, 128, 128, torch.bfloat16, 11, init_state=True)  # ragged last chunk
    q, k, v, g, beta, s0 = (t.cuda() if t is not None else None for t in make_gdn_inputs(w))
    _, _, A = fa.gdn_prefill(q, k, v, g, beta, s0=s0)
    B, T, Hqk, DK = q.shape
    Hv, DV = v.shape[2], v.shape[3]
    ws_bytes = fa.gdn_chunk_workspace_size(B, T, Hv, DV) if two_kernel else 0
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    outs = []
    for fill in (float("nan"), 0.0):
        o = torch.full((B, T, Hv, DV), fill, dtype=q.dtype, device=q.device)
        sf = torch.full((B, Hv, DK, DV), fill, dtype=torch.float32, device=q.device)
        rc = fa.gdn_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), A.data_ptr(),
                              s0.data_ptr(), o.data_ptr(), sf.data_ptr(), B, T, Hqk, Hv, DK, DV,
                              1.0 / math.sqrt(DK), fa.FA_BF16, ws.data_ptr() if ws_bytes else None, ws_bytes,
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        outs.append((o, sf))
    (o_nan, sf_nan), (o_zero, sf_zero) = outs
    print(f"gdn two_kernel={two_kernel}: NaN in O {int(torch.isnan(o_nan).sum())}, in state "
          f"{int(torch.isnan(sf_nan).sum())}", flush=True)
    assert not torch.isnan(o_nan).any() and not torch.isnan(sf_nan).any()
    assert torch.equal(o_nan, o_zero) and torch.equal(sf_nan, sf_zero)


def test_gdn_segmented_writes_every_output():
    from gqa_attention_forward_amd.inputs import GdnWorkload, make_gdn_inputs

    # 5 chunks (the last ragged) in runs of 2, 2 and 1: only the last run writes the final state
    w = GdnWorkload("t", 2, 300, 2, 4, 128, 128, torch.bfloat16, 12, init_state=True)
    q, k, v, g, beta, s0 = (t.cuda() for t in make_gdn_inputs(w))
    _, _, A = fa.gdn_prefill(q, k, v, g, beta, s0=s0)
    B, T, Hqk, DK = q.shape
    Hv, DV = v.shape[2], v.shape[3]
    ws_bytes = fa.gdn_segmented_workspace_size(B, T, Hv, DV, 3)
    assert ws_bytes > 0
    outs = []
    for fill in (float("nan"), 0.0):
        ws = torch.full((ws_bytes // 4,), fill, dtype=torch.float32, device=q.device)  # stale workspace too
        o = torch.full((B, T, Hv, DV), fill, dtype=q.dtype, device=q.device)
        sf = torch.full((B, Hv, DK, DV), fill, dtype=torch.float32, device=q.device)
        rc = fa.gdn_chunk_fwd_segmented(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                        A.data_ptr(), s0.data_ptr(), o.data_ptr(), sf.data_ptr(), B, T, Hqk, Hv, DK,
                                        DV, 1.0 / math.sqrt(DK), fa.FA_BF16, 3, ws.data_ptr(), ws_bytes,
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        outs.append((o, sf))
    (o_nan, sf_nan), (o_zero, sf_zero) = outs
    print(f"gdn segmented: NaN in O {int(torch.isnan(o_nan).sum())}, in state {int(torch.isnan(sf_nan).sum())}",
          flush=True)
    assert not torch.isnan(o_nan).any() and not torch.isnan(sf_nan).any()
    assert torch.equal(o_nan, o_zero) and torch.equal(sf_nan, sf_zero)
