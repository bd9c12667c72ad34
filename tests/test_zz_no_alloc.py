"""fa_fwd_splitkv_noalloc (the key-split forward that allocates nothing) against fa_fwd_splitkv
with a caller workspace: the same kernels on the same plan, so every output bit must agree.  Two
calls in a row on the shared scratch, the second with a smaller input, then back to a larger one;
one case is also checked against the fp64 oracle.  Called through the C ABI (ctypes binding)."""
import math

import numpy as np
import pytest
import torch

import gqa_attention_forward_amd as fa
import oracle
from gqa_attention_forward_amd.inputs import make_custom

pytestmark = pytest.mark.gpu


def _dt(t):
    return fa.FA_F16 if t.dtype == torch.float16 else fa.FA_BF16


def _run(q, k, v, causal, tiles, noalloc):
    B, Hq, M, D = q.shape
    _, Hkv, N, _ = k.shape
    scale = 1.0 / math.sqrt(D)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, M), float("nan"), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        rc = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                                       Hkv, M, N, D, scale, causal, _dt(q), tiles, stream)
    else:
        _, _, ws_bytes = fa.fa_splitkv_plan(B, Hq, Hkv, M, N, D, causal, tiles)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        rc = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, M,
                               N, D, scale, causal, _dt(q), tiles, ws.data_ptr(), ws_bytes, stream)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    return o, lse


# B, Hq, Hkv, M, N, D, causal, dtype, tiles_per_split (0: automatic)
SEQUENCES = [
    [(8, 32, 8, 1, 8192, 128, True, torch.bfloat16, 0),      # decode: stacked heads, 1 MB of partials
     (2, 8, 2, 1, 3000, 64, True, torch.float16, 0)],        # smaller, ragged keys
    [(4, 32, 8, 64, 8192, 128, True, torch.float16, 0),      # 64-row chunk: 17 MB of partials
     (1, 4, 1, 100, 2500, 128, False, torch.bfloat16, 4)],   # smaller, forced shares, non-causal
    [(1, 8, 8, 512, 8192, 128, True, torch.float16, 0),
     (1, 2, 1, 130, 700, 64, True, torch.bfloat16, 2),
     (2, 16, 8, 1024, 1024, 128, True, torch.float16, 0)],   # a plan with no split: no scratch used
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join("x".join(str(x) for x in c[:6]) for c in s))
def test_noalloc_matches_workspace_entry_point(seq):
    for i, (B, Hq, Hkv, M, N, D, causal, dtype, tiles) in enumerate(seq):
        q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=1000 + 7 * i + M, device="cuda")
        o_ref, l_ref = _run(q, k, v, causal, tiles, noalloc=False)
        o, lse = _run(q, k, v, causal, tiles, noalloc=True)
        _, _, ws = fa.fa_splitkv_plan(B, Hq, Hkv, M, N, D, causal, tiles)
        same = torch.equal(o, o_ref) and torch.equal(lse.nan_to_num(), l_ref.nan_to_num())
        print(f"call {i}: {B}x{Hq}/{Hkv} M={M} N={N} D={D} causal={causal} {dtype}: scratch {ws} B, "
              f"bitwise equal to the workspace entry point: {same}", flush=True)
        assert same


def test_noalloc_matches_oracle():
    B, Hq, Hkv, M, N, D = 2, 8, 2, 3, 2000, 128
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=77)
    o, lse = _run(q.cuda(), k.cuda(), v.cuda(), True, 0, noalloc=True)
    ro, rlse = oracle.attn_fwd(q, k, v, 1.0 / math.sqrt(D), True)
    err = float(np.abs(o.cpu().double().numpy() - ro).max())
    lerr = float(np.abs(lse.cpu().double().numpy() - rlse).max())
    print(f"noalloc vs oracle: max|dO| {err:.3e} (tol 4e-3), max|dlse| {lerr:.3e} (tol 1e-3)", flush=True)
    assert err <= 4e-3 and lerr <= 1e-3


def test_noalloc_rejects_oversized_plan_on_gpu():
    q, k, v = (torch.zeros(1, 64, 4096, 128, dtype=torch.bfloat16, device="cuda"),
               torch.zeros(1, 64, 8192, 128, dtype=torch.bfloat16, device="cuda"),
               torch.zeros(1, 64, 8192, 128, dtype=torch.bfloat16, device="cuda"))
    o = torch.empty_like(q)
    lse = torch.empty(1, 64, 4096, dtype=torch.float32, device="cuda")
    rc = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 64, 64,
                                   4096, 8192, 128, 0.088, 1, fa.FA_BF16, 8, torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_ERR_SCRATCH_TOO_SMALL
