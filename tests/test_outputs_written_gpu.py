"""Every output element is written by every launch shape: O and lse are pre-filled with NaN (and,
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
