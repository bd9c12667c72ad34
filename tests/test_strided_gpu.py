"""Strided layouts through the C ABI: [B, S, H, D] buffers, K and V interleaved in one buffer,
padded rows and a batch-broadcast K/V, on both the plain and the key-split kernels.  Each case
is checked against the fp64 oracle (on contiguous copies) with fa_fwd's tolerances, and
against the contiguous launch of the same kernel, which must give the same bits."""
import math

import numpy as np
import pytest
import torch

import gqa_attention_forward_amd as fa
import oracle
from gqa_attention_forward_amd.inputs import make_custom

pytestmark = pytest.mark.gpu

TOL = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}


def _check_oracle(o, lse, q, k, v, causal, scale, dtype, what):
    ro, rlse = oracle.attn_fwd(q.cpu().contiguous(), k.cpu().contiguous(), v.cpu().contiguous(), scale, causal)
    og = o.cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    fin = np.isfinite(rlse)
    err = np.abs(og - ro).max()
    lerr = np.abs(lg[fin] - rlse[fin]).max() if fin.any() else 0.0
    print(f"{what}: max|dO| = {err:.3e}, max|dlse| = {lerr:.3e}", flush=True)
    assert err <= TOL[dtype] and lerr <= 1e-3, what
    assert np.all(np.isneginf(lg[~fin])) and np.all(og[~fin] == 0.0), what


def _bshd(t):
    """The same values stored as a [B, S, H, D] buffer, returned as a [B, H, S, D] view."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


CASES = [
    # B, Hq, Hkv, M, N, D, causal, dtype, split_kv
    (2, 8, 2, 300, 300, 128, True, torch.bfloat16, False),
    (1, 32, 8, 1024, 1024, 128, True, torch.float16, False),      # 8-wave tiles
    (2, 4, 4, 200, 333, 64, False, torch.float16, False),
    (2, 8, 2, 77, 900, 128, True, torch.bfloat16, 2),             # key-split, stacked heads
    (4, 32, 8, 1, 4096, 128, True, torch.bfloat16, "auto"),       # decode
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(x) for x in c[:7]) + f"-{c[8]}")
def test_bshd_layout(case):
    B, Hq, Hkv, M, N, D, causal, dtype, split = case
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=M + 3 * N)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o_ref, l_ref = fa.attention_forward(dq, dk, dv, causal=causal, scale=scale, split_kv=split)
    sq, sk, sv = _bshd(dq), _bshd(dk), _bshd(dv)
    assert not sk.is_contiguous() and sk.stride(3) == 1 and (M == 1 or not sq.is_contiguous())
    o, lse = fa.attention_forward(sq, sk, sv, causal=causal, scale=scale, split_kv=split)
    torch.cuda.synchronize()
    assert o.stride() == sq.stride(), "a new output takes q's layout"
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "strided and contiguous launches differ"
    _check_oracle(o, lse, q, k, v, causal, scale, dtype, f"bshd {case}")


@pytest.mark.parametrize("split", [False, 3])
def test_interleaved_kv_padded_rows_and_output_view(split):
    """K and V interleaved in one [B, N, 2, Hkv, D] buffer; Q in rows padded to D + 64 elements;
    O written into a [B, M, Hq, D] view of a larger buffer."""
    B, Hq, Hkv, M, N, D, dtype = 2, 8, 2, 150, 700, 64, torch.float16
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=11)
    scale = 0.125
    kv = torch.stack([k.transpose(1, 2), v.transpose(1, 2)], dim=2).cuda()  # [B, N, 2, Hkv, D]
    sk, sv = kv[:, :, 0].transpose(1, 2), kv[:, :, 1].transpose(1, 2)
    qpad = torch.zeros((B, Hq, M, D + 64), dtype=dtype, device="cuda")
    qpad[..., :D] = q.cuda()
    sq = qpad[..., :D]
    obuf = torch.full((B, M, Hq + 2, D), 7.0, dtype=dtype, device="cuda")
    o = obuf[:, :, 1:Hq + 1].transpose(1, 2)
    _, lse = fa.attention_forward(sq, sk, sv, causal=True, scale=scale, out=o, split_kv=split)
    o_ref, l_ref = fa.attention_forward(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale, split_kv=split)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert torch.all(obuf[:, :, 0] == 7.0) and torch.all(obuf[:, :, Hq + 1] == 7.0), "wrote outside the view"
    _check_oracle(o, lse, q, k, v, True, scale, dtype, f"interleaved kv, split {split}")


def test_batch_broadcast_kv():
    """One K/V shared by every batch entry through a zero batch stride."""
    B, Hq, Hkv, M, N, D, dtype = 3, 4, 2, 128, 256, 128, torch.bfloat16
    q, k1, v1 = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=21)
    k1, v1 = k1[:1], v1[:1]
    dk, dv = k1.cuda().expand(B, -1, -1, -1), v1.cuda().expand(B, -1, -1, -1)
    assert dk.stride(0) == 0
    o, lse = fa.attention_forward(q.cuda(), dk, dv, causal=True, split_kv=False)
    torch.cuda.synchronize()
    _check_oracle(o, lse, q, k1.expand(B, -1, -1, -1), v1.expand(B, -1, -1, -1), True, 1 / math.sqrt(D), dtype,
                  "broadcast kv")
