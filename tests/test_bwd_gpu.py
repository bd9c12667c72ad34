"""Parity of the backward pass (fa_bwd through the C ABI: prep, dQ and dK/dV kernels) against the
fp64 oracle's gradients, element by element, on shapes that span several tiles with ragged
tails, both masks, grouped heads, M != N and both head dims.

Tolerance (max-abs error over a tensor, relative to that tensor's largest reference value, with
a floor of 1e-3 for tensors that are exactly zero, such as dq of a row with a single visible
key): the kernels round P and dS to the input type before their MFMAs and the outputs once at
the end, so each output element carries a few half-ulps of the input type (2^-11 fp16, 2^-8
bf16) relative to the magnitudes being summed; 4e-3 (fp16) / 1.6e-2 (bf16) of max|ref| leaves
margin for the cancellation in dq and dk (their terms sum to zero over each row's keys).
Observed: <= 6.2e-4 (fp16) and <= 4.9e-3 (bf16).
"""
import math

import numpy as np
import pytest
import torch

import gqa_attention_forward_amd as fa
import oracle
from gqa_attention_forward_amd.inputs import make_custom

pytestmark = pytest.mark.gpu

REL = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}


def _dout(B, Hq, M, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, Hq, M, D), generator=g).to(dtype)


def _run(shape, seed):
    B, Hq, Hkv, M, N, D, causal, dtype = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=seed)
    do = _dout(B, Hq, M, D, dtype, seed + 1)
    scale = 1.0 / math.sqrt(D)
    dq_, dk_, dv_, ddo = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.attention_forward(dq_, dk_, dv_, causal=causal, scale=scale, split_kv=False)
    gq, gk, gv = fa.attention_backward(dq_, dk_, dv_, o, lse, ddo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, scale, causal)
    return (gq.cpu(), gk.cpu(), gv.cpu()), (rq, rk, rv)


def _check(got, ref, dtype, what):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().numpy()
        assert np.all(np.isfinite(g)), f"{what} {name} not finite"
        scale = max(np.abs(r).max(), 1e-3)
        err = np.abs(g - r).max()
        print(f"{what} {name}: max|err| {err:.3e}, max|ref| {scale:.3e}, rel {err / scale:.2e}", flush=True)
        assert err <= REL[dtype] * scale, f"{what} {name}"


SHAPES = [
    # B, Hq, Hkv, M, N, D, causal, dtype
    (1, 2, 1, 128, 128, 128, True, torch.float16),
    (1, 2, 1, 128, 128, 128, False, torch.bfloat16),
    (2, 4, 2, 300, 300, 128, True, torch.bfloat16),      # ragged tiles
    (1, 8, 2, 77, 300, 128, True, torch.float16),        # M < N: bottom-right offset
    (1, 4, 1, 300, 77, 128, True, torch.bfloat16),       # M > N: first 223 rows see no key
    (2, 2, 2, 200, 333, 128, False, torch.float16),
    (1, 4, 4, 129, 65, 64, False, torch.bfloat16),
    (1, 6, 3, 256, 520, 64, True, torch.float16),
    (3, 2, 1, 1, 1, 128, True, torch.float16),           # one query, one key
    (1, 2, 1, 1, 500, 64, True, torch.bfloat16),         # one query row
    (1, 8, 1, 512, 512, 128, True, torch.bfloat16),      # 8 query heads per KV head
    # grids that fill the CUs with 8-wave (256-row) dQ workgroups, ragged in M and N
    (2, 64, 8, 300, 333, 128, True, torch.bfloat16),
    (1, 256, 32, 260, 200, 128, False, torch.float16),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(str(x) for x in s[:7]) + str(s[7]).split(".")[-1])
def test_bwd_matches_oracle(shape):
    got, ref = _run(shape, seed=sum(shape[:6]))
    _check(got, ref, shape[7], f"bwd {shape}")


def test_bwd_deterministic():
    B, Hq, Hkv, M, N, D, causal, dtype = 2, 8, 2, 300, 400, 128, True, torch.bfloat16
    q, k, v = (t.cuda() for t in make_custom(B, Hq, Hkv, M, N, D, dtype, seed=3))
    do = _dout(B, Hq, M, D, dtype, 4).cuda()
    o, lse = fa.attention_forward(q, k, v, causal=causal, split_kv=False)
    a = fa.attention_backward(q, k, v, o, lse, do, causal=causal)
    b = fa.attention_backward(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_key_gradients_sum_to_zero_on_gpu():
    """sum_j dk_j = 0 for every (b, kv head) at a size the oracle is not run on (fp32 sum of the
    rounded outputs, relative to the summed magnitudes)."""
    B, Hq, Hkv, M, N, D, causal, dtype = 1, 8, 2, 2048, 2048, 128, True, torch.bfloat16
    q, k, v = (t.cuda() for t in make_custom(B, Hq, Hkv, M, N, D, dtype, seed=8))
    do = _dout(B, Hq, M, D, dtype, 9).cuda()
    o, lse = fa.attention_forward(q, k, v, causal=causal, split_kv=False)
    _, dk, _ = fa.attention_backward(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    s = dk.float().sum(dim=2).abs().max().item()
    mag = dk.float().abs().sum(dim=2).max().item()
    print(f"max |sum_j dk_j| = {s:.3e} vs sum |dk_j| = {mag:.3e}", flush=True)
    assert s <= 1e-2 * mag


@pytest.mark.timeout(400)  # the oracle's pass over one KV head at this size takes about a minute on 16 cores
def test_long_causal_prefill_one_kv_head():
    """The backward at the long causal GQA prefill's full size (1 x 32/8 heads x 16384^2, bf16,
    peaky keys): dk and dv of one whole KV head (every key, summed over its 4 query heads) and dq
    of sampled rows of those heads -- the first and last 64 of each head and 512 random ones --
    against the oracle's per-group gradients."""
    from gqa_attention_forward_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS["long_causal_gqa_16k"]
    q, k, v, _ = make_inputs(w)
    do = _dout(w.B, w.Hq, w.M, w.D, w.dtype, 1003)
    dq_, dk_, dv_, ddo = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.attention_forward(dq_, dk_, dv_, causal=True, scale=w.scale, split_kv=False)
    gq, gk, gv = fa.attention_backward(dq_, dk_, dv_, o, lse, ddo, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    hk, g = 3, w.Hq // w.Hkv
    rng = np.random.default_rng(17)
    rows = set()
    for h in range(g):
        rows.update(range(h * w.M, h * w.M + 64))
        rows.update(range((h + 1) * w.M - 64, (h + 1) * w.M))
    rows.update(rng.choice(g * w.M, 512, replace=False).tolist())
    rows = np.array(sorted(rows), dtype=np.int64)
    print(f"GPU backward done; oracle over KV head {hk} ({g} query heads x {w.M} rows x {w.N} keys)", flush=True)
    rq, rk, rv = oracle.attn_bwd_slice(q, k, v, do, w.scale, True, 0, hk, (0, w.N), rows)
    got_q = gq[0, hk * g:(hk + 1) * g].reshape(g * w.M, w.D)[torch.from_numpy(rows).cuda()].cpu()
    _check((got_q, gk[0, hk].cpu(), gv[0, hk].cpu()), (rq, rk, rv), w.dtype,
           f"long causal prefill, KV head {hk}: all {w.N} keys, {rows.size} dq rows")
