"""Pins the fp64 oracle's backward (gradients of O with respect to q, k, v) to things other than
itself: torch's CPU float64 autograd through scaled_dot_product_attention (an independent
library derivation), central finite differences of the oracle's own (separately pinned)
forward on tiny inputs, and identities the mathematics fixes.

A mistake in the backward -- the softmax Jacobian's mean term dropped, a missing scale, dk and
dq swapped, dv from dP instead of P, the wrong KV head, a wrong mask -- fails at least one test.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gqa_attention_forward_amd.inputs import make_custom

SHAPES = [
    # B, Hq, Hkv, M, N, D, causal
    (1, 2, 1, 16, 16, 8, True),
    (2, 4, 2, 9, 23, 16, True),     # M < N: bottom-right offset 14
    (1, 3, 1, 20, 7, 4, True),      # M > N: first 13 rows see no key
    (2, 4, 4, 13, 17, 8, False),
    (1, 8, 2, 5, 40, 32, True),
]


def _mask(M, N, causal):
    i = torch.arange(M)[:, None]
    j = torch.arange(N)[None, :]
    return (j <= i + (N - M)) if causal else torch.ones(M, N, dtype=torch.bool)


def _torch_grads(q, k, v, do, scale, causal):
    """torch float64 autograd of SDPA with an explicit boolean mask; GQA by repeat-interleave
    (whose backward sums the group's heads).  Rows without a visible key are excluded from the
    loss (SDPA returns NaN for them; the definition gives O = 0 there, a constant)."""
    g = q.shape[1] // k.shape[1]
    qd = q.double().requires_grad_(True)
    kd = k.double().requires_grad_(True)
    vd = v.double().requires_grad_(True)
    mask = _mask(q.shape[2], k.shape[2], causal)
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd.repeat_interleave(g, dim=1),
                                                         vd.repeat_interleave(g, dim=1), attn_mask=mask, scale=scale)
    seen = mask.any(dim=1)
    loss = (o[:, :, seen] * do.double()[:, :, seen]).sum()
    loss.backward()
    return qd.grad.numpy(), kd.grad.numpy(), vd.grad.numpy(), seen.numpy()


def _dout(B, Hq, M, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, Hq, M, D), generator=g).to(dtype)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_matches_torch_autograd_float64(shape, dtype):
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=31)
    do = _dout(B, Hq, M, D, dtype, 32)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal)
    tq, tk, tv, seen = _torch_grads(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq[:, :, seen], tq[:, :, seen], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv, rtol=1e-10, atol=1e-11)
    assert np.all(dq[:, :, ~seen] == 0.0)  # a row that sees no key has no gradient


def _grid_inputs(B, Hq, Hkv, M, N, D, seed):
    """fp16 values on the grid of multiples of 2^-7 inside (-1.5, 1.5): every +-2^-10 step of
    one element is exactly representable in fp16 (ulp <= 2^-10 below 2)."""
    g = torch.Generator().manual_seed(seed)

    def draw(*s):
        return (torch.randint(-190, 191, s, generator=g).double() / 128.0).half()

    return draw(B, Hq, M, D), draw(B, Hkv, N, D), draw(B, Hkv, N, D), draw(B, Hq, M, D)


@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 7, 4, True), (1, 2, 2, 4, 3, 4, False), (2, 2, 1, 6, 4, 4, True)])
def test_central_differences_of_the_oracle_forward(shape):
    """dL/dx for L = sum(O * dO), by central differences of the oracle's fp64 forward with a step
    of 2^-10 (exact in fp16 on these inputs), for every element of q, k and v."""
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, v, do = _grid_inputs(B, Hq, Hkv, M, N, D, seed=sum(shape))
    scale = 0.5
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal)
    W = do.double().numpy()
    h = 2.0 ** -10

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, scale, causal)
        return float((o * W).sum())

    for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = t.reshape(-1)
        num = np.empty(flat.numel())
        for idx in range(flat.numel()):
            plus, minus = flat.clone(), flat.clone()
            plus[idx] = (flat[idx].double() + h).half()
            minus[idx] = (flat[idx].double() - h).half()
            assert plus[idx].double() - minus[idx].double() == 2 * h  # the step is exact
            args = {"q": q, "k": k, "v": v}
            args[name] = plus.reshape(t.shape)
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = minus.reshape(t.shape)
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad.reshape(-1), num, rtol=2e-5, atol=2e-6, err_msg=name)


@pytest.mark.parametrize("shape", SHAPES)
def test_key_gradients_sum_to_zero(shape):
    """Every row's softmax Jacobian annihilates constants, so sum_j dz_ij = 0 and therefore
    sum_j dk_j = scale * sum_i q_i sum_j dz_ij = 0 for every (b, kv head)."""
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=41)
    do = _dout(B, Hq, M, D, torch.float16, 42)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.3, causal)
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12 * max(1.0, np.abs(dk).max())


def test_key_shift_invariance():
    """Adding one vector c to every key leaves every softmax row unchanged, hence dv, dk and dq
    (dq_i = scale sum_j dz_ij (k_j + c) and sum_j dz_ij = 0).  Values on a coarse grid keep the
    shifted keys exact in fp16."""
    B, Hq, Hkv, M, N, D, causal = 1, 4, 2, 9, 12, 8, True
    q, k, v, do = _grid_inputs(B, Hq, Hkv, M, N, D, seed=5)
    c = torch.tensor([0.25, -0.5, 0.125, 0.0, 1.0, -0.25, 0.5, -1.0], dtype=torch.float64)
    k2 = (k.double() + c).half()
    assert torch.equal(k2.double(), k.double() + c)
    g1 = oracle.attn_bwd(q, k, v, do, 0.4, causal)
    g2 = oracle.attn_bwd(q, k2, v, do, 0.4, causal)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11)


def test_constant_upstream_gradient():
    """dO_i = u for every row: dv_j = sum_i P_ij u and each row's P sums to 1, so
    sum_j dv_j = (rows that see a key) * u, summed over the group's query heads."""
    B, Hq, Hkv, M, N, D, causal = 1, 6, 2, 10, 7, 8, True   # M > N: the first 3 rows see nothing
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=6)
    u = torch.linspace(-1, 1, D).to(torch.bfloat16)
    do = u.expand(B, Hq, M, D).contiguous()
    _, _, dv = oracle.attn_bwd(q, k, v, do, 0.35, causal)
    seen_rows = int(_mask(M, N, causal).any(dim=1).sum())
    g = Hq // Hkv
    expect = g * seen_rows * u.double().numpy()
    np.testing.assert_allclose(dv.sum(axis=2), np.broadcast_to(expect, (B, Hkv, D)), rtol=1e-12, atol=1e-12)


def test_constant_values_give_no_score_gradient():
    """With every v_j equal, dP_ij = dO_i . v does not depend on j, so dz = 0: dq = dk = 0,
    while dv_j = sum_i P_ij dO_i still flows."""
    B, Hq, Hkv, M, N, D, causal = 1, 2, 1, 8, 8, 8, True
    q, k, _ = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=7)
    v = torch.linspace(-2, 2, D).half().expand(B, Hkv, N, D).contiguous()
    do = _dout(B, Hq, M, D, torch.float16, 8)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.35, causal)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    assert np.abs(dv).max() > 0.1


def test_gqa_equals_summed_mha():
    """Grouped KV heads: dq equals the MHA gradient on repeat-interleaved K/V, and dk/dv equal the
    MHA dk/dv summed over each group's query heads (and differ from a wrong grouping)."""
    B, Hq, Hkv, M, N, D, causal = 2, 6, 2, 7, 11, 8, True
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=9)
    do = _dout(B, Hq, M, D, torch.float16, 10)
    g = Hq // Hkv
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.3, causal)
    mq, mk, mv = oracle.attn_bwd(q, k.repeat_interleave(g, dim=1), v.repeat_interleave(g, dim=1), do, 0.3, causal)
    np.testing.assert_allclose(dq, mq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, mk.reshape(B, Hkv, g, N, D).sum(axis=2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, mv.reshape(B, Hkv, g, N, D).sum(axis=2), rtol=1e-11, atol=1e-12)
    wrong = mk.reshape(B, g, Hkv, N, D).sum(axis=1)  # heads h % Hkv grouped instead
    assert np.abs(dk - wrong).max() > 1e-3


def test_zero_upstream_gradient():
    q, k, v = make_custom(1, 2, 1, 6, 6, 8, torch.float16, seed=12)
    do = torch.zeros(1, 2, 6, 8, dtype=torch.float16)
    for g in oracle.attn_bwd(q, k, v, do, 0.3, True):
        assert np.all(g == 0.0)


@pytest.mark.parametrize("shape", SHAPES)
def test_slice_matches_torch_autograd_float64(shape):
    """The per-group slice mode (dk, dv of a key range; dq of chosen rows) against torch autograd,
    for every group, a key range that starts and ends mid-sequence, and every row."""
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=41)
    do = _dout(B, Hq, M, D, torch.bfloat16, 42)
    scale = 1.0 / math.sqrt(D)
    tq, tk, tv, seen = _torch_grads(q, k, v, do, scale, causal)
    g = Hq // Hkv
    j0, j1 = N // 3, N - N // 4
    for b in range(B):
        for hk in range(Hkv):
            rows = np.arange(g * M)
            sq, sk, sv = oracle.attn_bwd_slice(q, k, v, do, scale, causal, b, hk, (j0, j1), rows)
            ref_q = tq[b, hk * g:(hk + 1) * g].reshape(g * M, D)
            row_seen = np.tile(seen, g)
            np.testing.assert_allclose(sq[row_seen], ref_q[row_seen], rtol=1e-10, atol=1e-11)
            assert np.all(sq[~row_seen] == 0.0)
            np.testing.assert_allclose(sk, tk[b, hk, j0:j1], rtol=1e-10, atol=1e-11)
            np.testing.assert_allclose(sv, tv[b, hk, j0:j1], rtol=1e-10, atol=1e-11)


def test_slice_equals_whole_backward_and_rejects_bad_arguments():
    B, Hq, Hkv, M, N, D = 2, 4, 2, 30, 41, 16
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=43)
    do = _dout(B, Hq, M, D, torch.float16, 44)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.25, True)
    rows = np.array([0, 5, 29, 30, 59], dtype=np.int64)   # rows of both heads of the group
    sq, sk, sv = oracle.attn_bwd_slice(q, k, v, do, 0.25, True, 1, 1, (0, N), rows)
    ref_q = dq[1, 2:4].reshape(2 * M, D)[rows]
    np.testing.assert_allclose(sq, ref_q, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sk, dk[1, 1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sv, dv[1, 1], rtol=1e-12, atol=1e-14)
    for bad in (dict(b=2), dict(hk=2), dict(key_range=(5, 3)), dict(key_range=(0, N + 1)),
                dict(rows=np.array([2 * M], dtype=np.int64))):
        a = dict(b=0, hk=0, key_range=(0, N), rows=rows)
        a.update(bad)
        with pytest.raises(ValueError):
            oracle.attn_bwd_slice(q, k, v, do, 0.25, True, a["b"], a["hk"], a["key_range"], a["rows"])
