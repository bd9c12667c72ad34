"""Pins the fp64 oracle with properties that the mathematics of masked softmax attention fixes,
and with an independent library routine (torch's CPU float64 scaled_dot_product_attention
given an explicit bottom-right boolean mask).

A mistake in any part of the oracle -- a dropped scale, a wrong sign, the wrong KV head,
the wrong mask offset, a transposed operand, a missing max subtraction -- fails at least
one test here or in test_oracle_hand.py.
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
    (2, 4, 2, 9, 23, 16, True),     # M < N: bottom-right offset 14, ragged sizes
    (1, 3, 1, 20, 7, 4, True),      # M > N: first 13 rows see no key
    (2, 4, 4, 13, 17, 8, False),
    (1, 8, 2, 5, 64, 32, True),
]


def _mask(M, N, causal):
    i = torch.arange(M)[:, None]
    j = torch.arange(N)[None, :]
    return (j <= i + (N - M)) if causal else torch.ones(M, N, dtype=torch.bool)


def _sdpa_reference(q, k, v, scale, causal):
    """torch CPU float64 SDPA with an explicit boolean mask and repeat-interleaved KV heads."""
    g = q.shape[1] // k.shape[1]
    kk = k.double().repeat_interleave(g, dim=1)
    vv = v.double().repeat_interleave(g, dim=1)
    mask = _mask(q.shape[2], k.shape[2], causal)
    o = torch.nn.functional.scaled_dot_product_attention(q.double(), kk, vv, attn_mask=mask, scale=scale)
    s = torch.matmul(q.double(), kk.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy(), mask


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_matches_torch_sdpa_float64(shape, dtype):
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=11)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal)
    ro, rlse, mask = _sdpa_reference(q, k, v, scale, causal)
    seen = mask.any(dim=1).numpy()  # rows with at least one visible key
    np.testing.assert_allclose(o[:, :, seen], ro[:, :, seen], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, seen], rlse[:, :, seen], rtol=1e-12, atol=1e-12)
    # rows with no visible key: O = 0 and lse = -inf by definition
    assert np.all(o[:, :, ~seen] == 0.0)
    assert np.all(np.isneginf(lse[:, :, ~seen]))


@pytest.mark.parametrize("shape", SHAPES)
def test_probabilities_rows_sum_to_one_and_mask_is_exact(shape):
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, _ = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=3)
    mask = _mask(M, N, causal).numpy()
    for b in range(B):
        for h in range(Hq):
            P = oracle.attn_probs(q, k, 1.0 / math.sqrt(D), causal, b, h)
            assert np.all(P[~mask] == 0.0)
            assert np.all(P[mask] > 0.0)
            seen = mask.any(axis=1)
            np.testing.assert_allclose(P[seen].sum(axis=1), 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES)
def test_constant_v_returns_v(shape):
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, _ = make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=5)
    c = torch.linspace(-3, 3, D).to(torch.bfloat16)
    v = c.expand(B, Hkv, N, D).contiguous()
    o, _ = oracle.attn_fwd(q, k, v, 0.3, causal)
    seen = _mask(M, N, causal).any(dim=1).numpy()
    want = np.broadcast_to(c.double().numpy(), o[:, :, seen].shape)
    np.testing.assert_allclose(o[:, :, seen], want, rtol=1e-14, atol=1e-14)


def test_causal_first_row_is_v0():
    B, Hq, Hkv, M, N, D = 2, 4, 2, 32, 32, 16
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=7)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_fwd(q, k, v, scale, True)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            v0 = v[b, h // g, 0].double().numpy()
            assert np.array_equal(o[b, h, 0], v0)
            s00 = scale * float((q[b, h, 0].double() * k[b, h // g, 0].double()).sum())
            assert lse[b, h, 0] == pytest.approx(s00, rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("M,N", [(8, 64), (16, 16), (5, 3), (512 // 32, 8192 // 32)])
def test_zero_queries_give_mean_of_visible_values(M, N):
    """q = 0 makes every visible logit 0: O_i is the mean of the visible v_j and
    lse_i = ln(#visible) = ln(min(N, i + 1 + N - M)).  This pins the bottom-right offset."""
    B, Hq, Hkv, D = 1, 2, 1, 8
    _, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=9)
    q = torch.zeros(B, Hq, M, D, dtype=torch.float16)
    o, lse = oracle.attn_fwd(q, k, v, 0.125, True)
    vd = v.double().numpy()
    for i in range(M):
        n = min(N, max(0, i + 1 + N - M))
        if n == 0:
            assert np.all(o[0, :, i] == 0.0) and np.all(np.isneginf(lse[0, :, i]))
            continue
        want = vd[0, 0, :n].mean(axis=0)
        np.testing.assert_allclose(o[0, 0, i], want, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=1e-14)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("block", [1, 3, 64, 10**6])
def test_online_softmax_modes_agree_with_definition(shape, block):
    B, Hq, Hkv, M, N, D, causal = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=13, peak_rate=0.2)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal)
    for fn in (oracle.attn_fwd_blockwise, oracle.attn_fwd_stepnorm):
        o2, lse2 = fn(q, k, v, scale, causal, block)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
        fin = np.isfinite(lse)
        np.testing.assert_allclose(lse2[fin], lse[fin], rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(lse2[~fin]))


@pytest.mark.parametrize("causal", [True, False])
def test_gqa_equals_mha_on_repeated_kv(causal):
    B, Hq, Hkv, M, N, D = 2, 8, 2, 12, 12, 16
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=17)
    g = Hq // Hkv
    o, lse = oracle.attn_fwd(q, k, v, 0.25, causal)
    o2, lse2 = oracle.attn_fwd(q, k.repeat_interleave(g, 1).contiguous(), v.repeat_interleave(g, 1).contiguous(),
                               0.25, causal)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # a different (wrong) head mapping gives a different result
    o3, _ = oracle.attn_fwd(q, k.repeat(1, g, 1, 1).contiguous(), v.repeat(1, g, 1, 1).contiguous(), 0.25, causal)
    assert not np.allclose(o, o3)


def test_key_shift_changes_lse_only():
    """Adding u to every key adds scale*q.u to every logit of a row: O is unchanged and
    lse shifts by exactly that amount.  Integer-valued inputs keep k + u exact."""
    B, Hq, Hkv, M, N, D = 1, 2, 1, 6, 10, 4
    g = torch.Generator().manual_seed(21)
    q = torch.randint(-3, 4, (B, Hq, M, D), generator=g).to(torch.float16)
    k = torch.randint(-3, 4, (B, Hkv, N, D), generator=g).to(torch.float16)
    v = torch.randn(B, Hkv, N, D, generator=g).to(torch.float16)
    u = torch.tensor([1.0, -2.0, 0.0, 3.0], dtype=torch.float16)
    scale = 0.25
    for causal in (True, False):
        o, lse = oracle.attn_fwd(q, k, v, scale, causal)
        o2, lse2 = oracle.attn_fwd(q, (k + u).contiguous(), v, scale, causal)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
        shift = scale * (q.double() @ u.double()).numpy()
        fin = np.isfinite(lse)
        np.testing.assert_allclose((lse2 - lse)[fin], shift[fin], rtol=1e-12, atol=1e-12)


def test_joint_permutation_of_keys_is_invisible_without_mask():
    B, Hq, Hkv, M, N, D = 1, 2, 2, 7, 19, 8
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=23)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(1))
    o, lse = oracle.attn_fwd(q, k, v, 0.3, False)
    o2, lse2 = oracle.attn_fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), 0.3, False)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)
    # ... but the causal mask does see the order
    o3, _ = oracle.attn_fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), 0.3, True)
    o4, _ = oracle.attn_fwd(q, k, v, 0.3, True)
    assert not np.allclose(o3, o4)


def test_rows_mode_equals_full_mode():
    B, Hq, Hkv, M, N, D = 2, 4, 2, 33, 47, 16
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=29)
    o, lse = oracle.attn_fwd(q, k, v, 0.25, True)
    rows = np.array([0, 5, 32, 33, 100, B * Hq * M - 1])
    o2, lse2 = oracle.attn_fwd_rows(q, k, v, 0.25, True, rows)
    assert np.array_equal(o2, o.reshape(-1, D)[rows])
    assert np.array_equal(lse2, lse.reshape(-1)[rows])


def test_scale_enters_the_logits():
    """Doubling the scale equals doubling q (exact in fp16): pins where scale is applied."""
    B, Hq, Hkv, M, N, D = 1, 2, 1, 8, 8, 8
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=31)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    o2, lse2 = oracle.attn_fwd((q * 2).contiguous(), k, v, 0.25, True)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


def test_result_does_not_depend_on_thread_count():
    # every row is computed on its own, in index order: one thread and many give the same bits
    q, k, v = make_custom(2, 4, 2, 37, 53, 64, torch.float16, seed=11)
    full_o, full_lse = oracle.attn_fwd(q, k, v, 0.125, True)
    prev = oracle.set_threads(1)
    try:
        assert oracle.threads_used() == 1
        one_o, one_lse = oracle.attn_fwd(q, k, v, 0.125, True)
    finally:
        oracle.set_threads(prev)
    assert oracle.threads_used() == prev
    assert np.array_equal(full_o, one_o) and np.array_equal(full_lse, one_lse)
