"""Properties of the HIP path that hold at any size (checked bitwise where the arithmetic is
identical), complementing the element-wise parity tests."""
import math

import pytest
import torch

import gqa_attention_forward_amd as fa
from gqa_attention_forward_amd.inputs import make_custom

pytestmark = pytest.mark.gpu


def _fwd(q, k, v, causal, scale=None):
    o, lse = fa.attention_forward(q, k, v, causal=causal, scale=scale, split_kv=False)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("causal", [True, False])
def test_deterministic(dtype, causal):
    q, k, v = make_custom(2, 8, 2, 700, 900, 128, dtype, seed=1, device="cuda")
    o1, l1 = _fwd(q, k, v, causal)
    o2, l2 = _fwd(q, k, v, causal)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D", [64, 128])
def test_gqa_equals_mha_on_repeated_kv(D):
    """Each (b, h) computes the same arithmetic on the same K/V values whether they come from a
    shared KV head or from a repeated copy: the results are bitwise equal."""
    B, Hq, Hkv, M, N = 2, 8, 2, 333, 444
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=2, device="cuda")
    g = Hq // Hkv
    o1, l1 = _fwd(q, k, v, True)
    o2, l2 = _fwd(q, k.repeat_interleave(g, 1).contiguous(), v.repeat_interleave(g, 1).contiguous(), True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("M,N", [(512, 512), (300, 1000), (1000, 300)])
def test_future_keys_do_not_leak(M, N):
    """Causal: replacing every key/value a row cannot see by other finite values leaves the row
    bitwise unchanged (masked logits give probability exactly 0)."""
    B, Hq, Hkv, D = 1, 4, 2, 128
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=3, device="cuda")
    o1, l1 = _fwd(q, k, v, True)
    # poison the keys after position `cut` and check the rows that only see keys <= cut
    cut = N // 2
    k2, v2 = k.clone(), v.clone()
    gen = torch.Generator(device="cpu").manual_seed(4)
    k2[:, :, cut + 1:] = (torch.randn(k2[:, :, cut + 1:].shape, generator=gen) * 30).to(k.dtype).cuda()
    v2[:, :, cut + 1:] = (torch.randn(v2[:, :, cut + 1:].shape, generator=gen) * 1000).to(v.dtype).cuda()
    o2, l2 = _fwd(q, k2, v2, True)
    last_row = cut - (N - M)  # rows i <= last_row see only keys j <= cut
    if last_row >= 0:
        assert torch.equal(o1[:, :, : last_row + 1], o2[:, :, : last_row + 1])
        assert torch.equal(l1[:, :, : last_row + 1], l2[:, :, : last_row + 1])
    if last_row + 1 < M:
        assert not torch.equal(o1[:, :, last_row + 1:], o2[:, :, last_row + 1:])


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_constant_v_returns_v(dtype):
    B, Hq, Hkv, M, N, D = 1, 4, 1, 256, 256, 128
    q, k, _ = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=5, device="cuda")
    c = torch.linspace(-2, 2, D, device="cuda").to(dtype)
    v = c.expand(B, Hkv, N, D).contiguous()
    o, _ = _fwd(q, k, v, True)
    # P is rounded to the input dtype before the MFMA while the row sum is not: the relative
    # deviation is at most about one rounding unit of the dtype
    rel = 2.0 ** -8 if dtype == torch.float16 else 2.0 ** -6
    assert (o.float() - c.float()).abs().max().item() <= rel * 2


def test_first_causal_row_is_v0():
    B, Hq, Hkv, M, N, D = 2, 4, 2, 128, 128, 64
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=6, device="cuda")
    o, lse = _fwd(q, k, v, True)
    g = Hq // Hkv
    for h in range(Hq):
        assert torch.equal(o[:, h, 0], v[:, h // g, 0])
    s00 = (q[:, :, 0].float() * k.repeat_interleave(g, 1)[:, :, 0].float()).sum(-1) / math.sqrt(D)
    assert torch.allclose(lse[:, :, 0], s00, atol=1e-4, rtol=1e-5)


def test_no_visible_key_rows():
    q, k, v = make_custom(1, 2, 1, 200, 50, 128, torch.bfloat16, seed=7, device="cuda")
    o, lse = _fwd(q, k, v, True)
    assert torch.all(o[:, :, :150] == 0)
    assert torch.all(torch.isneginf(lse[:, :, :150]))
    assert torch.isfinite(lse[:, :, 150:]).all()


def test_respects_stream():
    q, k, v = make_custom(1, 4, 2, 256, 256, 128, torch.float16, seed=8, device="cuda")
    o_ref, l_ref = _fwd(q, k, v, True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.attention_forward(q, k, v, causal=True, split_kv=False)
    s.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


@pytest.mark.parametrize("split_kv", [False, "auto", 3])
def test_forward_launcher_repeats_attention_forward(split_kv):
    """A launcher planned once gives, launch after launch, the bits attention_forward gives for
    the same call (plain and key-split paths; the split workspace lives in the launcher)."""
    q, k, v = make_custom(1, 8, 2, 77, 3000, 128, torch.float16, seed=4, device="cuda")
    o_ref, l_ref = fa.attention_forward(q, k, v, causal=True, split_kv=split_kv)
    launch, o, lse = fa.forward_launcher(q, k, v, causal=True, split_kv=split_kv)
    for _ in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        launch()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
