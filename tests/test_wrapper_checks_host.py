"""The torch wrappers check every tensor against the sizes they pass to the C ABI before any
launch: a tensor of the wrong shape or element type would otherwise send the kernels past its
allocation.  These run on the CPU: the checks of shape and dtype come before the device check,
so a mismatched CPU tensor must raise about the mismatch, and a well-formed CPU set must raise
only because it is not on a device."""
import pytest
import torch

import gqa_attention_forward_amd as fa

B, Hq, Hkv, M, N, D = 2, 4, 2, 8, 12, 64


def _bwd_args(dtype=torch.bfloat16):
    q = torch.zeros(B, Hq, M, D, dtype=dtype)
    k = torch.zeros(B, Hkv, N, D, dtype=dtype)
    v = torch.zeros(B, Hkv, N, D, dtype=dtype)
    o = torch.zeros(B, Hq, M, D, dtype=dtype)
    lse = torch.zeros(B, Hq, M, dtype=torch.float32)
    do = torch.zeros(B, Hq, M, D, dtype=dtype)
    return dict(q=q, k=k, v=v, o=o, lse=lse, dout=do)


BWD_BAD = [
    ("k", torch.zeros(B + 1, Hkv, N, D, dtype=torch.bfloat16), "shape"),
    ("k", torch.zeros(B, Hkv, N, D // 2, dtype=torch.bfloat16), "shape"),
    ("v", torch.zeros(B, Hkv, N + 1, D, dtype=torch.bfloat16), "shape"),
    ("v", torch.zeros(B, Hkv, N, D, dtype=torch.float16), "dtype"),
    ("o", torch.zeros(B, Hq, M, D, dtype=torch.float32), "dtype"),
    ("dout", torch.zeros(B, Hq, M, D, dtype=torch.float32), "dtype"),
    ("dout", torch.zeros(B, Hq, M + 1, D, dtype=torch.bfloat16), "shape"),
    ("lse", torch.zeros(B, Hq, M, dtype=torch.float16), "dtype"),
    ("lse", torch.zeros(B, Hq, M + 1, dtype=torch.float32), "shape"),
    ("o", torch.zeros(B, Hq, D, M, dtype=torch.bfloat16).transpose(2, 3), "contiguous"),
]


@pytest.mark.parametrize("name,bad,what", BWD_BAD, ids=[f"{n}-{w}-{i}" for i, (n, _, w) in enumerate(BWD_BAD)])
def test_backward_rejects_mismatch(name, bad, what):
    a = _bwd_args()
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=what):
        fa.attention_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], causal=True)


def test_backward_well_formed_cpu_tensors_fail_only_on_device():
    a = _bwd_args()
    with pytest.raises(ValueError, match="device tensor"):
        fa.attention_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], causal=True)


def test_backward_rejects_fp32_inputs():
    a = _bwd_args(torch.float32)
    with pytest.raises(TypeError):
        fa.attention_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"])


Bg, T, Hqk, Hv, DK, DV = 1, 70, 2, 4, 128, 64


def _gdn_args():
    dt = torch.bfloat16
    return dict(q=torch.zeros(Bg, T, Hqk, DK, dtype=dt), k=torch.zeros(Bg, T, Hqk, DK, dtype=dt),
                v=torch.zeros(Bg, T, Hv, DV, dtype=dt), g=torch.zeros(Bg, T, Hv), beta=torch.zeros(Bg, T, Hv),
                s0=torch.zeros(Bg, Hv, DK, DV), A=torch.zeros(Bg, T, Hv, 64, dtype=dt))


GDN_BAD = [
    ("k", torch.zeros(Bg, T - 1, Hqk, DK, dtype=torch.bfloat16), "shape"),
    ("k", torch.zeros(Bg, T, Hqk, DK, dtype=torch.float16), "dtype"),
    ("v", torch.zeros(Bg, T + 1, Hv, DV, dtype=torch.bfloat16), "shape"),
    ("g", torch.zeros(Bg, T, Hv - 1), "shape"),
    ("g", torch.zeros(Bg, T, Hv, dtype=torch.float64), "dtype"),
    ("beta", torch.zeros(Bg, T - 1, Hv), "shape"),
    ("s0", torch.zeros(Bg, Hv, DK, DV // 2), "shape"),
    ("s0", torch.zeros(Bg, Hv, DK, DV, dtype=torch.bfloat16), "dtype"),
    ("A", torch.zeros(Bg, T, Hv, 32, dtype=torch.bfloat16), "shape"),
    ("A", torch.zeros(Bg, T, Hv, 64, dtype=torch.float32), "dtype"),
]


@pytest.mark.parametrize("name,bad,what", GDN_BAD, ids=[f"{n}-{w}-{i}" for i, (n, _, w) in enumerate(GDN_BAD)])
def test_gdn_rejects_mismatch(name, bad, what):
    a = _gdn_args()
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=what):
        fa.gdn_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], s0=a["s0"], A=a["A"])


def test_gdn_well_formed_cpu_tensors_fail_only_on_device():
    a = _gdn_args()
    with pytest.raises(ValueError, match="device tensor"):
        fa.gdn_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], s0=a["s0"], A=a["A"])
