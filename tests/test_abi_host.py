"""The C-ABI library loads, exports every symbol include/fa.h declares, and rejects bad
arguments before touching the GPU (no compute calls here: this runs without a GPU)."""
import ctypes
import os
import re

import pytest

import gqa_attention_forward_amd as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    assert "fa_fwd" in names and "fa_strerror" in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_strerror_texts():
    assert fa.fa_strerror(0) == "success"
    for code in (-1, -2, -3, 12345):
        assert isinstance(fa.fa_strerror(code), str) and fa.fa_strerror(code)


GOOD = dict(q=0x1000, k=0x2000, v=0x3000, o=0x4000, lse=0x5000, B=1, Hq=2, Hkv=1, M=16, N=16, D=64,
            scale=0.125, causal=1, dtype=0, stream=None)


def _call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["M"], a["N"], a["D"],
                     a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(B=0), dict(Hq=0), dict(Hkv=0), dict(M=0), dict(N=-1), dict(D=0),
    dict(Hq=3, Hkv=2), dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(dtype=2), dict(dtype=-1),
])
def test_invalid_arguments(bad):
    assert _call(**bad) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(D=96), dict(D=256), dict(D=32), dict(q=0x1008), dict(lse=0x5004)])
def test_unsupported(bad):
    assert _call(**bad) == fa.FA_ERR_UNSUPPORTED
