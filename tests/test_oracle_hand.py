"""Pins the fp64 oracle to hand-sized cases with closed-form answers (tests/golden/hand_cases.json)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
CONST = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0), "-inf": -math.inf,
         "7/3": 7.0 / 3.0, "15/4": 15.0 / 4.0, "1+ln2": 1.0 + math.log(2.0)}


def _val(x):
    return CONST[x] if isinstance(x, str) else float(x)


def _arr(nested):
    return np.vectorize(_val, otypes=[np.float64])(np.array(nested, dtype=object))


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_case(case, dtype):
    q = torch.tensor(_arr(case["q"]), dtype=torch.float64).to(dtype)
    k = torch.tensor(_arr(case["k"]), dtype=torch.float64).to(dtype)
    v = torch.tensor(_arr(case["v"]), dtype=torch.float64).to(dtype)
    # the inputs are small integers / dyadic fractions: exact in both dtypes
    assert torch.equal(q.double(), torch.tensor(_arr(case["q"])))
    scale = _val(case["scale"])
    o, lse = oracle.attn_fwd(q, k, v, scale, case["causal"])
    want_o, want_lse = _arr(case["o"]), _arr(case["lse"])
    np.testing.assert_allclose(o, want_o, rtol=1e-14, atol=1e-14)
    finite = np.isfinite(want_lse)
    np.testing.assert_allclose(lse[finite], want_lse[finite], rtol=1e-14, atol=1e-14)
    assert np.all(np.isneginf(lse[~finite]))
    # the two online-softmax modes reproduce the same closed forms
    for block in (1, 2, 3):
        for fn in (oracle.attn_fwd_blockwise, oracle.attn_fwd_stepnorm):
            o2, lse2 = fn(q, k, v, scale, case["causal"], block)
            np.testing.assert_allclose(o2, want_o, rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(lse2[finite], want_lse[finite], rtol=1e-14, atol=1e-14)
            assert np.all(np.isneginf(lse2[~finite]))


def test_rows_mode_matches_closed_form():
    case = [c for c in _cases() if c["name"] == "causal_two_by_two"][0]
    q = torch.tensor(_arr(case["q"])).half()
    k = torch.tensor(_arr(case["k"])).half()
    v = torch.tensor(_arr(case["v"])).half()
    o, lse = oracle.attn_fwd_rows(q, k, v, _val(case["scale"]), True, [1, 0])
    np.testing.assert_allclose(o[:, 0], [7.0, 4.0], rtol=1e-14)
    np.testing.assert_allclose(lse, [math.log(4.0), 0.0], rtol=1e-14, atol=1e-15)
