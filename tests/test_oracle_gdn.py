"""Pins the fp64 Gated DeltaNet oracle: the page's chunk recurrence (with A from the triangular
solve) against the token-by-token gated delta rule it rewrites, and both against closed forms
(no writes: pure decay; no decay and orthonormal keys: exact recall of stored values)."""
import numpy as np
import pytest
import torch

import oracle
from gqa_attention_forward_amd.inputs import GdnWorkload, make_gdn_inputs


def _w(Hqk, Hv, DK, DV, init, seed=1, dtype=torch.bfloat16):
    return GdnWorkload("t", 1, 1, Hqk, Hv, DK, DV, dtype, seed, init_state=init)


@pytest.mark.parametrize("case", [
    # B, T, Hqk, Hv, DK, DV, init_state
    (1, 64, 1, 1, 16, 8, False),
    (2, 150, 2, 4, 16, 16, True),     # ragged last chunk, value heads in pairs
    (1, 200, 1, 3, 8, 12, True),      # three value heads on one key head
    (1, 130, 2, 2, 32, 32, False),
])
def test_chunked_equals_token_recurrence(case):
    B, T, Hqk, Hv, DK, DV, init = case
    w = _w(Hqk, Hv, DK, DV, init, seed=sum(case))
    q, k, v, g, beta, s0 = make_gdn_inputs(w, B=B, T=T)
    scale = DK ** -0.5
    A = oracle.gdn_kkt(k, g, beta, Hv)
    oc, sc = oracle.gdn_chunked(q, k, v, g, beta, A, scale, s0)
    orr, sr = oracle.gdn_recurrent(q, k, v, g, beta, scale, s0)
    np.testing.assert_allclose(oc, orr, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(sc, sr, rtol=1e-9, atol=1e-11)


def test_kkt_structure():
    """A = (I + L)^-1 with L strictly lower: unit diagonal, zero above it, and A = I without writes."""
    w = _w(1, 2, 16, 8, False, seed=3)
    q, k, v, g, beta, _ = make_gdn_inputs(w, B=1, T=100)
    A = oracle.gdn_kkt(k, g, beta, 2)
    for c0 in (0, 64):
        blk = A[0, c0:c0 + 64, 0, :]
        n = min(64, 100 - c0)
        assert np.allclose(np.diag(blk[:n, :n]), 1.0)
        assert np.all(np.triu(blk[:n, :n], 1) == 0.0)
        assert np.all(blk[:, n:] == 0.0)
    A0 = oracle.gdn_kkt(k, g, torch.zeros_like(beta), 2)
    for c0 in (0, 64):
        n = min(64, 100 - c0)
        assert np.array_equal(A0[0, c0:c0 + n, 0, :n], np.eye(n))


def test_no_writes_pure_decay():
    """beta = 0: nothing is written, S decays by the product of the gates and o_t = scale S_t^T q_t."""
    B, T, Hqk, Hv, DK, DV = 1, 100, 1, 2, 8, 4
    w = _w(Hqk, Hv, DK, DV, True, seed=4)
    q, k, v, g, beta, s0 = make_gdn_inputs(w, B=B, T=T)
    beta = torch.zeros_like(beta)
    A = oracle.gdn_kkt(k, g, beta, Hv)
    o, sf = oracle.gdn_chunked(q, k, v, g, beta, A, 0.5, s0)
    gd = g.double().numpy()
    total = gd[0, 63] + gd[0, 99]  # last cumulative log-gate of each chunk
    np.testing.assert_allclose(sf[0], np.exp(total)[:, None, None] * s0[0].double().numpy(), rtol=1e-12)
    qd = q.double().numpy()
    for t in (0, 63, 64, 99):
        decay = np.exp(gd[0, t] + (gd[0, 63] if t >= 64 else 0.0))
        expect = 0.5 * decay[:, None] * np.einsum("d,hde->he", qd[0, t, 0], s0[0].double().numpy())
        np.testing.assert_allclose(o[0, t], expect, rtol=1e-11, atol=1e-14)


def test_exact_recall_without_decay():
    """No decay (g = 0), beta = 1, orthonormal keys e_0, e_1, ...: the delta rule stores v_t under
    k_t exactly, so querying with k_i after step i returns scale * v_i (across chunk borders)."""
    B, T, Hqk, Hv, DK, DV = 1, 96, 1, 1, 128, 8
    w = _w(Hqk, Hv, DK, DV, False, seed=5)
    _, _, v, g, beta, _ = make_gdn_inputs(w, B=B, T=T)
    k = torch.zeros((B, T, Hqk, DK))
    for t in range(T):
        k[0, t, 0, t] = 1.0
    k = k.to(torch.bfloat16)
    qi = torch.zeros_like(k)
    rec = [3, 70, 95]  # query k_3 at every step >= 3 etc.: here query a stored key at t
    for t in range(T):
        qi[0, t, 0, rec[0] if t >= rec[0] else 0] = 1.0
    g = torch.zeros_like(g)
    beta = torch.ones_like(beta)
    A = oracle.gdn_kkt(k, g, beta, Hv)
    o, sf = oracle.gdn_chunked(qi, k, v, g, beta, A, 0.25)
    orr, _ = oracle.gdn_recurrent(qi, k, v, g, beta, 0.25)
    vd = v.double().numpy()
    for t in (3, 10, 64, 95):
        np.testing.assert_allclose(o[0, t, 0], 0.25 * vd[0, 3, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(orr[0, t, 0], 0.25 * vd[0, 3, 0], rtol=1e-12, atol=1e-14)
    # every stored pair is recalled from the final state
    for t in range(T):
        np.testing.assert_allclose(sf[0, 0, t], vd[0, t, 0], rtol=1e-12, atol=1e-14)


def test_gva_heads_read_their_key_head():
    """Value head h reads key/query head h // (Hv / Hqk): permuting the key heads permutes the
    outputs of the value heads in step."""
    B, T, Hqk, Hv, DK, DV = 1, 70, 2, 4, 8, 4
    w = _w(Hqk, Hv, DK, DV, False, seed=6)
    q, k, v, g, beta, _ = make_gdn_inputs(w, B=B, T=T)
    o, _ = oracle.gdn_recurrent(q, k, v, g, beta, 0.3)
    perm = [1, 0]
    vperm = v[:, :, [2, 3, 0, 1]]
    o2, _ = oracle.gdn_recurrent(q[:, :, perm], k[:, :, perm], vperm, g[:, :, [2, 3, 0, 1]],
                                 beta[:, :, [2, 3, 0, 1]], 0.3)
    np.testing.assert_allclose(o2, o[:, :, [2, 3, 0, 1]], rtol=1e-12, atol=1e-14)
    # and a wrong mapping (h % Hqk) would differ
    o3, _ = oracle.gdn_recurrent(q[:, :, perm], k[:, :, perm], v, g, beta, 0.3)
    assert np.abs(o3 - o).max() > 1e-3
