"""Parity of the Gated DeltaNet kernels (through the C ABI) against the fp64 oracle.

gdn_kkt: A against the oracle's (I + L)^-1, within the rounding of A to the input type
(max-abs error <= 2^-7 max(1, max|A|) for bf16, 2^-10 for fp16: half an ulp plus the fp32 solve).
gdn_chunk_fwd: output and final state against the oracle's chunk recurrence fed the same A (the
GPU's, decoded), within the page's 5e-3 max error scaled by the reference's magnitude (floor 1);
and against the token-by-token recurrence (exact A) within twice that.
"""
import math

import numpy as np
import pytest
import torch

import gqa_attention_forward_amd as fa
import oracle
from gqa_attention_forward_amd.inputs import GDN_WORKLOADS, GdnWorkload, make_gdn_inputs

pytestmark = pytest.mark.gpu

A_TOL = {torch.bfloat16: 2.0 ** -7, torch.float16: 2.0 ** -10}
TOL = 5e-3


def _case(B, T, Hqk, Hv, DV, dtype, init, seed):
    w = GdnWorkload("t", B, T, Hqk, Hv, 128, DV, dtype, seed, init_state=init)
    return w, make_gdn_inputs(w)


def _err(got, ref, what):
    m = max(1.0, float(np.abs(ref).max()))
    e = float(np.abs(got - ref).max())
    print(f"{what}: max|err| {e:.3e}, max|ref| {np.abs(ref).max():.3e}", flush=True)
    return e / m


CASES = [
    # B, T, Hqk, Hv, DV, dtype, init_state
    (1, 64, 1, 1, 64, torch.bfloat16, False),
    (1, 200, 2, 4, 128, torch.bfloat16, True),    # ragged last chunk, value heads in pairs
    (2, 256, 1, 3, 64, torch.float16, True),      # three value heads per key head
    (1, 1000, 4, 4, 128, torch.bfloat16, False),  # 16 chunks
    (1, 1, 1, 2, 64, torch.float16, False),        # one token
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(x) for x in c[:5]) + str(c[5]).split(".")[-1] + str(c[6]))
def test_gdn_matches_oracle(case):
    B, T, Hqk, Hv, DV, dtype, init = case
    w, (q, k, v, g, beta, s0) = _case(B, T, Hqk, Hv, DV, dtype, init, seed=T + Hv)
    dev = [t.cuda() if t is not None else None for t in (q, k, v, g, beta, s0)]
    o, sf, A = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale)
    torch.cuda.synchronize()
    A_ref = oracle.gdn_kkt(k, g, beta, Hv)
    A_gpu = A.cpu().double().numpy()
    n_rows = np.arange(T) % 64
    valid = np.arange(64)[None, :] <= (np.minimum(64, T - (np.arange(T) // 64) * 64) - 1)[:, None]
    diff = np.abs(A_gpu - A_ref)[:, :, :, :] * valid[None, :, None, :]
    a_err = diff.max() / max(1.0, np.abs(A_ref).max())
    print(f"A: max rel err {a_err:.3e} (tol {A_TOL[dtype]:.1e})", flush=True)
    assert a_err <= A_TOL[dtype]
    # the chunk recurrence on the GPU's A
    A_used = A_gpu * valid[None, :, None, :]
    ro, rs = oracle.gdn_chunked(q, k, v, g, beta, A_used, w.scale, s0)
    assert np.all(np.isfinite(o.cpu().float().numpy()))
    assert _err(o.cpu().double().numpy(), ro, "O vs chunked oracle") <= TOL
    assert _err(sf.cpu().double().numpy(), rs, "state vs chunked oracle") <= TOL
    # and the token recurrence with the exact A
    to, ts = oracle.gdn_recurrent(q, k, v, g, beta, w.scale, s0)
    assert _err(o.cpu().double().numpy(), to, "O vs token recurrence") <= 2 * TOL
    assert _err(sf.cpu().double().numpy(), ts, "state vs token recurrence") <= 2 * TOL


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(x) for x in c[:5]) + str(c[5]).split(".")[-1] + str(c[6]))
def test_gdn_two_modes_identical(case):
    """The one-kernel mode and the state walk + parallel output kernels apply the same products
    in the same order to the same rounded operands: their outputs and states agree bit for bit."""
    B, T, Hqk, Hv, DV, dtype, init = case
    w, (q, k, v, g, beta, s0) = _case(B, T, Hqk, Hv, DV, dtype, init, seed=T + Hv + 1)
    dev = [t.cuda() if t is not None else None for t in (q, k, v, g, beta, s0)]
    o1, s1, A = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, two_kernel=False)
    o2, s2, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, two_kernel=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_gdn_deterministic():
    w, (q, k, v, g, beta, s0) = _case(1, 300, 2, 4, 128, torch.bfloat16, True, seed=11)
    dev = [t.cuda() for t in (q, k, v, g, beta, s0)]
    a = fa.gdn_prefill(*dev[:5], s0=dev[5])
    b = fa.gdn_prefill(*dev[:5], s0=dev[5])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _valid_cols(T):
    """[T, 64] mask of the A columns inside each token's chunk (a ragged last chunk is shorter)."""
    return np.arange(64)[None, :] <= (np.minimum(64, T - (np.arange(T) // 64) * 64) - 1)[:, None]


@pytest.mark.parametrize("name", list(GDN_WORKLOADS))
def test_gdn_workload_full(name):
    """The benchmark workloads at full length: every token and value head of batch 0 (the long
    workload has one batch), so the final state is compared after every chunk of the sequence.
    A against the oracle's (I + L)^-1; O and the final state against the oracle's chunk recurrence
    fed the GPU's A (the page's 5e-3 bar) and fed its own exact A (twice that: the GPU's A is
    rounded to the input type)."""
    w = GDN_WORKLOADS[name]
    q, k, v, g, beta, s0 = make_gdn_inputs(w)
    dev = [t.cuda() if t is not None else None for t in (q, k, v, g, beta, s0)]
    o, sf, A = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(sf).all() and torch.isfinite(o.float()).all()
    for mode in (False, True):  # the library's pick equals both modes, bit for bit
        o1, s1, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, two_kernel=mode)
        torch.cuda.synchronize()
        assert torch.equal(o, o1) and torch.equal(sf, s1), f"two_kernel={mode} differs"
        del o1, s1
    del dev
    T = w.T
    sl = lambda t: t[:1].contiguous() if t is not None else None  # noqa: E731
    qb, kb, vb, gb, bb, s0b = (sl(t) for t in (q, k, v, g, beta, s0))
    valid = _valid_cols(T)[None, :, None, :]
    A_gpu = A[:1].cpu().double().numpy() * valid
    A_ref = oracle.gdn_kkt(kb, gb, bb, w.Hv) * valid
    a_err = float(np.abs(A_gpu - A_ref).max()) / max(1.0, float(np.abs(A_ref).max()))
    print(f"{name} A ({T} tokens x {w.Hv} heads of batch 0): max rel err {a_err:.3e} (tol {A_TOL[w.dtype]:.1e})",
          flush=True)
    assert a_err <= A_TOL[w.dtype]
    og = o[:1].cpu().double().numpy()
    sg = sf[:1].cpu().double().numpy()
    ro, rs = oracle.gdn_chunked(qb, kb, vb, gb, bb, A_gpu, w.scale, s0b)
    assert _err(og, ro, f"{name} O, all {T} tokens of batch 0, oracle on the GPU's A") <= TOL
    assert _err(sg, rs, f"{name} state after {(T + 63) // 64} chunks, oracle on the GPU's A") <= TOL
    ro, rs = oracle.gdn_chunked(qb, kb, vb, gb, bb, A_ref, w.scale, s0b)
    assert _err(og, ro, f"{name} O, all {T} tokens of batch 0, oracle on its own A") <= 2 * TOL
    assert _err(sg, rs, f"{name} state after {(T + 63) // 64} chunks, oracle on its own A") <= 2 * TOL
