"""Parity of the Gated DeltaNet kernels (through the C ABI) against the fp64 oracle.

gdn_kkt: A against the oracle's (I + L)^-1, within the rounding of A to the input type
(max-abs error <= 2^-7 max(1, max|A|) for bf16, 2^-10 for fp16: half an ulp plus the fp32 solve).
gdn_chunk_fwd: output and final state against the oracle's chunk recurrence fed the same A (the
GPU's, decoded), within the page's 5e-3 max error scaled by the reference's magnitude (floor 1);
and against the token-by-token recurrence (exact A) within twice that.
gdn_chunk_fwd_segmented: the same bars.  It re-associates the recurrence (run start states from
the runs' linear maps), so it is compared with the oracle, not bit for bit with the sequential
modes; gates close to 1 keep those maps far from zero, so the combine of start states is
exercised (with the default gates a map dies out within a few chunks).
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
    runs = fa.gdn_segment_plan(w.B, w.T, w.Hv, w.DV)
    print(f"{name}: the library picks {runs} run(s) of chunks", flush=True)
    # the sequential modes agree bit for bit; the library's pick is their result or, segmented,
    # the explicit segmented call's
    o_one, s_one, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, two_kernel=False)
    o_two, s_two, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, two_kernel=True)
    o_pick, s_pick, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, segments=runs)
    torch.cuda.synchronize()
    assert torch.equal(o_one, o_two) and torch.equal(s_one, s_two), "the two sequential modes differ"
    assert torch.equal(o, o_pick) and torch.equal(sf, s_pick), "the library's pick differs from its mode"
    del o_two, s_two, o_pick, s_pick, dev
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
    if runs > 1:  # the sequential result too
        assert _err(o_one[:1].cpu().double().numpy(), ro, f"{name} O, one-kernel mode, oracle on the GPU's A") <= TOL
        assert _err(s_one[:1].cpu().double().numpy(), rs, f"{name} state, one-kernel mode, oracle on the GPU's A") <= TOL
    del o_one, s_one
    ro, rs = oracle.gdn_chunked(qb, kb, vb, gb, bb, A_ref, w.scale, s0b)
    assert _err(og, ro, f"{name} O, all {T} tokens of batch 0, oracle on its own A") <= 2 * TOL
    assert _err(sg, rs, f"{name} state after {(T + 63) // 64} chunks, oracle on its own A") <= 2 * TOL


# B, T, Hqk, Hv, DV, dtype, init_state, (gate_lo, gate_span), run counts asked for
SEG_CASES = [
    (1, 1000, 2, 4, 128, torch.bfloat16, True, (0.999, 0.001), [2, 3, 16]),   # 16 chunks, one per run
    (1, 200, 2, 4, 128, torch.bfloat16, True, (0.9, 0.1), [2, 4, 9]),         # ragged last chunk; 9 > chunks
    (2, 700, 1, 3, 64, torch.float16, False, (0.99, 0.01), [3, 5]),           # runs of 4 and 3 chunks
    (1, 64 * 40 + 17, 4, 4, 128, torch.bfloat16, True, (1.0, 0.0), [7, 41]),  # no decay at all
]


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: "x".join(str(x) for x in c[:5]) +
                         str(c[5]).split(".")[-1] + f"-s0{int(c[6])}-a{c[7][0]}")
def test_gdn_segmented_matches_oracle(case):
    B, T, Hqk, Hv, DV, dtype, init, (lo, span), runs = case
    w = GdnWorkload("seg", B, T, Hqk, Hv, 128, DV, dtype, T + Hv, init_state=init, gate_lo=lo, gate_span=span)
    q, k, v, g, beta, s0 = make_gdn_inputs(w)
    dev = [t.cuda() if t is not None else None for t in (q, k, v, g, beta, s0)]
    o1, s1, A = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, two_kernel=False)
    torch.cuda.synchronize()
    A_np = A.cpu().double().numpy() * _valid_cols(T)[None, :, None, :]
    ro, rs = oracle.gdn_chunked(q, k, v, g, beta, A_np, w.scale, s0)
    to, ts = oracle.gdn_recurrent(q, k, v, g, beta, w.scale, s0)
    for P in runs:
        o, sf, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, segments=P)
        o2, s2, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, segments=P)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(sf, s2), "not deterministic"
        assert torch.isfinite(o.float()).all() and torch.isfinite(sf).all()
        og, sg = o.cpu().double().numpy(), sf.cpu().double().numpy()
        print(f"segments={P}: max|O - one-kernel O| {float((o.float() - o1.float()).abs().max()):.3e}", flush=True)
        assert _err(og, ro, f"segments={P} O vs chunked oracle") <= TOL
        assert _err(sg, rs, f"segments={P} state vs chunked oracle") <= TOL
        assert _err(og, to, f"segments={P} O vs token recurrence") <= 2 * TOL
        assert _err(sg, ts, f"segments={P} state vs token recurrence") <= 2 * TOL


def test_gdn_segmented_single_run_is_one_kernel():
    """Asked for one run, or for runs on a one-chunk sequence, the segmented entry point runs the
    one-kernel mode: the same bits, and no workspace needed."""
    for T, P in ((300, 1), (64, 4), (10, 2)):
        w, (q, k, v, g, beta, s0) = _case(1, T, 2, 4, 128, torch.bfloat16, True, seed=T)
        dev = [t.cuda() for t in (q, k, v, g, beta, s0)]
        o1, s1, A = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, two_kernel=False)
        assert fa.gdn_segmented_workspace_size(1, T, 4, 128, P) == 0
        o2, s2, _ = fa.gdn_prefill(*dev[:5], s0=dev[5], scale=w.scale, A=A, segments=P)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2), (T, P)
