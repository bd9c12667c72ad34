"""Parity of the HIP kernels (through the C ABI) against the fp64 CPU oracle, element by element.

Tolerances: max-abs error of O <= 4e-3 (fp16) / 1.6e-2 (bf16); logsumexp within 1e-3.
Rows that see no key must give O = 0 exactly and lse = -inf.
"""
import math

import numpy as np
import pytest
import torch

import gqa_attention_forward_amd as fa
import oracle
from gqa_attention_forward_amd.inputs import WORKLOADS, make_custom, make_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
LSE_TOL = 1e-3


def _run_gpu(q, k, v, causal, scale):
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.attention_forward(dq, dk, dv, causal=causal, scale=scale, split_kv=False)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what):
    o_gpu = o_gpu.double().numpy()
    lse_gpu = lse_gpu.double().numpy()
    fin = np.isfinite(lse_ref)
    err = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    lerr = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    print(f"{what}: max|dO| = {err:.3e} (tol {TOL[dtype]:.1e}), max|dlse| = {lerr:.3e}", flush=True)
    assert np.all(np.isfinite(o_gpu)), what
    assert err <= TOL[dtype], what
    assert lerr <= LSE_TOL, what
    # rows without a visible key
    assert np.all(np.isneginf(lse_gpu[~fin])), what
    assert np.all(o_gpu[~fin] == 0.0), what


SMALL = [
    # B, Hq, Hkv, M, N, D, causal, dtype        (several tiles, ragged tails, M != N both ways)
    (1, 2, 1, 128, 128, 64, True, torch.float16),
    (2, 4, 2, 300, 300, 128, True, torch.bfloat16),
    (1, 8, 2, 77, 300, 128, True, torch.float16),
    (1, 4, 1, 300, 77, 128, True, torch.bfloat16),      # first 223 rows see no key
    (2, 2, 2, 200, 333, 128, False, torch.float16),
    (1, 4, 4, 129, 65, 64, False, torch.bfloat16),
    (1, 6, 3, 256, 1000, 64, True, torch.bfloat16),
    (3, 2, 1, 1, 1, 128, True, torch.float16),           # one query, one key
    (1, 2, 1, 1, 500, 128, True, torch.float16),         # decode-like: one query row
    (1, 2, 2, 64, 64, 128, False, torch.bfloat16),       # a single half-filled query tile
    # grids large enough for the 8-wave (256-row) workgroups, ragged in M and N
    (8, 32, 8, 300, 333, 128, True, torch.bfloat16),
    (4, 64, 64, 260, 130, 64, False, torch.float16),
    (2, 128, 16, 513, 700, 128, True, torch.float16),
    (1, 256, 32, 256, 64, 64, True, torch.bfloat16),      # exactly one key tile per row
    (2, 64, 16, 700, 1111, 128, False, torch.bfloat16),   # non-causal, 18 key tiles, ragged last
    (1, 128, 16, 1000, 1999, 128, True, torch.float16),   # 32 key tiles, bottom-right mask, ragged
    # more ragged small grids
    (5, 20, 4, 300, 400, 128, True, torch.float16),
    (1, 4, 2, 200, 200, 128, True, torch.bfloat16),
    (1, 2, 2, 100, 333, 64, False, torch.float16),
    (1, 2, 1, 64, 130, 128, False, torch.bfloat16),
    (1, 3, 1, 400, 100, 128, True, torch.float16),       # M > N: whole query tiles with no key
    # small grids with 16+ key tiles: 8-wave workgroups whose two key groups split the tiles,
    # with even and odd tile counts, ragged N, masked rows (M > N) and a single query row
    (1, 2, 1, 128, 1024, 128, True, torch.float16),
    (1, 4, 2, 300, 1023, 128, True, torch.bfloat16),
    (2, 2, 2, 200, 1030, 64, False, torch.float16),      # 17 tiles: the second group pads one
    (1, 2, 1, 1200, 1000, 128, True, torch.bfloat16),    # first 200 rows see no key
    (1, 4, 1, 77, 2049, 128, True, torch.float16),
    (1, 8, 8, 1, 1500, 64, True, torch.bfloat16),
    (3, 5, 5, 129, 1300, 128, False, torch.float16),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(str(x) for x in s[:7]) + str(s[7]).split(".")[-1])
def test_small_shapes_full_compare(shape):
    B, Hq, Hkv, M, N, D, causal, dtype = shape
    q, k, v = make_custom(B, Hq, Hkv, M, N, D, dtype, seed=M * 7 + N)
    scale = 1.0 / math.sqrt(D)
    o, lse = _run_gpu(q, k, v, causal, scale)
    ro, rlse = oracle.attn_fwd(q, k, v, scale, causal)
    _check(o, lse, ro, rlse, dtype, f"shape {shape}")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_peaky_keys_small(dtype):
    """Peaky logits (10% of K rows x8) exercise the running-max rescale."""
    q, k, v = make_custom(1, 4, 1, 512, 512, 128, dtype, seed=99, peak_rate=0.1)
    scale = 1.0 / math.sqrt(128)
    o, lse = _run_gpu(q, k, v, True, scale)
    ro, rlse = oracle.attn_fwd(q, k, v, scale, True)
    _check(o, lse, ro, rlse, dtype, "peaky")


def _kv_group_slices(w):
    """(b, kv head) slices: the g query heads of one KV group with their K/V head.  Every
    element of O and lse belongs to exactly one slice."""
    g = w.Hq // w.Hkv
    for b in range(w.B):
        for hk in range(w.Hkv):
            yield b, hk, slice(hk * g, (hk + 1) * g)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name):
    """Every workload at its full size, in the launch configuration the benchmark times, compared
    with the oracle on every element of O and lse.  The oracle runs one (b, kv head) group at a
    time (the group's query heads against its K/V head) to bound host memory; the groups cover
    the whole output."""
    w = WORKLOADS[name]
    q, k, v, n_peaky = make_inputs(w)
    print(f"{name}: {w}, peaky rows {n_peaky}", flush=True)
    o, lse = _run_gpu(q, k, v, w.causal, w.scale)
    assert torch.isfinite(o.float()).all()
    err = lerr = 0.0
    rows = 0
    for b, hk, hs in _kv_group_slices(w):
        qs = q[b:b + 1, hs].contiguous()
        ks, vs = k[b:b + 1, hk:hk + 1].contiguous(), v[b:b + 1, hk:hk + 1].contiguous()
        ro, rlse = oracle.attn_fwd(qs, ks, vs, w.scale, w.causal)
        og = o[b:b + 1, hs].double().numpy()
        lg = lse[b:b + 1, hs].double().numpy()
        fin = np.isfinite(rlse)
        assert np.all(np.isfinite(og)), (name, b, hk)
        err = max(err, float(np.abs(og - ro).max()))
        if fin.any():
            lerr = max(lerr, float(np.abs(lg[fin] - rlse[fin]).max()))
        assert np.all(np.isneginf(lg[~fin])) and np.all(og[~fin] == 0.0), (name, b, hk)
        rows += rlse.size
    assert rows == w.B * w.Hq * w.M
    print(f"{name}: all {rows} rows x {w.D} columns compared: max|dO| = {err:.3e} (tol {TOL[w.dtype]:.1e}), "
          f"max|dlse| = {lerr:.3e} (tol {LSE_TOL:.0e})", flush=True)
    assert err <= TOL[w.dtype], name
    assert lerr <= LSE_TOL, name
