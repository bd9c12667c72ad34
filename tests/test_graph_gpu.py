"""HIP-graph capture of the entry points.

A call into the library only enqueues kernels on the given stream: no allocation, memset or
synchronisation happens inside it, so a call can be captured into a graph.  Each test captures
one call of a torch-level wrapper (its output and workspace tensors come from the graph's
memory pool) into a torch CUDA graph -- a HIP graph on ROCm -- then replays it several times,
with eager work of the program in between (the outputs are overwritten with NaN, an eager call
of the same wrapper runs), and checks every replay against an eager call bit for bit: the
kernels are deterministic, so captured and eager launches must agree exactly.
"""
import math

import pytest
import torch

import gqa_attention_forward_amd as fa
from gqa_attention_forward_amd.inputs import GdnWorkload, make_custom, make_gdn_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture_and_replay(fn, what):
    ref = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as torch's capture expects
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            same = torch.equal(a, b) or (a.dtype.is_floating_point and torch.equal(torch.nan_to_num(a, nan=1.5),
                                                                                   torch.nan_to_num(b, nan=1.5)))
            print(f"{what}: replay {rep} output {i} {'identical' if same else 'DIFFERS'}", flush=True)
            assert same, f"{what}: replay {rep}, output {i}"
        eager = fn()  # the program's own work between replays
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(eager, ref)), what


FWD_CASES = {  # split_kv, shape (B, Hq, Hkv, M, N, D)
    "plain": (False, (1, 8, 2, 300, 700, 128)),
    "plain_key_groups": (False, (1, 8, 2, 300, 1100, 128)),  # 17 key tiles on a small grid
    "split": ("auto", (4, 16, 4, 1, 4096, 128)),
}


@pytest.mark.parametrize("case", list(FWD_CASES))
def test_forward_capture(case):
    split_kv, (B, Hq, Hkv, M, N, D) = FWD_CASES[case]
    q, k, v = (t.cuda() for t in make_custom(B, Hq, Hkv, M, N, D, torch.bfloat16, seed=71))
    scale = 1 / math.sqrt(D)

    def fn():
        return fa.attention_forward(q, k, v, causal=True, scale=scale, split_kv=split_kv)

    if split_kv == "auto":
        _, _, ws = fa.fa_splitkv_plan(B, Hq, Hkv, M, N, D, True)
        assert ws > 0, "this shape should take the key-split path"
    _capture_and_replay(fn, f"forward split_kv={split_kv}")


def test_backward_capture():
    B, Hq, Hkv, M, N, D = 1, 4, 2, 200, 300, 64
    q, k, v = (t.cuda() for t in make_custom(B, Hq, Hkv, M, N, D, torch.float16, seed=72))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(73)).to(q.dtype).cuda()
    o, lse = fa.attention_forward(q, k, v, causal=True, split_kv=False)

    def fn():
        return fa.attention_backward(q, k, v, o, lse, do, causal=True)

    _capture_and_replay(fn, "backward")


def test_gdn_capture():
    w = GdnWorkload("graph", 1, 200, 2, 4, 128, 128, torch.bfloat16, 74, init_state=True)
    q, k, v, g, beta, s0 = make_gdn_inputs(w, device="cuda")

    def fn():
        return fa.gdn_prefill(q, k, v, g, beta, s0=s0, scale=w.scale)

    _capture_and_replay(fn, "gdn prefill")


def test_gdn_segmented_capture():
    # 16 chunks in 4 runs: transition walks, the start-state combine and the output walks replayed
    w = GdnWorkload("graph", 1, 1000, 2, 4, 128, 128, torch.bfloat16, 75, init_state=True, gate_lo=0.999,
                    gate_span=0.001)
    q, k, v, g, beta, s0 = make_gdn_inputs(w, device="cuda")
    assert fa.gdn_segmented_workspace_size(1, 1000, 4, 128, 4) > 0

    def fn():
        return fa.gdn_prefill(q, k, v, g, beta, s0=s0, scale=w.scale, segments=4)

    _capture_and_replay(fn, "gdn prefill, segmented")
