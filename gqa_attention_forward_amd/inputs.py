"""Seeded synthetic inputs for the attention forward workloads.

This module holds no attention arithmetic: it only draws the Q/K/V tensors that
both the HIP path and the fp64 oracle consume, so that the two see identical bits.

Recipe (identical for every workload):
  * a CPU ``torch.Generator`` seeded with the workload's seed;
  * draw order q, k, v, each i.i.d. N(0, 1) in fp32, then rounded to the input
    dtype (round-to-nearest-even, torch's ``.to``);
  * for the "peaky" workload, a Bernoulli(rate) draw per (b, kv-head, key) row
    *after* v, and the selected K rows multiplied by ``peak_factor`` (8: exact in
    fp16/bf16, it only shifts the exponent);
  * contiguous layout: q, o [B, Hq, M, D]; k, v [B, Hkv, N, D].
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    M: int
    N: int
    D: int
    dtype: torch.dtype
    causal: bool
    seed: int
    peak_rate: float = 0.0     # fraction of K rows scaled by peak_factor
    peak_factor: float = 8.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def groups(self) -> int:
        return self.Hq // self.Hkv


# The five workloads: tiny causal GQA, the pages' benchmark shape, non-causal MHA,
# long causal GQA prefill with peaky keys, chunked-prefill with M != N.
WORKLOADS = {
    "tiny_causal_gqa": Workload("tiny_causal_gqa", 1, 2, 1, 128, 128, 64, torch.float16, True, 0),
    "pages_causal_gqa_1k": Workload("pages_causal_gqa_1k", 2, 16, 8, 1024, 1024, 128, torch.float16, True, 1),
    "mha_noncausal_4k": Workload("mha_noncausal_4k", 8, 32, 32, 4096, 4096, 128, torch.bfloat16, False, 2),
    "long_causal_gqa_16k": Workload("long_causal_gqa_16k", 1, 32, 8, 16384, 16384, 128, torch.bfloat16, True, 3,
                                    peak_rate=0.01),
    "chunked_prefill_512x8k": Workload("chunked_prefill_512x8k", 4, 32, 4, 512, 8192, 128, torch.float16, True, 4),
}
WORKLOAD_ORDER = list(WORKLOADS)

# Small-grid shapes for the key-split forward: decode (one query row per head against an
# 8k-key cache) and a short 64-row query chunk, both GQA with 4 query heads per KV head.
SMALL_GRID_WORKLOADS = {
    "decode_gqa_8k": Workload("decode_gqa_8k", 8, 32, 8, 1, 8192, 128, torch.bfloat16, True, 5),
    "short_query_gqa_8k": Workload("short_query_gqa_8k", 4, 32, 8, 64, 8192, 128, torch.float16, True, 6),
}
ALL_WORKLOADS = {**WORKLOADS, **SMALL_GRID_WORKLOADS}


def make_inputs(w: Workload, device: str | torch.device = "cpu"):
    """Returns (q, k, v, n_peaky_rows). The draw always happens on the CPU generator."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.M, w.D), generator=g, dtype=torch.float32).to(w.dtype)
    k = torch.randn((w.B, w.Hkv, w.N, w.D), generator=g, dtype=torch.float32).to(w.dtype)
    v = torch.randn((w.B, w.Hkv, w.N, w.D), generator=g, dtype=torch.float32).to(w.dtype)
    n_peaky = 0
    if w.peak_rate > 0:
        rows = torch.rand((w.B, w.Hkv, w.N), generator=g) < w.peak_rate
        n_peaky = int(rows.sum())
        k = torch.where(rows[..., None], k * w.peak_factor, k)
    if str(device) != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v, n_peaky


def make_custom(B, Hq, Hkv, M, N, D, dtype, seed, *, peak_rate=0.0, device="cpu"):
    """Inputs for an arbitrary shape with the same recipe (parity tests, ragged cases)."""
    w = Workload("custom", B, Hq, Hkv, M, N, D, dtype, False, seed, peak_rate=peak_rate)
    return make_inputs(w, device)[:3]


# ------------------------------------------------------------ Gated DeltaNet prefill inputs

@dataclasses.dataclass(frozen=True)
class GdnWorkload:
    """Chunked Gated DeltaNet prefill: q, k [B,T,Hqk,DK]; v [B,T,Hv,DV]; per value head and token
    the gate's cumulative log inside each 64-token chunk (g) and beta; optional fp32 initial
    state [B,Hv,DK,DV]."""
    name: str
    B: int
    T: int
    Hqk: int
    Hv: int
    DK: int
    DV: int
    dtype: torch.dtype
    seed: int
    init_state: bool = False
    chunk: int = 64
    gate_lo: float = 0.9     # per-token gate a ~ U(gate_lo, gate_lo + gate_span)
    gate_span: float = 0.1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.DK)


GDN_WORKLOADS = {
    # long sequence, few state slices (value heads share query/key heads in pairs)
    "gdn_long_gva_32k": GdnWorkload("gdn_long_gva_32k", 1, 32768, 8, 16, 128, 128, torch.bfloat16, 7),
    # wide: many state slices, with an initial state
    "gdn_wide_state_4k": GdnWorkload("gdn_wide_state_4k", 8, 4096, 16, 32, 128, 128, torch.bfloat16, 8,
                                     init_state=True),
}


def make_gdn_inputs(w: GdnWorkload, device: str | torch.device = "cpu", *, B=None, T=None):
    """Returns (q, k, v, g, beta, s0). Recipe, CPU generator seeded with w.seed, draw order:
    q, k, v ~ N(0, 1) in fp32; q and k rows scaled to unit L2 norm (the usual normalised
    delta-rule keys), then rounded to the dtype; per (token, value head) a gate
    a ~ U(gate_lo, gate_lo + gate_span) (U(0.9, 1) by default) whose log is summed inside each
    chunk (g, fp32); beta ~ U(0, 1) (fp32); the initial state
    ~ N(0, 0.1^2) (fp32) when the workload has one, else None.  B and T may be overridden for
    smaller parity cases with the same recipe."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    gen = torch.Generator(device="cpu").manual_seed(w.seed)
    q = torch.randn((B, T, w.Hqk, w.DK), generator=gen)
    k = torch.randn((B, T, w.Hqk, w.DK), generator=gen)
    v = torch.randn((B, T, w.Hv, w.DV), generator=gen)
    q = (q / q.norm(dim=-1, keepdim=True)).to(w.dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(w.dtype)
    v = v.to(w.dtype)
    a = w.gate_lo + w.gate_span * torch.rand((B, T, w.Hv), generator=gen)
    la = torch.log(a)
    pad = (-T) % w.chunk
    la = torch.nn.functional.pad(la, (0, 0, 0, pad)).reshape(B, (T + pad) // w.chunk, w.chunk, w.Hv)
    g = la.cumsum(dim=2).reshape(B, T + pad, w.Hv)[:, :T].contiguous().float()
    beta = torch.rand((B, T, w.Hv), generator=gen).float()
    s0 = (0.1 * torch.randn((B, w.Hv, w.DK, w.DV), generator=gen)).float() if w.init_state else None
    if str(device) != "cpu":
        q, k, v, g, beta = (t.to(device) for t in (q, k, v, g, beta))
        s0 = s0.to(device) if s0 is not None else None
    return q, k, v, g, beta, s0
