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
