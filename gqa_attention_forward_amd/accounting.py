"""Work and traffic accounting for the attention forward (measurement only).

* visible pairs: the (query, key) pairs the mask keeps, counted exactly per (b, h);
* causal-adjusted flops: 4*D per visible pair (2*D for the score dot product, 2*D for
  the weighted sum of V);
* compulsory bytes: Q, K, V read once and O, LSE written once.
"""
from __future__ import annotations


def visible_pairs_per_head(M: int, N: int, causal: bool) -> int:
    """Row i sees keys j <= i + (N - M) (bottom-right causal) or all N keys."""
    if not causal:
        return M * N
    off = N - M
    return sum(min(N, max(0, i + 1 + off)) for i in range(M))


def causal_adjusted_flops(B, Hq, M, N, D, causal) -> int:
    return 4 * B * Hq * D * visible_pairs_per_head(M, N, causal)


def compulsory_bytes(B, Hq, Hkv, M, N, D, elem_bytes=2) -> int:
    q = B * Hq * M * D * elem_bytes
    kv = 2 * B * Hkv * N * D * elem_bytes
    return 2 * q + kv + B * Hq * M * 4


def workload_flops(w) -> int:
    return causal_adjusted_flops(w.B, w.Hq, w.M, w.N, w.D, w.causal)


def workload_bytes(w) -> int:
    return compulsory_bytes(w.B, w.Hq, w.Hkv, w.M, w.N, w.D)
