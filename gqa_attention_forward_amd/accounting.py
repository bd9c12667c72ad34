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


# ------------------------------------------------------------ Gated DeltaNet chunked prefill

def gdn_flops(B: int, T: int, Hv: int, DK: int, DV: int, chunk: int = 64) -> float:
    """Algorithmic flops of the chunk recurrence, per value head and chunk of n tokens (2 flops
    per multiply-add): U' = K S (n DK DV), Q S (n DK DV), the scores Q K^T (n n DK),
    V_new = A W' (n n DV), scores V_new (n n DV), the state update K^T V_new (DK n DV)."""
    total = 0.0
    for c0 in range(0, T, chunk):
        n = min(chunk, T - c0)
        total += 2.0 * (3 * n * DK * DV + n * n * DK + 2 * n * n * DV)
    return total * B * Hv


def gdn_bytes(B: int, T: int, Hqk: int, Hv: int, DK: int, DV: int, init_state: bool, chunk: int = 64,
              elem: int = 2) -> int:
    """Compulsory HBM bytes of one chunk-recurrence call: q, k, v, A read once, g and beta (fp32)
    read once, the initial state read (if any) and the final state written (fp32), o written."""
    qk = 2 * B * T * Hqk * DK * elem
    vo = 2 * B * T * Hv * DV * elem
    a = B * T * Hv * chunk * elem
    gb = 2 * B * T * Hv * 4
    st = B * Hv * DK * DV * 4 * (2 if init_state else 1)
    return qk + vo + a + gb + st
