"""fp64 CPU oracle for the fused attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path
(``gqa_attention_forward_amd``) never imports, loads or calls it, and it never
imports the product path: the two share nothing but the seeded input generator.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, libm); this module only
marshals 16-bit input patterns in and fp64 results out through ctypes.  The C file's
header states what is computed and which page passages each mode follows:

* ``attn_fwd``            -- the definition of masked softmax attention (page
  "从零开始写Qwen3", FlashAttention derivation article, sections "简易情况-三矩阵相乘"
  and "FlashAttention"), with grouped KV heads ``hk = h // (Hq // Hkv)``, causal mask
  ``j <= i + (N - M)`` and ``lse = m + ln l``;
* ``attn_fwd_rows``       -- the same definition on a chosen list of rows;
* ``attn_fwd_blockwise``  -- the page's FlashAttention-2 loop (running max, running
  denominator, rescaled accumulator, one division after the loop), in fp64;
* ``attn_fwd_stepnorm``   -- the page's per-step-normalised online-softmax recurrence
  (section "在线softmax"), in fp64;
* ``attn_probs``          -- the softmax weight matrix of one (b, h);
* ``attn_bwd``            -- gradients of O with respect to q, k, v for an upstream dO,
  the chain rule of the definition written out (not on the pages; see the C file);
* ``attn_bwd_slice``      -- the same gradients for one (b, kv head) group: dk and dv of a key
  range and dq of chosen rows, parallel enough to check full-size problems;
* ``gdn_chunked``, ``gdn_recurrent``, ``gdn_kkt`` -- the Gated DeltaNet chunked prefill of the
  page "lab3：GDN Prefill 前向优化" (section "算法与数据依赖"), the token recurrence it rewrites,
  and its A = (I + L)^-1 (``gdn_oracle.c``).

Every function is pinned by the ``-m "not gpu"`` tests against closed forms, page
worked numbers, invariants and an independent library routine.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16 = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        ci, cd, cl = ctypes.c_int, ctypes.c_double, ctypes.c_long
        shape = [ci, ci, ci, ci, ci, ci, ci, cd, ci]  # dtype,B,Hq,Hkv,M,N,D,scale,causal
        lib.oracle_attn_fwd.argtypes = [u16p, u16p, u16p] + shape + [dp, dp]
        lib.oracle_attn_fwd_rows.argtypes = [u16p, u16p, u16p] + shape + [i64p, ctypes.c_int64, dp, dp]
        lib.oracle_attn_fwd_blockwise.argtypes = [u16p, u16p, u16p] + shape + [cl, dp, dp]
        lib.oracle_attn_fwd_stepnorm.argtypes = [u16p, u16p, u16p] + shape + [cl, dp, dp]
        lib.oracle_attn_probs.argtypes = [u16p, u16p] + shape + [ci, ci, dp]
        lib.oracle_attn_bwd.argtypes = [u16p, u16p, u16p, u16p] + shape + [dp, dp, dp]
        lib.oracle_set_threads.argtypes = [ci]
        lib.oracle_set_threads.restype = ci
        lib.oracle_attn_bwd.restype = ci
        lib.oracle_attn_bwd_slice.argtypes = [u16p, u16p, u16p, u16p] + shape + [ci, ci, cl, cl, i64p, ctypes.c_int64,
                                                                             dp, dp, dp]
        lib.oracle_attn_bwd_slice.restype = ci
        gshape = [ci, ci, ci, ci, ci, ci, ci, cd]  # B, T, Hqk, Hv, DK, DV, C, scale
        lib.oracle_gdn_recurrent.argtypes = [u16p, u16p, u16p, ci, dp, dp, dp] + gshape + [dp, dp]
        lib.oracle_gdn_chunked.argtypes = [u16p, u16p, u16p, ci, dp, dp, dp, dp] + gshape + [dp, dp]
        lib.oracle_gdn_kkt.argtypes = [u16p, ci, dp, dp, ci, ci, ci, ci, ci, ci, dp]
        for f in (lib.oracle_gdn_recurrent, lib.oracle_gdn_chunked, lib.oracle_gdn_kkt):
            f.restype = ci
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_f16.restype = cd
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = cd
        for f in (lib.oracle_attn_fwd, lib.oracle_attn_fwd_rows, lib.oracle_attn_fwd_blockwise,
                  lib.oracle_attn_fwd_stepnorm, lib.oracle_attn_probs):
            f.restype = ci
        _lib = lib
    return _lib


def _bits(x) -> np.ndarray:
    """Raw 16-bit patterns of an fp16/bf16 torch tensor (on the CPU) or a uint16 array."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch

    assert x.dtype in (torch.float16, torch.bfloat16), x.dtype
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _dtype_code(x) -> int:
    import torch

    if isinstance(x, np.ndarray):
        raise TypeError("pass dtype explicitly for raw uint16 arrays")
    return F16 if x.dtype == torch.float16 else BF16


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


def _shape(q, k, dtype):
    B, Hq, M, D = q.shape
    Bk, Hkv, N, Dk = k.shape
    assert B == Bk and D == Dk
    return B, Hq, Hkv, M, N, D


def _common(q, k, v, dtype):
    if dtype is None:
        dtype = _dtype_code(q)
    B, Hq, Hkv, M, N, D = _shape(q, k, dtype)
    return dtype, (B, Hq, Hkv, M, N, D), _bits(q), _bits(k), _bits(v)


def attn_fwd(q, k, v, scale: float, causal: bool, dtype: int | None = None):
    """Full forward. Returns (O [B,Hq,M,D] fp64, lse [B,Hq,M] fp64) as numpy arrays."""
    dtype, (B, Hq, Hkv, M, N, D), qb, kb, vb = _common(q, k, v, dtype)
    o = np.empty((B, Hq, M, D), np.float64)
    lse = np.empty((B, Hq, M), np.float64)
    rc = _load().oracle_attn_fwd(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16), _ptr(vb, ctypes.c_uint16),
                                 dtype, B, Hq, Hkv, M, N, D, float(scale), int(bool(causal)),
                                 _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_attn_fwd rejected its arguments")
    return o, lse


def attn_fwd_rows(q, k, v, scale: float, causal: bool, rows, dtype: int | None = None):
    """Rows given as flat indices (b*Hq + h)*M + i. Returns (O [n,D], lse [n]) fp64."""
    dtype, (B, Hq, Hkv, M, N, D), qb, kb, vb = _common(q, k, v, dtype)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if rows.size and (rows.min() < 0 or rows.max() >= B * Hq * M):
        raise ValueError("row index out of range")
    o = np.empty((rows.size, D), np.float64)
    lse = np.empty((rows.size,), np.float64)
    rc = _load().oracle_attn_fwd_rows(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                      _ptr(vb, ctypes.c_uint16), dtype, B, Hq, Hkv, M, N, D, float(scale),
                                      int(bool(causal)), _ptr(rows, ctypes.c_int64), rows.size,
                                      _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_attn_fwd_rows rejected its arguments")
    return o, lse


def _online(fn_name, q, k, v, scale, causal, block, dtype):
    dtype, (B, Hq, Hkv, M, N, D), qb, kb, vb = _common(q, k, v, dtype)
    o = np.empty((B, Hq, M, D), np.float64)
    lse = np.empty((B, Hq, M), np.float64)
    rc = getattr(_load(), fn_name)(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16), _ptr(vb, ctypes.c_uint16),
                                   dtype, B, Hq, Hkv, M, N, D, float(scale), int(bool(causal)), int(block),
                                   _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"{fn_name} rejected its arguments")
    return o, lse


def attn_fwd_blockwise(q, k, v, scale: float, causal: bool, block: int, dtype: int | None = None):
    """The FlashAttention-2 loop in fp64 over blocks of `block` keys (deferred normalisation)."""
    return _online("oracle_attn_fwd_blockwise", q, k, v, scale, causal, block, dtype)


def attn_fwd_stepnorm(q, k, v, scale: float, causal: bool, block: int, dtype: int | None = None):
    """The per-step-normalised online-softmax recurrence in fp64 over blocks of `block` keys."""
    return _online("oracle_attn_fwd_stepnorm", q, k, v, scale, causal, block, dtype)


def attn_probs(q, k, scale: float, causal: bool, b: int, h: int, dtype: int | None = None):
    """Softmax weights P [M, N] fp64 of one (b, h)."""
    if dtype is None:
        dtype = _dtype_code(q)
    B, Hq, M, D = q.shape
    _, Hkv, N, _ = k.shape
    qb, kb = _bits(q), _bits(k)
    P = np.empty((M, N), np.float64)
    rc = _load().oracle_attn_probs(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16), dtype, B, Hq, Hkv, M, N,
                                   D, float(scale), int(bool(causal)), int(b), int(h), _ptr(P, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_attn_probs rejected its arguments")
    return P


def attn_bwd(q, k, v, do, scale: float, causal: bool, dtype: int | None = None):
    """Gradients (dq [B,Hq,M,D], dk [B,Hkv,N,D], dv [B,Hkv,N,D]) fp64 of O for upstream dO."""
    dtype, (B, Hq, Hkv, M, N, D), qb, kb, vb = _common(q, k, v, dtype)
    dob = _bits(do)
    assert dob.shape == qb.shape
    dq = np.empty((B, Hq, M, D), np.float64)
    dk = np.empty((B, Hkv, N, D), np.float64)
    dv = np.empty((B, Hkv, N, D), np.float64)
    rc = _load().oracle_attn_bwd(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16), _ptr(vb, ctypes.c_uint16),
                                 _ptr(dob, ctypes.c_uint16), dtype, B, Hq, Hkv, M, N, D, float(scale),
                                 int(bool(causal)), _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                                 _ptr(dv, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_attn_bwd rejected its arguments")
    return dq, dk, dv


def attn_bwd_slice(q, k, v, do, scale: float, causal: bool, b: int, hk: int, key_range, rows,
                   dtype: int | None = None):
    """Gradients for one (b, kv head) group only: (dq of `rows` [n, D], dk and dv of the keys
    key_range = (j0, j1) [j1 - j0, D]) fp64; rows are indices (h - hk*g)*M + i of the group."""
    dtype, (B, Hq, Hkv, M, N, D), qb, kb, vb = _common(q, k, v, dtype)
    dob = _bits(do)
    assert dob.shape == qb.shape
    j0, j1 = (int(x) for x in key_range)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    dq = np.empty((rows.size, D), np.float64)
    dk = np.empty((max(j1 - j0, 0), D), np.float64)
    dv = np.empty((max(j1 - j0, 0), D), np.float64)
    rc = _load().oracle_attn_bwd_slice(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16),
                                       _ptr(vb, ctypes.c_uint16), _ptr(dob, ctypes.c_uint16), dtype, B, Hq, Hkv, M,
                                       N, D, float(scale), int(bool(causal)), int(b), int(hk), j0, j1,
                                       _ptr(rows, ctypes.c_int64), rows.size, _ptr(dq, ctypes.c_double),
                                       _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_attn_bwd_slice rejected its arguments")
    return dq, dk, dv


def _f64(x):
    if x is None:
        return None
    import torch

    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _dp(a):
    return None if a is None else _ptr(a, ctypes.c_double)


def _gdn_shape(q, v):
    B, T, Hqk, DK = q.shape
    _, _, Hv, DV = v.shape
    return B, T, Hqk, Hv, DK, DV


def gdn_recurrent(q, k, v, g, beta, scale: float, s0=None, chunk: int = 64, dtype: int | None = None):
    """Token-by-token gated delta rule. q, k [B,T,Hqk,DK]; v [B,T,Hv,DV] (fp16/bf16); g (cumulative
    log-gate inside each chunk of `chunk` tokens) and beta [B,T,Hv]; s0 [B,Hv,DK,DV] or None.
    Returns (o [B,T,Hv,DV], final state [B,Hv,DK,DV]) fp64."""
    if dtype is None:
        dtype = _dtype_code(q)
    B, T, Hqk, Hv, DK, DV = _gdn_shape(q, v)
    gb, bb, sb = _f64(g), _f64(beta), _f64(s0)
    o = np.empty((B, T, Hv, DV), np.float64)
    sf = np.empty((B, Hv, DK, DV), np.float64)
    rc = _load().oracle_gdn_recurrent(_ptr(_bits(q), ctypes.c_uint16), _ptr(_bits(k), ctypes.c_uint16),
                                      _ptr(_bits(v), ctypes.c_uint16), dtype, _dp(gb), _dp(bb), _dp(sb), B, T, Hqk,
                                      Hv, DK, DV, int(chunk), float(scale), _dp(o), _dp(sf))
    if rc != 0:
        raise ValueError("oracle_gdn_recurrent rejected its arguments")
    return o, sf


def gdn_chunked(q, k, v, g, beta, A, scale: float, s0=None, chunk: int = 64, dtype: int | None = None):
    """The page's chunk recurrence with A [B,T,Hv,chunk] given (fp64 or a tensor). Same returns."""
    if dtype is None:
        dtype = _dtype_code(q)
    B, T, Hqk, Hv, DK, DV = _gdn_shape(q, v)
    gb, bb, ab, sb = _f64(g), _f64(beta), _f64(A), _f64(s0)
    o = np.empty((B, T, Hv, DV), np.float64)
    sf = np.empty((B, Hv, DK, DV), np.float64)
    rc = _load().oracle_gdn_chunked(_ptr(_bits(q), ctypes.c_uint16), _ptr(_bits(k), ctypes.c_uint16),
                                    _ptr(_bits(v), ctypes.c_uint16), dtype, _dp(gb), _dp(bb), _dp(ab), _dp(sb), B, T,
                                    Hqk, Hv, DK, DV, int(chunk), float(scale), _dp(o), _dp(sf))
    if rc != 0:
        raise ValueError("oracle_gdn_chunked rejected its arguments")
    return o, sf


def gdn_kkt(k, g, beta, Hv: int, chunk: int = 64, dtype: int | None = None):
    """A [B,T,Hv,chunk] fp64: per chunk (I + L)^-1, L_ts = beta_t (k_t . k_s) exp(g_t - g_s), s < t."""
    if dtype is None:
        dtype = _dtype_code(k)
    B, T, Hqk, DK = k.shape
    gb, bb = _f64(g), _f64(beta)
    A = np.empty((B, T, Hv, chunk), np.float64)
    rc = _load().oracle_gdn_kkt(_ptr(_bits(k), ctypes.c_uint16), dtype, _dp(gb), _dp(bb), B, T, Hqk, Hv, DK,
                                int(chunk), _dp(A))
    if rc != 0:
        raise ValueError("oracle_gdn_kkt rejected its arguments")
    return A


def decode(bits: int, dtype: int) -> float:
    """Decode one 16-bit pattern with the oracle's own decoder."""
    lib = _load()
    return lib.oracle_decode_f16(bits) if dtype == F16 else lib.oracle_decode_bf16(bits)


def decode_array(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Vectorised over a numpy uint16 array (one ctypes call per element; for tests only)."""
    lib = _load()
    f = lib.oracle_decode_f16 if dtype == F16 else lib.oracle_decode_bf16
    return np.array([f(int(b)) for b in bits.ravel()], dtype=np.float64).reshape(bits.shape)


_threads_override = None


def set_threads(n: int) -> int:
    """Threads for later oracle calls; returns the previous count (for restoring it)."""
    global _threads_override
    prev = threads_used()
    lib = _load()
    lib.oracle_set_threads(int(n))
    _threads_override = int(n)
    return prev


def threads_used() -> int:
    """OpenMP threads the oracle will use (set_threads, else OMP_NUM_THREADS or the process's
    CPU affinity)."""
    if _threads_override is not None:
        return _threads_override
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
