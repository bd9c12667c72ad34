"""MI355X (gfx950) fused attention forward: a thin Python binding over libfa.so.

Every step of the computation runs in the HIP kernels of ``csrc/fa_fwd.hip`` (forward and
key-split forward), ``csrc/fa_bwd.hip`` (backward) and ``csrc/gdn_fwd.hip`` (Gated DeltaNet
chunked prefill); this module only marshals arguments through the C ABI declared in
``include/fa.h`` and ``include/gdn.h``.  There is no fallback: if ``libfa.so`` is missing or
cannot be loaded, every call raises.

Functions with the C ABI's names take raw device pointers and sizes:

    fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, M, N, D, scale, causal, dtype, stream)
    fa_fwd_strided(q_ptr, ..., D, q_strides, k_strides, v_strides, o_strides, scale, causal, dtype, stream)
    fa_fwd_splitkv(..., dtype, tiles_per_split, workspace_ptr, workspace_bytes, stream)
    fa_fwd_splitkv_noalloc(..., dtype, tiles_per_split, stream)
    fa_fwd_splitkv_strided(..., D, q_strides, ..., o_strides, scale, ..., workspace_bytes, stream)
    fa_splitkv_plan(B, Hq, Hkv, M, N, D, causal, tiles_per_split)
    fa_strerror(code), fa_tile_shape(B, Hq, M, D), fa_tile_counts(...), fa_schedule(...)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, M, N, D, scale, causal, dtype, ws, ws_bytes, stream)
    fa_bwd_workspace_size(B, Hq, M)
    gdn_kkt(k, g, beta, A, B, T, Hqk, Hv, DK, dtype, stream)
    gdn_chunk_fwd(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DK, DV, scale, dtype, ws, ws_bytes, stream)
    gdn_chunk_workspace_size(B, T, Hv, DV), gdn_chunk_plan(B, T, Hv, DV)
    gdn_chunk_fwd_segmented(q, k, ..., scale, dtype, segments, ws, ws_bytes, stream)
    gdn_segmented_workspace_size(B, T, Hv, DV, segments), gdn_segment_plan(B, T, Hv, DV)

``attention_forward``, ``attention_backward`` and ``gdn_prefill`` are the torch-tensor
convenience wrappers (torch is used only for device memory, workspaces and the current stream).
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_F16, FA_BF16 = 0, 1
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH, FA_ERR_SCRATCH_TOO_SMALL = 0, -1, -2, -3, -4
FA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/fa.h: scratch of fa_fwd_splitkv_noalloc, per GPU

_lib = None


class fa_strides(ctypes.Structure):
    """Element strides of the batch, head and row axes of a [B, H, S, D] tensor (D has unit stride)."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


class FaError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {fa_strerror(code)} (code {code})")
        self.code = code


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m gqa_attention_forward_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci, cf, cll = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp]
    lib.fa_fwd.restype = ci
    lib.fa_strerror.argtypes = [ci]
    lib.fa_strerror.restype = ctypes.c_char_p
    ip, llp = ctypes.POINTER(ci), ctypes.POINTER(cll)
    lib.fa_tile_shape.argtypes = [ci, ci, ci, ci, ip, ip]
    lib.fa_tile_shape.restype = ci
    lib.fa_tile_counts.argtypes = [ci, ci, ci, ci, ci, llp, llp, llp]
    lib.fa_tile_counts.restype = ci
    lib.fa_schedule.argtypes = [ci, ci, ci, ci, ci, ci, cll, ip, ip, ip]
    lib.fa_schedule.restype = ci
    sz = ctypes.c_size_t
    lib.fa_splitkv_plan.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ip, llp, ctypes.POINTER(sz)]
    lib.fa_splitkv_plan.restype = ci
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, ci, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = ci
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, ci, vp]
    lib.fa_fwd_splitkv_noalloc.restype = ci
    sp = ctypes.POINTER(fa_strides)
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, sp, sp, sp, sp, cf, ci, ci, vp]
    lib.fa_fwd_strided.restype = ci
    lib.fa_fwd_splitkv_strided.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, sp, sp, sp, sp, cf, ci, ci, ci,
                                           vp, sz, vp]
    lib.fa_fwd_splitkv_strided.restype = ci
    lib.fa_bwd_workspace_size.argtypes = [ci, ci, ci]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp, sz, vp]
    lib.fa_bwd.restype = ci
    fp = ctypes.POINTER(ctypes.c_float)
    lib.gdn_kkt.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, vp]
    lib.gdn_kkt.restype = ci
    lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp, sz, vp]
    lib.gdn_chunk_fwd.restype = ci
    lib.gdn_chunk_workspace_size.argtypes = [ci, ci, ci, ci]
    lib.gdn_chunk_workspace_size.restype = sz
    lib.gdn_chunk_plan.argtypes = [ci, ci, ci, ci, ctypes.POINTER(sz)]
    lib.gdn_chunk_plan.restype = ci
    lib.gdn_chunk_fwd_segmented.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp,
                                            sz, vp]
    lib.gdn_chunk_fwd_segmented.restype = ci
    lib.gdn_segmented_workspace_size.argtypes = [ci, ci, ci, ci, ci]
    lib.gdn_segmented_workspace_size.restype = sz
    lib.gdn_segment_plan.argtypes = [ci, ci, ci, ci, ctypes.POINTER(ci)]
    lib.gdn_segment_plan.restype = ci
    _lib = lib
    return lib


def library():
    """The loaded ctypes handle of libfa.so (raises if it is not built)."""
    return _load()


# ------------------------------------------------------------- C ABI, by name

def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, M, N, D, scale, causal, dtype, stream) -> int:
    """Raw C ABI call: pointers are integers (device addresses), stream an int or None."""
    return _load().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, M, N, D, float(scale), int(causal), int(dtype), stream)


def _st(x):
    """None -> NULL; a (batch, head, row) triple or fa_strides -> pointer to fa_strides."""
    if x is None:
        return None
    if not isinstance(x, fa_strides):
        x = fa_strides(*[int(v) for v in x])
    return ctypes.pointer(x)


def fa_fwd_strided(q, k, v, o, lse, B, Hq, Hkv, M, N, D, q_strides, k_strides, v_strides, o_strides, scale, causal,
                   dtype, stream) -> int:
    """Raw C ABI call with element strides (batch, head, row) per tensor, None for contiguous."""
    return _load().fa_fwd_strided(q, k, v, o, lse, B, Hq, Hkv, M, N, D, _st(q_strides), _st(k_strides),
                                  _st(v_strides), _st(o_strides), float(scale), int(causal), int(dtype), stream)


def fa_fwd_splitkv_strided(q, k, v, o, lse, B, Hq, Hkv, M, N, D, q_strides, k_strides, v_strides, o_strides, scale,
                           causal, dtype, tiles_per_split, workspace, workspace_bytes, stream) -> int:
    """Raw C ABI call of the strided key-split forward."""
    return _load().fa_fwd_splitkv_strided(q, k, v, o, lse, B, Hq, Hkv, M, N, D, _st(q_strides), _st(k_strides),
                                          _st(v_strides), _st(o_strides), float(scale), int(causal), int(dtype),
                                          int(tiles_per_split), workspace, int(workspace_bytes), stream)


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, M, N, D, scale, causal, dtype, tiles_per_split, workspace,
                   workspace_bytes, stream) -> int:
    """Raw C ABI call of the key-split forward (pointers as integers)."""
    return _load().fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, M, N, D, float(scale), int(causal), int(dtype),
                                  int(tiles_per_split), workspace, int(workspace_bytes), stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, M, N, D, scale, causal, dtype, tiles_per_split,
                           stream) -> int:
    """Raw C ABI call of the key-split forward that allocates nothing (its partial results go to
    the library's per-GPU scratch of FA_NOALLOC_SCRATCH_BYTES bytes)."""
    return _load().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, M, N, D, float(scale), int(causal), int(dtype),
                                          int(tiles_per_split), stream)


def fa_splitkv_plan(B: int, Hq: int, Hkv: int, M: int, N: int, D: int, causal: bool, tiles_per_split: int = 0):
    """(tiles_used, workgroups, workspace_bytes) of the key-split forward for this problem."""
    t, wg, ws = ctypes.c_int(), ctypes.c_longlong(), ctypes.c_size_t()
    rc = _load().fa_splitkv_plan(B, Hq, Hkv, M, N, D, int(bool(causal)), int(tiles_per_split), ctypes.byref(t),
                                 ctypes.byref(wg), ctypes.byref(ws))
    if rc != FA_OK:
        raise FaError(rc, "fa_splitkv_plan")
    return t.value, wg.value, ws.value


def fa_bwd_workspace_size(B: int, Hq: int, M: int) -> int:
    return int(_load().fa_bwd_workspace_size(B, Hq, M))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, M, N, D, scale, causal, dtype, workspace, workspace_bytes,
           stream) -> int:
    """Raw C ABI call of the backward pass (pointers as integers)."""
    return _load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, M, N, D, float(scale), int(causal),
                          int(dtype), workspace, int(workspace_bytes), stream)


def gdn_kkt(k, g, beta, A, B, T, Hqk, Hv, DK, dtype, stream) -> int:
    """Raw C ABI call (include/gdn.h): A = (I + L)^-1 per 64-token chunk."""
    return _load().gdn_kkt(k, g, beta, A, B, T, Hqk, Hv, DK, int(dtype), stream)


def gdn_chunk_fwd(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DK, DV, scale, dtype, workspace,
                  workspace_bytes, stream) -> int:
    """Raw C ABI call (include/gdn.h): the Gated DeltaNet chunk recurrence (workspace None: the
    one-kernel mode; else the state walk plus the parallel output kernel)."""
    return _load().gdn_chunk_fwd(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DK, DV, float(scale), int(dtype),
                                 workspace, int(workspace_bytes), stream)


def gdn_chunk_fwd_segmented(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DK, DV, scale, dtype, segments,
                            workspace, workspace_bytes, stream) -> int:
    """Raw C ABI call (include/gdn.h): the chunk recurrence with the chunks split into runs walked
    in parallel (transition walks, start-state combine, output walks)."""
    return _load().gdn_chunk_fwd_segmented(q, k, v, g, beta, A, s0, o, s_final, B, T, Hqk, Hv, DK, DV, float(scale),
                                           int(dtype), int(segments), workspace, int(workspace_bytes), stream)


def gdn_segmented_workspace_size(B: int, T: int, Hv: int, DV: int, segments: int) -> int:
    """Bytes of the gdn_chunk_fwd_segmented workspace (0 when the chunks form a single run)."""
    return int(_load().gdn_segmented_workspace_size(B, T, Hv, DV, segments))


def gdn_segment_plan(B: int, T: int, Hv: int, DV: int) -> int:
    """Runs of chunks the library picks for the segmented mode (1: it picks a sequential mode)."""
    n = ctypes.c_int()
    rc = _load().gdn_segment_plan(B, T, Hv, DV, ctypes.byref(n))
    if rc != FA_OK:
        raise FaError(rc, "gdn_segment_plan")
    return int(n.value)


def gdn_chunk_workspace_size(B: int, T: int, Hv: int, DV: int) -> int:
    """Bytes of the gdn_chunk_fwd workspace of the two-kernel mode."""
    return int(_load().gdn_chunk_workspace_size(B, T, Hv, DV))


def gdn_chunk_plan(B: int, T: int, Hv: int, DV: int) -> int:
    """Workspace bytes of the mode the library picks for this shape (0: the one-kernel mode)."""
    ws = ctypes.c_size_t()
    rc = _load().gdn_chunk_plan(B, T, Hv, DV, ctypes.byref(ws))
    if rc != FA_OK:
        raise FaError(rc, "gdn_chunk_plan")
    return int(ws.value)


def fa_strerror(code: int) -> str:
    return _load().fa_strerror(int(code)).decode()


def fa_tile_shape(B: int, Hq: int, M: int, D: int):
    """(BM, BN): query-tile and key-tile heights fa_fwd uses for this problem."""
    bm, bn = ctypes.c_int(), ctypes.c_int()
    rc = _load().fa_tile_shape(B, Hq, M, D, ctypes.byref(bm), ctypes.byref(bn))
    if rc != FA_OK:
        raise FaError(rc, "fa_tile_shape")
    return bm.value, bn.value


def fa_tile_counts(M: int, N: int, BM: int, BN: int, causal: bool):
    """(full, masked, skipped) key tiles of one (b, h)."""
    f, m, s = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_longlong()
    rc = _load().fa_tile_counts(M, N, BM, BN, int(bool(causal)), ctypes.byref(f), ctypes.byref(m), ctypes.byref(s))
    if rc != FA_OK:
        raise FaError(rc, "fa_tile_counts")
    return f.value, m.value, s.value


def fa_schedule(B: int, Hq: int, Hkv: int, M: int, D: int, causal: bool, wg: int):
    """(b, h, q_tile) computed by workgroup `wg` of fa_fwd's grid."""
    b, h, qt = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = _load().fa_schedule(B, Hq, Hkv, M, D, int(bool(causal)), int(wg), ctypes.byref(b), ctypes.byref(h),
                             ctypes.byref(qt))
    if rc != FA_OK:
        raise FaError(rc, "fa_schedule")
    return b.value, h.value, qt.value


# ------------------------------------------------------- torch convenience API

def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def forward_launcher(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, stream=None,
                     split_kv="auto"):
    """Checks and plans one forward the way attention_forward does (same arguments, same
    dispatch) and returns (launch, out, lse): launch() enqueues that forward again with no
    further checks or allocation (the key-split workspace, if any, is allocated here once and
    kept by the closure).  For loops that run the same shapes many times; the tensors must stay
    alive and keep their shapes."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, S, D]")
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have unit stride along D")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, M, D = q.shape
    Bk, Hkv, N, Dk = k.shape
    if tuple(v.shape) != (Bk, Hkv, N, Dk) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)  # preserves q's layout when q is a permuted dense tensor
    if out.stride(3) != 1 or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype, with unit stride along D")
    if lse is None:
        lse = torch.empty((B, Hq, M), dtype=torch.float32, device=q.device)
    if not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, M) or lse.dtype != torch.float32:
        raise ValueError("lse must be a contiguous float32 [B, Hq, M] tensor")
    strided = not all(t.is_contiguous() for t in (q, k, v, out))
    sts = [tuple(t.stride()[:3]) if strided else None for t in (q, k, v, out)]
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lib = _load()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    dt = _dtype_code(q)
    if split_kv is not False:
        tiles = 0 if split_kv == "auto" else int(split_kv)
        if tiles < 0:
            raise ValueError("split_kv must be 'auto', False or a positive tile count")
        M_ok = M <= 128 * 128  # the split plan describes at most 128 query tiles per head
        if M_ok and D in (64, 128):
            _, _, ws_bytes = fa_splitkv_plan(B, Hq, Hkv, M, N, D, causal, tiles)
            if ws_bytes > 0 or split_kv != "auto" or (M < 128 and Hq > Hkv):
                ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
                args = (*ptrs, B, Hq, Hkv, M, N, D, *[_st(x) for x in sts], float(scale), int(causal), dt,
                        tiles, ws.data_ptr(), ws_bytes, stream)

                def launch_split(_ws=ws):  # the closure keeps the workspace alive
                    rc = lib.fa_fwd_splitkv_strided(*args)
                    if rc != FA_OK:
                        raise FaError(rc, "fa_fwd_splitkv")

                return launch_split, out, lse
        elif split_kv != "auto":
            raise ValueError("the key-split forward needs D in (64, 128) and M <= 16384")
    args = (*ptrs, B, Hq, Hkv, M, N, D, *[_st(x) for x in sts], float(scale), int(causal), dt, stream)

    def launch():
        rc = lib.fa_fwd_strided(*args)
        if rc != FA_OK:
            raise FaError(rc, "fa_fwd")

    return launch, out, lse


def attention_forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, stream=None,
                      split_kv="auto"):
    """O, lse = softmax(mask(q k^T * scale)) v for device tensors q [B,Hq,M,D], k/v [B,Hkv,N,D]
    (fp16 or bf16) with unit stride along D and any other strides that keep rows 16-byte aligned
    (e.g. [B,S,H,D] buffers passed as .transpose(1, 2) views).  Returns (o [B,Hq,M,D], lse
    [B,Hq,M] fp32); a new `o` takes q's memory layout.

    split_kv: "auto" runs the key-split forward when its plan splits some query tile (small
    grids) or when M < 128 with grouped KV heads (the key-split kernel then stacks the query
    heads of a group into one tile's rows), and fa_fwd otherwise; False always runs fa_fwd;
    an int > 0 runs the key-split forward with at most that many key tiles per share.  The
    split workspace comes from torch's caching allocator.  Kernels are enqueued on `stream`
    (default: torch's current stream) and not waited for."""
    launch, out, lse = forward_launcher(q, k, v, causal, scale, out, lse, stream, split_kv)
    launch()
    return out, lse


def _expect_all(specs):
    """Checks tensor arguments against the sizes and element type the C ABI will be told.
    specs: (name, tensor, shape, dtype) tuples; the first tensor's device is the reference.  All
    shapes, then dtypes and contiguity, are checked before any device check (a tensor smaller
    than the sizes passed would send the kernels past its allocation), then that every tensor is
    a device tensor on the first one's device."""
    for name, t, shape, dtype in specs:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    for name, t, shape, dtype in specs:
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    device = specs[0][1].device
    for name, t, shape, dtype in specs:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def attention_backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, stream=None):
    """dq, dk, dv for contiguous device tensors: q, dout, o [B,Hq,M,D], k, v [B,Hkv,N,D] (fp16/bf16)
    and lse [B,Hq,M] fp32 from attention_forward on the same inputs.  The workspace comes from
    torch's caching allocator; kernels are enqueued on `stream` (default: the current stream)."""
    import torch

    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D: q [B, Hq, M, D], k [B, Hkv, N, D]")
    B, Hq, M, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    _dtype_code(q)  # fp16 or bf16
    _expect_all([("q", q, (B, Hq, M, D), q.dtype), ("k", k, (B, Hkv, N, D), q.dtype),
                 ("v", v, (B, Hkv, N, D), q.dtype), ("o", o, (B, Hq, M, D), q.dtype),
                 ("dout", dout, (B, Hq, M, D), q.dtype), ("lse", lse, (B, Hq, M), torch.float32)])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa_bwd_workspace_size(B, Hq, M)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, M, N, D, scale, causal, _dtype_code(q), ws.data_ptr(),
                ws_bytes, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv


def gdn_prefill(q, k, v, g, beta, s0=None, scale: float | None = None, A=None, stream=None, two_kernel="auto",
                segments: int | None = None):
    """Gated DeltaNet chunked prefill on contiguous device tensors: q, k [B,T,Hqk,128], v [B,T,Hv,DV]
    (fp16/bf16), g and beta [B,T,Hv] fp32 (g: cumulative log-gate inside each 64-token chunk),
    s0 [B,Hv,128,DV] fp32 or None.  A [B,T,Hv,64] (dtype) is computed with gdn_kkt when not given.
    two_kernel: True for the state walk plus the parallel output kernel (workspace from torch's
    caching allocator), False for the one-kernel mode -- these two give the same bits -- and
    "auto" for the library's pick: the segmented mode when gdn_segment_plan picks more than one
    run, else gdn_chunk_plan's mode.  segments: an int >= 1 runs the segmented mode
    (gdn_chunk_fwd_segmented) with that many runs of chunks (1 gives the one-kernel bits).
    Returns (o [B,T,Hv,DV], final state [B,Hv,128,DV] fp32, A)."""
    import torch

    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be 4-D: q [B, T, Hqk, 128], v [B, T, Hv, DV]")
    B, T, Hqk, DK = q.shape
    Hv, DV = v.shape[2], v.shape[3]
    _dtype_code(q)  # fp16 or bf16
    specs = [("q", q, (B, T, Hqk, DK), q.dtype), ("k", k, (B, T, Hqk, DK), q.dtype), ("v", v, (B, T, Hv, DV), q.dtype),
             ("g", g, (B, T, Hv), torch.float32), ("beta", beta, (B, T, Hv), torch.float32)]
    if s0 is not None:
        specs.append(("s0", s0, (B, Hv, DK, DV), torch.float32))
    if A is not None:
        specs.append(("A", A, (B, T, Hv, 64), q.dtype))
    _expect_all(specs)
    if scale is None:
        scale = 1.0 / math.sqrt(DK)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    dt = _dtype_code(q)
    if A is None:
        A = torch.empty((B, T, Hv, 64), dtype=q.dtype, device=q.device)
        rc = gdn_kkt(k.data_ptr(), g.data_ptr(), beta.data_ptr(), A.data_ptr(), B, T, Hqk, Hv, DK, dt, stream)
        if rc != FA_OK:
            raise FaError(rc, "gdn_kkt")
    o = torch.empty((B, T, Hv, DV), dtype=q.dtype, device=q.device)
    sf = torch.empty((B, Hv, DK, DV), dtype=torch.float32, device=q.device)
    ws, ws_bytes = None, 0
    if segments is None and two_kernel == "auto":
        planned = gdn_segment_plan(B, T, Hv, DV)
        segments = planned if planned > 1 else None
    if segments is not None:
        ws_bytes = gdn_segmented_workspace_size(B, T, Hv, DV, segments)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
        rc = gdn_chunk_fwd_segmented(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                     A.data_ptr(), s0.data_ptr() if s0 is not None else None, o.data_ptr(),
                                     sf.data_ptr(), B, T, Hqk, Hv, DK, DV, scale, dt, segments,
                                     ws.data_ptr() if ws is not None else None, ws_bytes, stream)
        if rc != FA_OK:
            raise FaError(rc, "gdn_chunk_fwd_segmented")
        return o, sf, A
    if two_kernel == "auto":
        ws_bytes = gdn_chunk_plan(B, T, Hv, DV)
    elif two_kernel:
        ws_bytes = gdn_chunk_workspace_size(B, T, Hv, DV)
    if ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    rc = gdn_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), A.data_ptr(),
                       s0.data_ptr() if s0 is not None else None, o.data_ptr(), sf.data_ptr(), B, T, Hqk, Hv, DK, DV,
                       scale, dt, ws.data_ptr() if ws is not None else None, ws_bytes, stream)
    if rc != FA_OK:
        raise FaError(rc, "gdn_chunk_fwd")
    return o, sf, A


__all__ = ["gdn_kkt", "gdn_chunk_fwd", "gdn_chunk_workspace_size", "gdn_chunk_plan", "gdn_prefill",
           "gdn_chunk_fwd_segmented", "gdn_segmented_workspace_size", "gdn_segment_plan",
           "fa_bwd", "fa_bwd_workspace_size", "attention_backward", "fa_fwd", "fa_fwd_strided",
           "fa_fwd_splitkv", "fa_fwd_splitkv_strided", "fa_fwd_splitkv_noalloc", "FA_NOALLOC_SCRATCH_BYTES", "fa_splitkv_plan", "fa_strides",
           "fa_strerror", "fa_tile_shape", "fa_tile_counts", "fa_schedule", "attention_forward", "forward_launcher",
           "library", "FaError", "FA_F16", "FA_BF16", "LIB_PATH"]
