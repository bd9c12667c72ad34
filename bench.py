#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

One step is one fa_fwd call over the whole workload (inputs resident in HBM).  The default
workload is the long causal GQA prefill (B=1, Hq=32, Hkv=8, M=N=16384, D=128, bf16, 1% of
K rows scaled by 8).  Prints ONE JSON line on stdout:

  value     causal-adjusted TFLOPS = 4*D*(visible query/key pairs)*B*Hq / (wall time per step)
  roofline  the kernel's average duration from HIP events recorded around every timed launch
            on the launch stream, against the dense bf16/fp16 MFMA peak (2500 TFLOP/s); plus
            HBM traffic per launch from the committed rocprofv3 counter summary, or null when
            the kernel source changed since the counters were taken
  cpu_baseline  the fp64 CPU oracle timed on a bounded random sample of the same workload's
            rows, in the same unit

``--all`` also prints one line per workload to stderr (not part of the contract); for the two
small, cache-resident workloads the line adds a cold-cache median (a 512 MiB buffer is
overwritten between calls) and the oracle's rate on one core.  Those lines warm the GPU for a
quarter second after their --warmup calls (the clock ramps up after each idle spell while the
next inputs are drawn on the host); the benchmark line takes exactly --warmup untimed steps.
``--calibrate-copy BYTES`` runs only a plain device-to-device copy of BYTES bytes (used to
scale the FETCH_SIZE / WRITE_SIZE counters of the profiles).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
KERNEL_SRCS = [os.path.join(ROOT, "gqa_attention_forward_amd", "csrc", f)
               for f in ("fa_fwd.hip", "fa_device.h", "fa_tiles.h", "fa_mfma_run.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_kernel_long_causal_gqa_16k_traffic.md")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_causal_gqa_16k")
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="time the forward, or the backward (dq, dk, dv from a forward's O and lse)")
    ap.add_argument("--layout", choices=["bhsd", "bshd"], default="bhsd",
                    help="memory layout of q, k, v, o: contiguous [B,H,S,D] or [B,S,H,D] buffers (strided path)")
    ap.add_argument("--gdn-mode", choices=["auto", "one", "two", "seg"], default="auto",
                    help="Gated DeltaNet workloads: the library's pick, the one-kernel, the two-kernel or the "
                         "segmented mode")
    ap.add_argument("--gdn-segments", type=int, default=0,
                    help="runs of chunks for --gdn-mode seg (0: the library's plan)")
    ap.add_argument("--split-kv", default="auto",
                    help="'auto' (key-split forward for small grids), 'off', or key tiles per share")
    return ap.parse_args()


def source_digest() -> str:
    """First 16 hex digits of the SHA-256 of the forward kernel's sources (fa_fwd.hip, then the
    headers it includes from csrc/, in that order)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch recorded in the committed counter summary, if it matches the
    current kernel source."""
    if workload != "long_causal_gqa_16k" or not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def roofline(w, flops, avg_ms, traffic):
    """The bound that applies to the workload: MFMA when its arithmetic intensity (causal-adjusted
    flops per compulsory HBM byte) exceeds the machine balance, HBM otherwise (decode-like shapes)."""
    from gqa_attention_forward_amd import accounting

    nbytes = accounting.workload_bytes(w)
    if flops / nbytes >= MFMA_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        achieved, peak, bound, unit = flops / (avg_ms * 1e-3) / 1e12, MFMA_PEAK_TFLOPS, "mfma", "TFLOP/s"
    else:
        achieved, peak, bound, unit = nbytes / (avg_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "hbm", "GB/s"
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel_avg_us": round(avg_ms * 1e3, 3)}


def step_stats(durs):
    """Per-launch kernel times (ms, in launch order): median, min and mean, and the means of the
    first and last five launches, so that a clock still ramping up during the timed steps shows."""
    srt = sorted(durs)
    n5 = min(5, len(durs))
    return {"median": round(srt[len(srt) // 2], 4), "min": round(srt[0], 4),
            "mean": round(sum(durs) / len(durs), 4),
            "mean_first5": round(sum(durs[:n5]) / n5, 4), "mean_last5": round(sum(durs[-n5:]) / n5, 4)}


# workloads whose inputs fit in the 256 MB last-level cache (the small parity shapes)
SMALL_CACHE_RESIDENT = ("tiny_causal_gqa", "pages_causal_gqa_1k")


def warm_until(call, min_seconds):
    """Keeps calling until min_seconds of GPU work have passed (the engine clock ramps up over
    tens of milliseconds after an idle spell, e.g. while the next workload's inputs are drawn on
    the host).  Used for the informational per-workload lines only; the benchmark line itself
    takes exactly --warmup untimed steps."""
    import torch

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(8):
            call()
        torch.cuda.synchronize()


def time_gpu(fa, w, q, k, v, steps, warmup, split_kv="auto", min_warm_s=0.0):
    import torch

    stream = torch.cuda.current_stream()
    # the arguments are checked and the launch planned once; each step then only enqueues it, so
    # the host keeps ahead of short kernels and the events bracket the kernels alone
    launch, o, lse = fa.forward_launcher(q, k, v, causal=w.causal, scale=w.scale, split_kv=split_kv)
    for _ in range(warmup):
        launch()
    warm_until(launch, min_warm_s)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = [s.elapsed_time(e) for s, e in zip(starts, ends)]  # ms, in launch order
    return wall, durs, o, lse


def time_gpu_cold(fa, w, q, k, v, steps, split_kv="auto", flush_bytes=512 << 20):
    """Per-call kernel times (ms, sorted) with the on-package caches flushed before every call:
    a 512 MiB buffer is overwritten between calls, outside the timed events."""
    import torch

    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.M), dtype=torch.float32, device=q.device)
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    fa.attention_forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, split_kv=split_kv)
    for i in range(steps):
        scratch.fill_(i % 251 + 1)
        starts[i].record(stream)
        fa.attention_forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, split_kv=split_kv)
        ends[i].record(stream)
    torch.cuda.synchronize()
    del scratch
    return sorted(s_.elapsed_time(e) for s_, e in zip(starts, ends))


def oracle_one_thread(w, q, k, v, target_s=3.0):
    """The oracle on one thread over a row sample of about target_s seconds (all rows when
    they fit): the single-core reference point for the small workloads."""
    import numpy as np

    import oracle

    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    total_rows = w.B * w.Hq * w.M
    vis = (lambda i: np.clip(i + 1 + (w.N - w.M), 0, w.N)) if w.causal else (lambda i: np.full(i.shape, w.N))
    prev = oracle.set_threads(1)
    try:
        rng = np.random.default_rng(4321)
        n = min(total_rows, 256)
        for attempt in range(3):
            rows = np.sort(rng.choice(total_rows, size=n, replace=False)).astype(np.int64)
            t0 = time.perf_counter()
            oracle.attn_fwd_rows(qc, kc, vc, w.scale, w.causal, rows)
            dt = time.perf_counter() - t0
            if n == total_rows or dt >= 0.5 * target_s or attempt == 2:
                break
            n = int(min(total_rows, n * target_s / max(dt, 1e-3)))
    finally:
        oracle.set_threads(prev)
    fl = float(4 * w.D * vis(rows % w.M).sum())
    return {"value": fl / dt / 1e12, "unit": "TFLOPS", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {total_rows} query rows, {fl / 1e9:.3f} GFLOP in {dt:.2f} s, fp64"}


def time_gpu_bwd(fa, w, q, k, v, steps, warmup, min_warm_s=0.0):
    """Backward calls on fixed q, k, v, dO and the forward's O and lse (per-call HIP events)."""
    import torch

    g = torch.Generator(device="cpu").manual_seed(w.seed + 1000)
    do = torch.randn(q.shape, generator=g).to(w.dtype).to(q.device)
    q, k, v = (t.contiguous() for t in (q, k, v))
    o, lse = fa.attention_forward(q, k, v, causal=w.causal, scale=w.scale, split_kv=False)
    for _ in range(warmup):
        fa.attention_backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    warm_until(lambda: fa.attention_backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale), min_warm_s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        grads = fa.attention_backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]  # ms, in launch order
    return wall, durs, grads[0], lse


def run_gdn(args, fa, w):
    """Gated DeltaNet chunked prefill: A comes from gdn_kkt before the timed region (the page's
    framework computes it outside its timing too); the timed call is gdn_chunk_fwd."""
    import torch

    from gqa_attention_forward_amd import accounting
    from gqa_attention_forward_amd.inputs import make_gdn_inputs

    q, k, v, g, beta, s0 = make_gdn_inputs(w, device="cuda")
    _, _, A = fa.gdn_prefill(q, k, v, g, beta, s0=s0, scale=w.scale)
    B, T, Hqk, DK = q.shape
    Hv, DV = v.shape[2], v.shape[3]
    o = torch.empty((B, T, Hv, DV), dtype=q.dtype, device="cuda")
    sf = torch.empty((B, Hv, DK, DV), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    dt = 0 if q.dtype == torch.float16 else 1
    segments = 1
    if args.gdn_mode == "auto":
        segments = fa.gdn_segment_plan(B, T, Hv, DV)
    elif args.gdn_mode == "seg":
        segments = args.gdn_segments or max(2, fa.gdn_segment_plan(B, T, Hv, DV))
    if segments > 1:
        ws_bytes = fa.gdn_segmented_workspace_size(B, T, Hv, DV, segments)
    else:
        ws_bytes = {"auto": lambda: fa.gdn_chunk_plan(B, T, Hv, DV), "one": lambda: 0,
                    "two": lambda: fa.gdn_chunk_workspace_size(B, T, Hv, DV)}[args.gdn_mode]()
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def call():
        common = (q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), A.data_ptr(),
                  s0.data_ptr() if s0 is not None else None, o.data_ptr(), sf.data_ptr(), B, T, Hqk, Hv, DK, DV,
                  w.scale, dt)
        if segments > 1:
            rc = fa.gdn_chunk_fwd_segmented(*common, segments, ws.data_ptr() if ws_bytes else None, ws_bytes,
                                            stream.cuda_stream)
        else:
            rc = fa.gdn_chunk_fwd(*common, ws.data_ptr() if ws_bytes else None, ws_bytes, stream.cuda_stream)
        assert rc == 0, rc

    for _ in range(args.warmup):
        call()
    warm_until(call, 0.0 if w.name == args.workload else 0.25)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    avg_ms = sum(durs) / len(durs)
    flops = accounting.gdn_flops(B, T, Hv, DK, DV)
    nbytes = accounting.gdn_bytes(B, T, Hqk, Hv, DK, DV, s0 is not None)
    assert torch.isfinite(sf).all().item(), "non-finite state"
    if segments > 1:
        path = f"gdn_chunk_fwd_segmented ({segments} runs: transition walks, combine, output walks)"
    else:
        path = "gdn_chunk_fwd (state walk + parallel outputs)" if ws_bytes else "gdn_chunk_fwd (one kernel)"
    line = {"workload": w.name, "path": path, "ms": round(avg_ms, 4),
            "median_ms": round(durs[len(durs) // 2], 4), "tflops": round(flops / (avg_ms * 1e-3) / 1e12, 2),
            "compulsory_gbs": round(nbytes / (avg_ms * 1e-3) / 1e9, 1),
            "state_walkers": B * Hv * (DV // 64), "runs": segments}
    print(json.dumps(line), file=sys.stderr, flush=True)
    achieved = flops / (avg_ms * 1e-3) / 1e12
    return {
        "metric": "Gated DeltaNet chunked prefill ms per call and TFLOPS (algorithmic chunk products)",
        "value": round(flops * args.steps / wall / 1e12, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "Hqk": Hqk, "Hv": Hv, "DK": DK, "DV": DV,
                   "init_state": s0 is not None, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel_avg_us": round(avg_ms * 1e3, 3)},
        "cpu_baseline": None,
    }


# parity bar of the timed output against the oracle's rows: max-abs error of O, and of lse
O_TOL = {"f16": 4e-3, "bf16": 1.6e-2}
LSE_TOL = 1e-3


def cpu_baseline(w, q, k, v, target_s, o=None, lse=None):
    """Times the oracle (as it stands) on a random sample of rows of the workload.  When the timed
    GPU output (o, lse) is given, the same rows of it are compared with the oracle's: the errors go
    into the report, and a result outside the parity bar ends the benchmark with an error."""
    import numpy as np

    import oracle
    from gqa_attention_forward_amd import accounting

    total_rows = w.B * w.Hq * w.M
    rng = np.random.default_rng(1234)

    def flops_of(rows):
        i = rows % w.M
        if w.causal:
            vis = np.clip(i + 1 + (w.N - w.M), 0, w.N)
        else:
            vis = np.full(rows.shape, w.N)
        return float(4 * w.D * vis.sum())

    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    # each oracle call decodes the whole inputs first (a fixed cost); time two probe sizes,
    # fit time = fixed + flops / rate, then size the timed sample to about target_s seconds
    times = []
    for n_probe in (64, 512):
        probe = rng.integers(0, total_rows, size=n_probe).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attn_fwd_rows(qc, kc, vc, w.scale, w.causal, probe)
        times.append((flops_of(probe), time.perf_counter() - t0))
    (f1, t1), (f2, t2) = times
    per_flop = max((t2 - t1) / max(f2 - f1, 1.0), 1e-15)
    fixed = max(t1 - f1 * per_flop, 0.0)
    avg_row = accounting.causal_adjusted_flops(1, 1, w.M, w.N, w.D, w.causal) / w.M
    n = int(min(total_rows, max(256, (target_s - fixed) / per_flop / avg_row)))
    # the probes run below full thread efficiency, so a first sample can come out short: one
    # resize from its own measured rate
    for attempt in range(2):
        rows = np.sort(rng.choice(total_rows, size=n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        ro, rlse = oracle.attn_fwd_rows(qc, kc, vc, w.scale, w.causal, rows)
        dt = time.perf_counter() - t0
        fl = flops_of(rows)
        if dt >= 0.6 * target_s or n == total_rows or attempt == 1:
            break
        n = int(min(total_rows, n * target_s / max(dt, 1e-3)))
    out = {
        "value": fl / dt / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.threads_used(),
        "kind": "oracle",
        "sample": (f"all {total_rows} query rows" if n == total_rows else f"{n} random query rows (of {total_rows})")
                  + f" of {w.name}, all their visible keys; {fl / 1e9:.1f} GFLOP causal-adjusted in {dt:.1f} s, fp64",
    }
    if o is not None:
        import torch

        idx = torch.from_numpy(rows)
        og = o.reshape(-1, w.D)[idx.to(o.device)].double().cpu().numpy()
        lg = lse.reshape(-1)[idx.to(lse.device)].double().cpu().numpy()
        fin = np.isfinite(rlse)
        err_o = float(np.abs(og - ro).max())
        err_l = float(np.abs(lg[fin] - rlse[fin]).max()) if fin.any() else 0.0
        tol = O_TOL["bf16" if w.dtype == torch.bfloat16 else "f16"]
        ok = (np.isfinite(og).all() and err_o <= tol and err_l <= LSE_TOL and np.all(np.isneginf(lg[~fin]))
              and np.all(og[~fin] == 0.0))
        out["check"] = {"rows": int(rows.size), "max_abs_err_o": err_o, "tol_o": tol, "max_abs_err_lse": err_l,
                        "tol_lse": LSE_TOL, "ok": bool(ok)}
    return out


def calibrate_copy(nbytes: int):
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}))


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward of this library runs on a single "
              "device (no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch

    import gqa_attention_forward_amd as fa
    from gqa_attention_forward_amd import accounting
    from gqa_attention_forward_amd.inputs import ALL_WORKLOADS as WORKLOADS, make_inputs

    if not os.path.exists(fa.LIB_PATH):
        from gqa_attention_forward_amd import build as hip_build

        hip_build.build()

    split_kv = {"auto": "auto", "off": False}.get(args.split_kv)
    if split_kv is None:
        split_kv = int(args.split_kv)
    from gqa_attention_forward_amd.inputs import GDN_WORKLOADS

    names = (list(WORKLOADS) + (list(GDN_WORKLOADS) if args.which == "fwd" else [])) if args.all else [args.workload]
    result = None
    for name in names:
        if name in GDN_WORKLOADS:
            r = run_gdn(args, fa, GDN_WORKLOADS[name])
            if name == args.workload:
                result = r
            continue
        w = WORKLOADS[name]
        q, k, v, _ = make_inputs(w, device="cuda")
        if args.layout == "bshd":  # the same values in [B, S, H, D] buffers, passed as [B, H, S, D] views
            q, k, v = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
        torch.cuda.synchronize()
        # extra time-based warm-up for the informational lines only (see warm_until)
        warm_s = 0.0 if name == args.workload else 0.25
        if args.which == "bwd":
            wall, durs, o, lse = time_gpu_bwd(fa, w, q, k, v, args.steps, args.warmup, warm_s)
        else:
            wall, durs, o, lse = time_gpu(fa, w, q, k, v, args.steps, args.warmup, split_kv, warm_s)
        path = "fa_fwd"
        if split_kv is not False and w.M <= 16384:
            tiles, wgs, ws = fa.fa_splitkv_plan(w.B, w.Hq, w.Hkv, w.M, w.N, w.D, w.causal,
                                                0 if split_kv == "auto" else split_kv)
            if args.which == "fwd" and (ws > 0 or split_kv != "auto"):
                path = f"fa_fwd_splitkv ({tiles} key tiles a share, {wgs} workgroups, merge)"
        # backward: five products per visible pair (S, dP, dV, dK, dQ) against the forward's two
        flops = accounting.workload_flops(w) * (2.5 if args.which == "bwd" else 1.0)
        tflops = flops * args.steps / wall / 1e12
        avg_ms = sum(durs) / len(durs)
        stats = step_stats(durs)
        durs = sorted(durs)
        achieved = flops / (avg_ms * 1e-3) / 1e12
        bm, bn = fa.fa_tile_shape(w.B, w.Hq, w.M, w.D)
        f_, m_, _ = fa.fa_tile_counts(w.M, w.N, bm, bn, w.causal)
        issued = 4 * bm * bn * w.D * (f_ + m_) * w.B * w.Hq * (2.5 if args.which == "bwd" else 1.0)
        line = {
            "workload": name, "pass": args.which, "layout": args.layout,
            "path": "fa_bwd (prep, dq, dk/dv)" if args.which == "bwd" else path, "tflops": round(tflops, 2), "kernel_avg_us": round(avg_ms * 1e3, 2),
            "kernel_median_us": round(durs[len(durs) // 2] * 1e3, 2), "kernel_min_us": round(durs[0] * 1e3, 2),
            "pct_mfma_peak": round(100 * achieved / MFMA_PEAK_TFLOPS, 2),
            "issued_mfma_tflops": round(issued / (avg_ms * 1e-3) / 1e12, 2),
            "compulsory_gbs": round(accounting.workload_bytes(w) / (avg_ms * 1e-3) / 1e9, 1),
        }
        if args.all and args.which == "fwd" and name in SMALL_CACHE_RESIDENT:
            # these working sets fit in the on-package caches: also a cold-cache time, and the
            # oracle on one core
            cold = time_gpu_cold(fa, w, q, k, v, args.steps, split_kv)
            line["kernel_cold_median_us"] = round(cold[len(cold) // 2] * 1e3, 2)
            if not args.no_cpu_baseline:
                line["oracle_1thread"] = oracle_one_thread(w, q, k, v)
        print(json.dumps(line), file=sys.stderr, flush=True)
        if name == args.workload:
            assert torch.isfinite(o.float()).all().item(), "non-finite output"
            traffic = read_traffic(name) if args.which == "fwd" else None
            result = {
                "metric": ("attention fwd TFLOPS (causal-adjusted) and % of MI355X FP16/BF16 MFMA peak"
                           if args.which == "fwd" else
                           "attention bwd TFLOPS (causal-adjusted, 2.5x forward flops) and % of MI355X FP16/BF16 MFMA peak"),
                "value": round(tflops, 3),
                "unit": "TFLOPS",
                "n_gpus": 1,
                "steps": args.steps,
                "warmup": args.warmup,
                "ms_per_step": round(wall / args.steps * 1e3, 4),
                "higher_is_better": True,
                "scaling": "weak",
                "vs_baseline": None,
                "dtype": "bf16" if w.dtype == torch.bfloat16 else "f16",
                "data": "synthetic",
                "config": {"workload": name, "pass": args.which, "layout": args.layout, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "M": w.M, "N": w.N, "D": w.D,
                           "causal": w.causal, "seed": w.seed, "peaky_k_rows": w.peak_rate,
                           "parallelism": "single GPU"},
                "pct_of_peak": round(100 * tflops / MFMA_PEAK_TFLOPS, 3),
                # MFMA work the launch plan issues (whole tiles, including the masked parts of
                # diagonal tiles), beside the algorithmic count the metric uses
                "issued_mfma_tflop_per_step": round(issued / 1e12, 4),
                "algorithmic_tflop_per_step": round(flops / 1e12, 4),
                "step_ms": stats,
                "roofline": roofline(w, flops, avg_ms, traffic),
                "cpu_baseline": None,
            }
            if not args.no_cpu_baseline and args.which == "fwd":
                result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds, o, lse)
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)
    chk = (result.get("cpu_baseline") or {}).get("check") if result else None
    if chk is not None and not chk["ok"]:
        print(f"bench.py: the timed output disagrees with the oracle on {chk['rows']} sampled rows: {chk}",
              file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
