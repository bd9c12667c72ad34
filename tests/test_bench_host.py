"""bench.py's host-side contract (no GPU): the one-GPU refusal, the step statistics and the
roofline arithmetic of the JSON line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gqa_attention_forward_amd.inputs import ALL_WORKLOADS  # noqa: E402
from gqa_attention_forward_amd import accounting  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_step_stats():
    durs = [5.0, 4.0, 3.0, 2.0, 2.0, 2.0, 2.0, 2.0, 1.0, 1.5]
    st = bench.step_stats(durs)
    assert st["min"] == 1.0
    assert st["median"] == 2.0               # element len // 2 of the sorted list
    assert st["mean"] == round(sum(durs) / len(durs), 4)
    assert st["mean_first5"] == round((5 + 4 + 3 + 2 + 2) / 5, 4)
    assert st["mean_last5"] == round((2 + 2 + 2 + 1 + 1.5) / 5, 4)
    short = bench.step_stats([3.0, 1.0])     # fewer than five steps: means over what there is
    assert short["mean_first5"] == short["mean_last5"] == 2.0


def test_roofline_bound_and_fraction():
    # the long causal prefill is far above the machine balance: MFMA-bound
    w = ALL_WORKLOADS["long_causal_gqa_16k"]
    flops = accounting.workload_flops(w)
    r = bench.roofline(w, flops, 2.0, 5.0e8)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(flops / 2.0e-3 / 1e12, rel=1e-6)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, abs=1e-4)
    assert r["traffic"] == 5.0e8 and r["kernel_avg_us"] == 2000.0
    # decode reads every K/V byte once for 4 flops per byte or so: HBM-bound, in GB/s
    d = ALL_WORKLOADS["decode_gqa_8k"]
    r = bench.roofline(d, accounting.workload_flops(d), 0.05, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(accounting.workload_bytes(d) / 0.05e-3 / 1e9, rel=1e-6)
