"""Host-side checks of bench.py (no GPU): the algorithmic work it divides by,
the one-GPU contract and the lookup of the committed HBM counter passes."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fine_grained_mixture_top_amd import hbm_traffic  # noqa: E402
from fine_grained_mixture_top_amd import inputs as I  # noqa: E402


@pytest.mark.parametrize("name", ["fg7b_bf16", "olmoe_bf16", "sweep_e256", "prod_e256"])
def test_grouped_gemm_flops_add_up_to_the_step(name):
    """The six grouped GEMMs of a step do 18 P d n FLOPs (6 P d n forward,
    12 P d n backward), the MXFP8 ones the same as their bf16 kernels."""
    w = I.WORKLOADS[name]
    P = w.T * w.K
    es = 2
    total = sum(bench.kernel_work(k, w, P, es)[0] for k in ("up", "down", "dh", "dxt", "dw1", "dw2"))
    assert total == 18.0 * P * w.d * w.n
    fwd = sum(bench.kernel_work(k, w, P, es)[0] for k in ("up", "down"))
    assert fwd == 6.0 * P * w.d * w.n
    for k in ("up", "down", "dh", "dxt"):
        assert bench.kernel_work(k + "_mx", w, P, es) == bench.kernel_work(k, w, P, es)
    for k in ("up", "dw1", "agg_o", "agg_dx", "route_select"):
        amount, kind = bench.kernel_work(k, w, P, es)
        assert amount > 0 and kind == ("byte" if k in ("agg_o", "agg_dx", "route_select") else "flop")


def test_aggregation_bytes_count_each_row_once():
    w = I.WORKLOADS["fg7b_bf16"]
    P = w.T * w.K
    b, kind = bench.kernel_work("agg_o", w, P, 2)
    assert kind == "byte"
    # Y rows in, O out, gate + row index per row, token pointers
    assert b == P * w.d * 2 + w.T * w.d * 2 + P * 8 + (w.T + 1) * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on():
    """The benchmark line reports the committed counter passes' traffic only
    while the kernel sources hash to the value recorded with them."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_fg7b_bf16.json")
    rec = json.load(open(path))
    current = rec["source_hash"] == hbm_traffic.source_hash()
    for k in ("up", "down", "dh", "dxt", "dw1", "dw2", "agg_o", "agg_dx"):
        want = round(rec["kernels"][k]["bytes"]) if current else None
        assert bench.measured_traffic("fg7b_bf16", k) == want
    assert bench.measured_traffic("tiny_f32", "up") is None  # no counter passes for that workload


def test_cpu_baseline_reports_forward_and_backward_apart():
    """The oracle baseline names the CPU, times routing + forward and the
    backward apart, and takes a median on the tiny workload."""
    w = I.WORKLOADS["tiny_f32"]
    a = I.draw_all(w)
    r = bench.cpu_baseline(w, a, w.T, repeats=5)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["cpu"]
    assert r["fwd_s"] > 0 and r["bwd_s"] > 0
    assert "median of 5" in r["sample"]
    rows = w.T * w.K
    assert abs(r["value"] - 18.0 * rows * w.d * w.n / (r["fwd_s"] + r["bwd_s"]) / 1e12) <= 1e-2 * r["value"]
