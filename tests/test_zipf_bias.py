"""The skewed workload's stored router bias (written by oracle/zipf_bias.py).

Checks the capped-Zipf target loads against their definition and that the
stored bias, put through the oracle's routing on the workload's own tokens,
still gives the stored loads, close to the targets.
"""
import json
import os

import numpy as np

from fine_grained_mixture_top_amd import inputs as I
from oracle import moe_oracle as O
from oracle import zipf_bias as Z


def test_target_loads_are_capped_zipf():
    T, K, E, s = 1000, 8, 64, 1.1
    L = Z.target_loads(T, K, E, s)
    assert abs(L.sum() - T * K) < 1e-6 * T * K
    assert L.max() <= T + 1e-9
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    free = L < T - 1e-9
    ratio = L[free] / p[free]
    assert np.allclose(ratio, ratio[0])          # uncapped experts keep the Zipf shape
    assert np.all(L[~free] >= L[free].max())      # only the heaviest ranks are capped
    assert (~free).sum() >= 1                      # rank 1 alone would want 1.6 T rows here


def test_stored_bias_reproduces_its_loads():
    w = I.WORKLOADS["zipf_e256"]
    path = os.path.join(os.path.dirname(I.__file__), w.bias_file)
    rec = json.load(open(path))
    b = I.draw_bias(w)
    assert b.dtype == np.float32 and b.shape == (w.E,)
    z0 = O.router_logits(O.to_f64(I.draw_x(w), w.dtype), O.to_f64(I.draw_wr(w), w.dtype))
    got = Z.loads(z0, b.astype(np.float64), w.K)
    assert np.array_equal(got.astype(np.int64), np.asarray(rec["loads"]))
    assert got.sum() == w.T * w.K
    target = np.asarray(rec["target_loads"])
    assert abs(target.sum() - w.T * w.K) < 1e-3
    # the fit lands within 10% of the target, or within three standard
    # deviations of a Poisson count for the light experts, for nearly all
    close = np.abs(got - target) <= np.maximum(0.1 * target, 3 * np.sqrt(target))
    assert close.mean() >= 0.95, close.mean()
    assert got.max() >= 0.9 * w.T                  # the heaviest expert is near saturation
