"""The GPU parity checks' own arithmetic, on the CPU: a plausible kernel
mistake that the whole-tensor rel_F misses (one chunk of one row, one
token's share of one router-weight column) exceeds the per-row and
per-expert bounds of tests/gpu_util.compare_layer, while rounding-sized
noise stays inside them."""
import numpy as np
import pytest

from fine_grained_mixture_top_amd import inputs as I

import gpu_util as U


@pytest.fixture(scope="module")
def case():
    w = I.Workload("chk", T=1200, d=256, E=16, n=128, K=4, dtype="bf16", seed=5)
    a = I.draw_all(w)
    o = U.oracle_layer(w, a["x"], a["w_r"], a["w1"], a["w2"], a["d_o"])
    return w, o


def noisy(o, rel, rng):
    """The oracle's outputs with independent relative noise of size `rel`."""
    keys = ("O", "H", "A", "Y", "dH", "dXt", "dS", "dX", "dWr", "dW1", "dW2", "db")
    src = dict(dXt="dXt_row")
    return {k: o[src.get(k, k)] * (1 + rel * rng.standard_normal(o[src.get(k, k)].shape)) for k in keys}


def test_rounding_noise_passes(case):
    w, o = case
    g = noisy(o, 3e-3, np.random.default_rng(0))
    U.compare_layer(g, o, "bf16")


def test_one_wrong_chunk_fails_per_row(case):
    """8 of d = 256 columns of one dX row zeroed: rel_F stays tiny, the row
    check catches it."""
    w, o = case
    g = noisy(o, 1e-3, np.random.default_rng(1))
    g["dX"] = g["dX"].copy()
    g["dX"][17, 64:72] = 0.0
    assert U.relF(g["dX"], o["dX"]) < U.BF16_TOL
    with pytest.raises(AssertionError, match="dX/row"):
        U.compare_layer(g, o, "bf16")


def test_one_wrong_router_column_fails(case):
    """One expert's dW_r column 5% off (as a wrong per-expert factor would
    make it): rel_F over all 16 columns stays under the bar, the per-column
    check catches it."""
    w, o = case
    g = noisy(o, 1e-3, np.random.default_rng(2))
    g["dWr"] = g["dWr"].copy()
    g["dWr"][:, 5] *= 1.05
    assert U.relF(g["dWr"], o["dWr"]) < U.BF16_TOL
    with pytest.raises(AssertionError, match="dWr/row"):
        U.compare_layer(g, o, "bf16")


def test_cancelling_router_column_is_not_flagged():
    """An expert with a handful of tokens whose dz nearly cancel: an error of
    rounding size on the scores moves its column far more than the column's
    own norm, and the per-column bound follows the scores, not that norm."""
    w = I.Workload("chk_sparse", T=40, d=256, E=64, n=128, K=4, dtype="bf16", seed=5)
    a = I.draw_all(w)
    o = U.oracle_layer(w, a["x"], a["w_r"], a["w1"], a["w2"], a["d_o"])
    c = np.linalg.norm(o["dWr"], axis=0)
    live = c > 0
    ratio = o["dWr_scale"][live] / c[live]
    assert ratio.max() > 20  # this case has such a column
    # column errors of 0.5% of the scale (rounding-sized) pass everywhere
    g = noisy(o, 0.0, np.random.default_rng(3))
    rng = np.random.default_rng(4)
    d = rng.standard_normal(g["dWr"].shape)
    d *= 0.005 * np.where(o["dWr_scale"] > 0, o["dWr_scale"], 0) / np.maximum(np.linalg.norm(d, axis=0), 1e-30)
    g["dWr"] = o["dWr"] + d
    U.compare_layer(g, o, "bf16")


def test_router_column_scale_is_zero_only_for_empty_experts(case):
    w, o = case
    s = o["dWr_scale"]
    assert np.all((s == 0) == (o["counts"] == 0))
    assert np.all(s[o["counts"] > 0] > 0)
