"""Router bias of the skewed workload (zipf_e256): expert loads that follow a
capped Zipf law.

TEST / BENCHMARK INPUT GENERATION ONLY.  This script uses the oracle's
routing (fp64 logits, top-K on float32 scores) to fit a per-expert bias and
writes it to fine_grained_mixture_top_amd/zipf_e256_bias.json, from where the
input generator reads it.  Nothing here runs on the product path.

Recipe:
  1. Target loads L_e = T*K*p_e with p_e proportional to (e+1)^-s (s = 1.1),
     capped at T (an expert takes a token at most once); the excess of capped
     experts is spread over the others in proportion to p_e until none exceeds
     T (water filling).
  2. Starting from b = 0, 50 fixed-point steps
        b_e <- b_e + 0.5 * (ln L_e - ln max(load_e(b), 0.5)),
     where load_e(b) is the number of tokens whose top-K set (of X W_r + b on
     the workload's own X and W_r) contains e.
  3. The ranks are assigned to experts by a random permutation drawn from the
     bias child stream, so that the heavy experts are not all at low ids.

Run:  python -m oracle.zipf_bias
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import moe_oracle as O  # noqa: E402

OUT = os.path.join(ROOT, "fine_grained_mixture_top_amd", "zipf_e256_bias.json")


def target_loads(T: int, K: int, E: int, s: float) -> np.ndarray:
    """Zipf(s) loads of T*K rows over E ranks, capped at T with water filling."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    L = T * K * p
    capped = np.zeros(E, dtype=bool)
    while True:
        over = (L > T) & ~capped
        if not over.any():
            return L
        capped |= over
        excess = (L[capped] - T).sum()
        L[capped] = T
        free = ~capped
        L[free] += excess * p[free] / p[free].sum()


def loads(z0: np.ndarray, b: np.ndarray, K: int) -> np.ndarray:
    idx = O.topk(O.decision_scores(z0 + b[None, :]), K)
    return np.bincount(idx.ravel(), minlength=z0.shape[1]).astype(np.float64)


def fit(z0: np.ndarray, K: int, target: np.ndarray, steps: int = 50) -> np.ndarray:
    b = np.zeros(z0.shape[1], dtype=np.float64)
    for _ in range(steps):
        b += 0.5 * (np.log(target) - np.log(np.maximum(loads(z0, b, K), 0.5)))
    return b


def main():
    from fine_grained_mixture_top_amd import inputs as I
    w = I.WORKLOADS["zipf_e256"]
    s = 1.1
    x64 = O.to_f64(I.draw_x(w), w.dtype)
    wr64 = O.to_f64(I.draw_wr(w), w.dtype)
    g = np.random.Generator(np.random.PCG64(I._children(w.seed)[5]))
    perm = g.permutation(w.E)            # rank of expert e is perm[e]
    target = target_loads(w.T, w.K, w.E, s)[perm]
    z0 = O.router_logits(x64, wr64)
    b = fit(z0, w.K, target)
    b32 = b.astype(np.float32)
    got = loads(z0, b32.astype(np.float64), w.K)
    rec = {
        "workload": w.name, "zipf_s": s, "steps": 50,
        "bias": [float(v) for v in b32],
        "target_loads": [float(v) for v in target],
        "loads": [int(v) for v in got],
        "summary": {"max": int(got.max()), "min": int(got.min()), "median": float(np.median(got)),
                    "below_128": int((got < 128).sum()), "partial_tile": int((got % 128 != 0).sum())},
    }
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec["summary"]))


if __name__ == "__main__":
    main()
