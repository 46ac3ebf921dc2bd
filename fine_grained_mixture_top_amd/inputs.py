"""Seeded synthetic inputs for the fine-grained MoE layer.

This module only draws numbers: it holds none of the layer's arithmetic
(no routing, no GEMM, no activation).  Both the HIP path (through the
binding) and the fp64 oracle (through the tests) take their inputs from here.

Recipe (one child stream per tensor, numpy PCG64):
  SeedSequence(seed).spawn(6) -> children for x, W_r, W1, W2, dO, bias (in
  that order).  W1 and W2 spawn one further child per expert so one expert's
  weights can be drawn without drawing the others.  Every draw is
  ``standard_normal(dtype=float32) * std``; for bf16 workloads the fp32 values
  are rounded to bf16 by round-to-nearest-even on the bit pattern.

Distributions: x ~ N(0, 1), W_r, W1, W2 ~ N(0, 0.02^2) (0.02 is the standard
deviation), dO ~ N(0, 1), bias = 0 except for the skewed workload.

Shapes (row-major):  x [T, d], W_r [d, E], W1 [E, d, 2n] (columns 0..n-1 are
the SwiGLU gate half, n..2n-1 the up half), W2 [E, n, d], dO [T, d], bias [E]
(fp32).

bf16 tensors are returned as ``uint16`` bit patterns (numpy has no bf16).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import json
import math
import os
from typing import Optional

import numpy as np

W_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    n: int
    K: int
    dtype: str  # "f32" or "bf16"
    zipf_s: Optional[float] = None  # skewed per-expert bias when set
    seed: int = 0
    bias_file: Optional[str] = None  # fitted bias stored beside this module (overrides the closed form)

    @property
    def P(self) -> int:
        """Routed (token, expert) rows without token rounding."""
        return self.T * self.K

    def flops_fwd_bwd(self, rows: Optional[int] = None) -> float:
        """Useful FLOPs of the six expert GEMMs: 6*P*d*n forward, 12*P*d*n backward."""
        p = self.P if rows is None else rows
        return 18.0 * p * self.d * self.n


# The workloads the layer is measured and checked on.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=256, d=128, E=8, n=64, K=2, dtype="f32"),
    "fg7b_bf16": Workload("fg7b_bf16", T=32768, d=1536, E=128, n=256, K=8, dtype="bf16"),
    "sweep_e32": Workload("sweep_e32", T=16384, d=2048, E=32, n=1024, K=2, dtype="bf16"),
    "sweep_e64": Workload("sweep_e64", T=16384, d=2048, E=64, n=512, K=4, dtype="bf16"),
    "sweep_e128": Workload("sweep_e128", T=16384, d=2048, E=128, n=256, K=8, dtype="bf16"),
    "sweep_e256": Workload("sweep_e256", T=16384, d=2048, E=256, n=128, K=16, dtype="bf16"),
    "zipf_e256": Workload("zipf_e256", T=32768, d=2048, E=256, n=256, K=8, dtype="bf16",
                          zipf_s=1.1, bias_file="zipf_e256_bias.json"),
    "prod_e256": Workload("prod_e256", T=16384, d=7168, E=256, n=2048, K=8, dtype="bf16"),
    # the OLMoE-shaped layer the pages break down per kernel
    "olmoe_bf16": Workload("olmoe_bf16", T=32768, d=2048, E=64, n=1024, K=8, dtype="bf16"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(6)


def _draw(ss: np.random.SeedSequence, shape, std: float, dtype: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def draw_x(w: Workload, rows: Optional[np.ndarray] = None) -> np.ndarray:
    x = _draw(_children(w.seed)[0], (w.T, w.d), 1.0, w.dtype)
    return x if rows is None else x[rows]


def draw_wr(w: Workload) -> np.ndarray:
    return _draw(_children(w.seed)[1], (w.d, w.E), W_STD, w.dtype)


def draw_w1_expert(w: Workload, e: int) -> np.ndarray:
    ss = _children(w.seed)[2].spawn(w.E)[e]
    return _draw(ss, (w.d, 2 * w.n), W_STD, w.dtype)


def draw_w2_expert(w: Workload, e: int) -> np.ndarray:
    ss = _children(w.seed)[3].spawn(w.E)[e]
    return _draw(ss, (w.n, w.d), W_STD, w.dtype)


def _draw_experts(kids, shape, dtype) -> np.ndarray:
    """One array per expert child stream, drawn in parallel threads (numpy
    releases the GIL while filling); the values do not depend on threading."""
    out = np.empty((len(kids),) + shape, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(e):
        out[e] = _draw(kids[e], shape, W_STD, dtype)

    workers = max(1, min(16, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(len(kids))))
    return out


def draw_w1(w: Workload) -> np.ndarray:
    return _draw_experts(_children(w.seed)[2].spawn(w.E), (w.d, 2 * w.n), w.dtype)


def draw_w2(w: Workload) -> np.ndarray:
    return _draw_experts(_children(w.seed)[3].spawn(w.E), (w.n, w.d), w.dtype)


def draw_do(w: Workload) -> np.ndarray:
    return _draw(_children(w.seed)[4], (w.T, w.d), 1.0, w.dtype)


def draw_bias(w: Workload) -> Optional[np.ndarray]:
    """Per-expert router bias (fp32) for the skewed workloads, else None.

    A workload with a ``bias_file`` reads its bias from that JSON file: for
    zipf_e256 it was fitted so that the realised loads follow a capped
    Zipf(1.1) law on the workload's own tokens (see oracle/zipf_bias.py, which
    wrote it).  Otherwise the expected load of expert e is meant to follow Zipf(s): p_e proportional
    to (e+1)^-s.  The bias is set in closed form, with no routing involved:
    treating each logit's data part x.W_r[:, e] as noise of standard deviation
    sigma = 0.02*sqrt(d) and approximating that Gaussian noise by a Gumbel law
    of scale beta = sigma*sqrt(6)/pi (same variance), the Gumbel-max property
    makes the chance of an expert winning proportional to exp(b_e/beta), so
    b_e = beta*ln(p_e) (centred to zero mean) gives loads close to Zipf(s).
    A random permutation (drawn from the bias child stream) decides which
    expert takes which Zipf rank, so heavy experts are not all at low ids.
    """
    if w.bias_file is not None:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), w.bias_file)) as f:
            return np.asarray(json.load(f)["bias"], dtype=np.float32)
    if w.zipf_s is None:
        return None
    sigma = W_STD * math.sqrt(w.d)
    beta = sigma * math.sqrt(6.0) / math.pi
    ranks = np.arange(1, w.E + 1, dtype=np.float64)
    logp = -w.zipf_s * np.log(ranks)
    logp -= np.log(np.exp(logp).sum())
    b = beta * (logp - logp.mean())
    g = np.random.Generator(np.random.PCG64(_children(w.seed)[5]))
    perm = g.permutation(w.E)
    return b[perm].astype(np.float32)


def draw_logits(T: int, E: int, seed: int, ties: bool = True) -> np.ndarray:
    """fp32 router scores for routing-only checks (given-logits mode).

    With ``ties`` the values are drawn on a coarse grid (multiples of 1/64 in
    [-2, 2]) so that exactly equal scores are frequent and every tie-break rule
    is exercised.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    if ties:
        v = g.integers(-128, 129, size=(T, E)).astype(np.float32) / np.float32(64.0)
    else:
        v = g.standard_normal(size=(T, E), dtype=np.float32)
    return v


def draw_all(w: Workload) -> dict:
    """Every input of one workload (host arrays)."""
    return dict(x=draw_x(w), w_r=draw_wr(w), w1=draw_w1(w), w2=draw_w2(w), d_o=draw_do(w),
                bias=draw_bias(w))
