"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP layer through the C ABI, bring results back as float64, and compare with
the oracle.  Every expected value comes from oracle/ on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

from fine_grained_mixture_top_amd import binding as B
from fine_grained_mixture_top_amd import inputs as I
from oracle import moe_oracle as O

BF16_TOL = 1.5e-2
F32_TOL = 1e-5


def tol(dtype: str) -> float:
    return BF16_TOL if dtype == "bf16" else F32_TOL


def dev(a, dtype: str):
    """Host input (bf16 as uint16 bits, or float32) -> device tensor."""
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_int(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def relF(gpu: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm((gpu - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return float(num / den) if den > 0 else float(num)


def run_gpu(w: I.Workload, x, w_r, w1, w2, d_o, bias=None, round_mode=0, round_seed=0,
            scores=None, backward=True, flags=0, tile=128):
    """Route + forward (+ backward) on the GPU; returns the Layer and device inputs."""
    flags |= B.MOE_FLAG_SCORES_GIVEN if scores is not None else 0
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, w.dtype, round_mode=round_mode,
                       round_seed=round_seed, flags=flags, tile=tile)
    L = B.Layer(desc)
    X, WR, W1, W2, DO = (dev(a, w.dtype) for a in (x, w_r, w1, w2, d_o))
    bias_t = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    if scores is not None:
        L.routing.logits.copy_(torch.from_numpy(np.ascontiguousarray(scores, np.float32)).view(-1))
    L.route(X, WR, bias_t)
    L.forward(X, W1, W2)
    if backward:
        L.backward(X, WR, W1, W2, DO)
    torch.cuda.synchronize()
    return L, dict(x=X, w_r=WR, w1=W1, w2=W2, d_o=DO)


def routing_host(L: B.Layer, w: I.Workload) -> dict:
    r = L.routing
    P = int(host_int(r.offsets)[-1])
    return dict(
        logits=host64(r.logits).reshape(w.T, w.E),
        topk_idx=host_int(r.topk_idx).reshape(w.T, w.K),
        topk_gate=host64(r.topk_gate).reshape(w.T, w.K),
        counts=host_int(r.counts), counts_raw=host_int(r.counts_raw),
        offsets=host_int(r.offsets), tile_offsets=host_int(r.tile_offsets),
        row_token=host_int(r.row_token)[:P], row_expert=host_int(r.row_expert)[:P],
        row_gate=host64(r.row_gate)[:P], tok_ptr=host_int(r.tok_ptr), tok_row=host_int(r.tok_row)[:P],
        n_rows=P)


INT_KEYS = ("counts", "offsets", "tile_offsets", "row_token", "row_expert", "tok_ptr", "tok_row")


def assert_routing_equal(g: dict, o: dict, check_topk=True):
    if check_topk:
        assert np.array_equal(g["topk_idx"], o["topk_idx"]), "topk_idx"
    assert np.array_equal(g["counts_raw"], o["counts_raw"]), "counts_raw"
    for k in INT_KEYS:
        assert np.array_equal(np.asarray(g[k]), np.asarray(o[k])), k


def layer_outputs(L: B.Layer, w: I.Workload) -> dict:
    """Every float result of the GPU layer, per row in the GPU's row order."""
    P = int(host_int(L.routing.offsets)[-1])
    dt = B.TORCH_DTYPE[L.desc.dtype]
    n, d = w.n, w.d
    out = dict(
        O=host64(L.o), H=host64(L.h_cache[:P]),
        A=host64(L.ws_view(B.MOE_ITEM_A, P * n, dt)).reshape(P, n),
        Y=host64(L.ws_view(B.MOE_ITEM_Y, P * d, dt)).reshape(P, d),
        dH=host64(L.ws_view(B.MOE_ITEM_DH, P * 2 * n, dt)).reshape(P, 2 * n),
        dXt=host64(L.ws_view(B.MOE_ITEM_DXT, P * d, dt)).reshape(P, d),
        dS=host64(L.ds[:P]), dz_row=host64(L.ws_view(B.MOE_ITEM_DZ, P, torch.float32)),
        dX=host64(L.dx), dWr=host64(L.dw_r), dW1=host64(L.dw1), dW2=host64(L.dw2), db=host64(L.db))
    return out


def oracle_layer(w: I.Workload, x, w_r, w1, w2, d_o, bias=None, round_mode=0, round_seed=0,
                 scores=None, tile=128):
    return O.layer(x, w_r, w1, w2, d_o, w.dtype, w.K, bias=bias, tile=tile, round_mode=round_mode,
                   round_seed=round_seed, scores=scores)


def compare_layer(g: dict, o: dict, dtype: str, skip=()):
    """rel_F of every output; returns the dict of errors (asserts the tolerance)."""
    t = tol(dtype)
    errs = {}
    pairs = dict(O="O", H="H", A="A", Y="Y", dH="dH", dXt="dXt", dS="dS", dX="dX", dWr="dWr",
                 dW1="dW1", dW2="dW2")
    for gk, ok in pairs.items():
        if gk in skip:
            continue
        errs[gk] = relF(g[gk], o[ok])
    if "db" not in skip:
        # db sums per-row dz values that largely cancel (each token's dz sums to
        # zero), so its error is measured against the size of its summands
        scale = np.linalg.norm(np.abs(o["dz"]).sum(axis=0))
        errs["db"] = float(np.linalg.norm(g["db"] - o["db"]) / scale) if scale > 0 else 0.0
    bad = {k: v for k, v in errs.items() if not v <= t}
    assert not bad, f"outside tolerance {t}: {bad} (all: {errs})"
    return errs
