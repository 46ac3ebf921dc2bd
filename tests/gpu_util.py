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
    o = O.layer(x, w_r, w1, w2, d_o, w.dtype, w.K, bias=bias, tile=tile, round_mode=round_mode,
                round_seed=round_seed, scores=scores)
    o["dWr_scale"] = router_column_scale(o, np.linalg.norm(O.to_f64(x, w.dtype), axis=1), w.E)
    o["dXt_row"] = dxt_with_router_term(o["dXt"], o["dz"][o["row_token"], o["row_expert"]],
                                        O.to_f64(w_r, w.dtype), o["row_expert"])
    return o


def dxt_with_router_term(dXt, dz_rows, wr64, row_expert):
    """What the library keeps per routed row as its input gradient
    (MOE_ITEM_DXT): dXt_r plus the row's router term dz_r W_r[:, e_r]^T, so
    that dX_t is the plain sum of its rows."""
    return dXt + np.asarray(dz_rows)[:, None] * np.asarray(wr64)[:, np.asarray(row_expert)].T


def router_column_scale(o: dict, x_norm: np.ndarray, E: int) -> np.ndarray:
    """Per expert e, the size of the error that dW_r[:, e] = sum_t x_t dz[t,e]
    picks up from a relative error in the per-row scores dS: dz[t,e] =
    g_te (dS_te - sum_e' g_te' dS_te') moves by g_te (|dS_te| + sum_e' g_te'
    |dS_te'|) per unit of relative dS error, whatever the (possibly
    cancelling) value of dz itself, so the column's error scale is
    sqrt(sum_t ||x_t||^2 u_te^2) with u that bound.  Zero for an expert
    without rows."""
    rt, re_, g, dS = o["row_token"], o["row_expert"], o["row_gate"], np.abs(o["dS"])
    s_tok = np.zeros(x_norm.shape[0])
    np.add.at(s_tok, rt, g * dS)
    u = g * (dS + s_tok[rt])
    sq = np.zeros(E)
    np.add.at(sq, re_, (x_norm[rt] * u) ** 2)
    return np.sqrt(sq)


ROW_FACTOR = 3.0  # per-row / per-expert bound = ROW_FACTOR x the tensor tolerance


def row_rel_max(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest per-row relative error max_i ||gpu_i - ref_i|| / ||ref_i||.  A
    reference row that is exactly zero must be exactly zero on the GPU too
    (empty sets, empty experts)."""
    g = gpu.reshape(gpu.shape[0], -1)
    r = ref.reshape(ref.shape[0], -1)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), f"{int((num[zero] != 0).sum())} zero rows are not zero"
    return float((num[~zero] / den[~zero]).max()) if (~zero).any() else 0.0


def scalar_rel_max(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest error of a per-row scalar relative to the RMS of the reference
    (a scalar near zero has no meaningful relative error of its own)."""
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    err = np.abs(gpu - ref)
    if rms == 0:
        assert np.all(err == 0)
        return 0.0
    return float(err.max() / rms)


PER_ROW = ("O", "H", "A", "Y", "dH", "dXt", "dX")


def router_column_err_max(gpu: np.ndarray, ref: np.ndarray, scale: np.ndarray) -> float:
    """Largest ||dW_r[:, e] error|| / scale_e over experts (router_column_scale);
    an expert without rows must have an exactly zero column."""
    num = np.linalg.norm(gpu - ref, axis=0)
    zero = scale == 0
    assert np.all(num[zero] == 0), "a router column of an expert without rows is not zero"
    return float((num[~zero] / scale[~zero]).max()) if (~zero).any() else 0.0


def compare_layer(g: dict, o: dict, dtype: str, skip=()):
    """Every output within tolerance three ways: rel_F of the whole tensor
    (<= tol), the largest per-row error of every per-row tensor and of the
    per-row scores dS, and per expert rel_F of dW1 and dW2 (<= ROW_FACTOR x
    tol), and the error of each dW_r column against the error its dz can
    carry (router_column_scale; <= tol), so that one wrong row, chunk or
    expert cannot hide in a large tensor.  Returns the errors (asserts)."""
    t = tol(dtype)
    errs, rows = {}, {}
    pairs = dict(O="O", H="H", A="A", Y="Y", dH="dH", dXt="dXt_row", dS="dS", dX="dX", dWr="dWr",
                 dW1="dW1", dW2="dW2", db="db")
    for gk, ok in pairs.items():
        if gk in skip:
            continue
        errs[gk] = relF(g[gk], o[ok])
        if gk in PER_ROW:
            rows[gk] = row_rel_max(g[gk], o[ok])
        elif gk == "dS":
            rows[gk] = scalar_rel_max(g[gk], o[ok])
        elif gk in ("dW1", "dW2"):
            rows[gk] = row_rel_max(g[gk], o[ok])  # one "row" per expert
        elif gk == "dWr":
            rows[gk] = router_column_err_max(g[gk], o[ok], o["dWr_scale"])
    print("rel_F:", {k: f"{v:.2e}" for k, v in errs.items()},
          "max per row/expert:", {k: f"{v:.2e}" for k, v in rows.items()})
    bad = {k: v for k, v in errs.items() if not v <= t}
    # a dW_r column's scale already bounds its summands (about twice the norm
    # of a column whose dz do not cancel), so its bound is tol, not ROW_FACTOR tol
    bad.update({f"{k}/row": v for k, v in rows.items() if not v <= (t if k == "dWr" else ROW_FACTOR * t)})
    assert not bad, f"outside tolerance {t} (rows {ROW_FACTOR * t}): {bad} (all: {errs}, rows: {rows})"
    return errs
