"""GPU parity of the unfused layer (moe_fwd_unfused / moe_bwd_unfused): the
standard workflow with separate gather, SwiGLU and SwiGLU-backward kernels,
X_g / H / A / Y cached, dS = <dO_g, Y>.  Its outputs must match the fp64
oracle to the same tolerances as the fused layer, its cache must hold the
oracle's per-row activations, and the gathered rows must be exact copies."""
import numpy as np
import pytest
import torch

from fine_grained_mixture_top_amd import binding as B
from fine_grained_mixture_top_amd import inputs as I

from gpu_util import (assert_routing_equal, compare_layer, dev, host64, host_int, oracle_layer, relF,
                      routing_host, tol)

pytestmark = pytest.mark.gpu


def W(name, T, d, E, n, K, dtype, seed=0):
    return I.Workload(name, T=T, d=d, E=E, n=n, K=K, dtype=dtype, seed=seed)


def cache_views(L: B.Layer, w: I.Workload, P: int) -> dict:
    """X_g, H, A, Y of the first P rows, from the cache blocks (256-byte aligned, in that order)."""
    dt = B.TORCH_DTYPE[L.desc.dtype]
    es = torch.empty(0, dtype=dt).element_size()
    cap = L.routing.cap
    up = lambda v: (v + 255) // 256 * 256
    out, off = {}, 0
    for name, width in (("Xg", w.d), ("H", 2 * w.n), ("A", w.n), ("Y", w.d)):
        out[name] = L.cache[off:off + P * width * es].view(dt).reshape(P, width)
        off += up(cap * width * es)
    assert off == B.moe_unfused_cache_bytes(L.desc)
    return out


def run(w, a, unfused, round_mode=0, tile=128, flags=0):
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, w.dtype, round_mode=round_mode, round_seed=3, tile=tile,
                       flags=flags)
    L = B.Layer(desc, unfused=unfused)
    X, WR, W1, W2, DO = (dev(a[k], w.dtype) for k in ("x", "w_r", "w1", "w2", "d_o"))
    L.route(X, WR)
    L.forward(X, W1, W2)
    L.backward(X, WR, W1, W2, DO)
    torch.cuda.synchronize()
    return L, X


def outputs(L, P):
    return dict(O=host64(L.o), dS=host64(L.ds[:P]), dX=host64(L.dx), dWr=host64(L.dw_r),
                dW1=host64(L.dw1), dW2=host64(L.dw2), db=host64(L.db))


CASES = [
    # (workload, round_mode, tile, flags)
    (W("f32_ragged", 300, 128, 16, 64, 4, "f32", seed=5), 0, 128, 0),
    (W("bf16_small_dims", 700, 128, 16, 64, 3, "bf16", seed=6), 0, 128, 0),
    (W("bf16_256_tiles", 1200, 512, 16, 256, 4, "bf16", seed=7), 0, 128, 0),
    (W("bf16_gemm128", 1200, 512, 16, 256, 4, "bf16", seed=7), 0, 128, B.MOE_FLAG_GEMM_128),
    (W("bf16_empty_experts", 100, 256, 64, 256, 2, "bf16", seed=8), 0, 128, 0),
    (W("bf16_rounded", 1800, 256, 16, 256, 2, "bf16", seed=9), 2, 256, 0),
    # n = 128 with d = 256: the down-projection's K = 128 on the k = 64 row
    # kernel and dW2 from pre-gathered dO rows on the 128-row kernel
    (W("bf16_n128", 1000, 256, 16, 128, 4, "bf16", seed=10), 0, 128, 0),
]


@pytest.mark.parametrize("w,mode,tile,flags", CASES, ids=[c[0].name for c in CASES])
def test_unfused_layer_matches_oracle(w, mode, tile, flags):
    a = I.draw_all(w)
    L, X = run(w, a, True, mode, tile, flags)
    g_rt = routing_host(L, w)
    o = oracle_layer(w, a["x"], a["w_r"], a["w1"], a["w2"], a["d_o"], round_mode=mode, round_seed=3, tile=tile)
    assert_routing_equal(g_rt, o)
    P = g_rt["n_rows"]
    c = cache_views(L, w, P)
    # the gather is a copy: bit-exact
    rt = torch.from_numpy(g_rt["row_token"]).cuda()
    assert torch.equal(c["Xg"], X[rt]) if P else True
    g = outputs(L, P)
    g.update(H=host64(c["H"]), A=host64(c["A"]), Y=host64(c["Y"]))
    errs = compare_layer(g, o, w.dtype, skip=("dH", "dXt"))
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()})
    for e in np.nonzero(o["counts"] == 0)[0]:
        assert np.all(g["dW1"][e] == 0) and np.all(g["dW2"][e] == 0)


@pytest.mark.parametrize("w", [CASES[2][0], CASES[0][0]], ids=lambda w: w.name)
def test_unfused_agrees_with_fused(w):
    """Same inputs through both layers: identical routing, outputs within the
    dtype tolerance of each other."""
    a = I.draw_all(w)
    Lf, _ = run(w, a, False)
    Lu, _ = run(w, a, True)
    for k in ("offsets", "row_token", "row_gate", "tok_row"):
        assert torch.equal(getattr(Lf.routing, k), getattr(Lu.routing, k)), k
    P = int(host_int(Lf.routing.offsets)[-1])
    gf, gu = outputs(Lf, P), outputs(Lu, P)
    gf["H"] = host64(Lf.h_cache[:P])
    gu["H"] = host64(cache_views(Lu, w, P)["H"])
    for k in ("O", "H", "dS", "dX", "dWr", "dW1", "dW2"):
        assert relF(gu[k], gf[k]) <= tol(w.dtype), k


def test_unfused_is_deterministic():
    w = CASES[2][0]
    a = I.draw_all(w)
    L1, _ = run(w, a, True)
    L2, _ = run(w, a, True)
    for k in ("o", "dx", "dw_r", "dw1", "dw2"):
        assert torch.equal(getattr(L1, k), getattr(L2, k)), k


@pytest.mark.parametrize("name", ["fg7b_bf16", "olmoe_bf16"])
def test_unfused_full_size_agrees_with_fused(name):
    """Full workload size, the benchmark's configuration: the unfused layer
    against the fused one on the same inputs (the fused layer's full-size
    parity with the oracle is tested in test_gpu_fullsize.py); the gathered
    rows are exact copies."""
    w = I.WORKLOADS[name]
    a = I.draw_all(w)
    Lf, _ = run(w, a, False)
    Lu, X = run(w, a, True)
    assert torch.equal(Lf.routing.row_token, Lu.routing.row_token)
    P = int(host_int(Lf.routing.offsets)[-1])
    c = cache_views(Lu, w, P)
    assert torch.equal(c["Xg"], X[Lu.routing.row_token[:P].long()])
    for k in ("o", "dx", "dw_r", "dw1", "dw2"):
        e = relF(host64(getattr(Lu, k)), host64(getattr(Lf, k)))
        assert e <= tol(w.dtype), (k, e)
    assert relF(host64(c["H"]), host64(Lf.h_cache[:P])) <= tol(w.dtype)
