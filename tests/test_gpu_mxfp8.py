"""GPU parity of the MXFP8 forward (moe_fwd_mxfp8) with the fp64 MXFP8
oracle: every quantization code and block scale bit-exact (x, w1, w2, and A
quantized from the GPU's own bf16 A through the oracle's quantizer), and H,
A, Y, O within the bf16 tolerance of the oracle's forward on the same
quantized operands."""
import numpy as np
import pytest
import torch

from fine_grained_mixture_top_amd import binding as B
from fine_grained_mixture_top_amd import inputs as I
from oracle import moe_oracle as O
from oracle import mx_oracle as M

from gpu_util import assert_routing_equal, dev, dxt_with_router_term, host64, host_int, relF, routing_host

pytestmark = pytest.mark.gpu

TOL = 1.5e-2       # against the oracle on the same quantized operands
E2E_TOL = 3e-2     # O against the oracle's own quantization of A


def W(name, T, d, E, n, K, seed=0):
    return I.Workload(name, T=T, d=d, E=E, n=n, K=K, dtype="bf16", seed=seed)


def u8(L, item, count):
    return L.ws_view(item, count, torch.uint8).cpu().numpy()


def blocked_to_rows(s_blk, E, K, N):
    """[E][K/128][N][4] bytes -> [E][N][K/32]"""
    return s_blk.reshape(E, K // 128, N, 4).transpose(0, 2, 1, 3).reshape(E, N, K // 32)


def run_mx(w, a, round_mode=0, tile=128):
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, "bf16", round_mode=round_mode, round_seed=3, tile=tile)
    L = B.Layer(desc)
    X, WR, W1, W2 = (dev(a[k], "bf16") for k in ("x", "w_r", "w1", "w2"))
    L.route(X, WR)
    L.forward_mxfp8(X, W1, W2)
    torch.cuda.synchronize()
    return L, (X, WR, W1, W2)


CASES = [
    (W("mx_ragged", 700, 512, 16, 256, 4, seed=21), 0, 128),
    (W("mx_empty_experts", 100, 256, 64, 256, 2, seed=22), 0, 128),
    (W("mx_d2048", 300, 2048, 8, 256, 2, seed=23), 0, 128),
    (W("mx_n512_rounded", 1800, 256, 16, 512, 2, seed=24), 2, 256),
]


@pytest.mark.parametrize("w,mode,tile", CASES, ids=[c[0].name for c in CASES])
def test_mxfp8_forward_matches_oracle(w, mode, tile):
    a = I.draw_all(w)
    L, _ = run_mx(w, a, mode, tile)
    g_rt = routing_host(L, w)
    x64, wr64 = O.to_f64(a["x"], "bf16"), O.to_f64(a["w_r"], "bf16")
    w1_64, w2_64 = O.to_f64(a["w1"], "bf16"), O.to_f64(a["w2"], "bf16")
    rt = O.route(x64, wr64, None, w.K, tile, mode, 3)
    assert_routing_equal(g_rt, rt)
    o = M.forward_mxfp8(x64, w1_64, w2_64, rt)
    T, d, E, n, P = w.T, w.d, w.E, w.n, g_rt["n_rows"]
    # quantization codes and scales: bit-exact
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_XQ, T * d).reshape(T, d), o["xq"])
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_XS, T * d // 32).reshape(T, d // 32), o["xs"])
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_W1Q, E * 2 * n * d).reshape(E, 2 * n, d), o["w1q"])
    assert np.array_equal(blocked_to_rows(u8(L, B.MOE_ITEM_MX_W1S, E * d // 32 * 2 * n), E, d, 2 * n), o["w1s"])
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_W2Q, E * d * n).reshape(E, d, n), o["w2q"])
    assert np.array_equal(blocked_to_rows(u8(L, B.MOE_ITEM_MX_W2S, E * n // 32 * d), E, n, d), o["w2s"])
    A_gpu = host64(L.ws_view(B.MOE_ITEM_MX_A, P * n, torch.bfloat16)).reshape(P, n)
    aq_ref, as_ref = M.quantize(A_gpu)
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_AQ, P * n).reshape(P, n), aq_ref)
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_AS, P * n // 32).reshape(P, n // 32), as_ref)
    # float outputs.  H and A against the oracle; Y and O against the oracle's
    # down-projection and aggregation of the A codes the GPU chose (its A is
    # its own bf16 rounding, so a few codes sit one step from the oracle's)
    Y_gpu = host64(L.ws_view(B.MOE_ITEM_MX_Y, P * d, torch.bfloat16)).reshape(P, d)
    w2d = np.swapaxes(M.dequantize(o["w2q"], o["w2s"]), 1, 2)
    Ad = M.dequantize(aq_ref, as_ref)
    Y_ref = np.zeros((P, d))
    for e in range(E):
        s0, s1 = rt["offsets"][e], rt["offsets"][e + 1]
        Y_ref[s0:s1] = Ad[s0:s1] @ w2d[e]
    O_ref = np.zeros((T, d))
    np.add.at(O_ref, rt["row_token"], rt["row_gate"][:, None] * Y_ref)
    O_gpu = host64(L.o)
    errs = dict(H=relF(host64(L.h_cache[:P]), o["H"]), A=relF(A_gpu, o["A"]), Y=relF(Y_gpu, Y_ref),
                O=relF(O_gpu, O_ref))
    e2e = relF(O_gpu, o["O"])
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()}, f"O vs independent oracle {e2e:.2e}")
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, bad
    # end to end: the two sides' A roundings to E4M3 differ by one code step
    # where their bf16 A values straddle a rounding midpoint
    assert e2e <= E2E_TOL


def test_mxfp8_forward_then_bf16_backward():
    """The bf16 backward runs from the H the MXFP8 forward cached."""
    w = CASES[0][0]
    a = I.draw_all(w)
    L, (X, WR, W1, W2) = run_mx(w, a)
    DO = dev(a["d_o"], "bf16")
    L.backward(X, WR, W1, W2, DO)
    torch.cuda.synchronize()
    for t in (L.dx, L.dw1, L.dw2, L.dw_r):
        assert torch.isfinite(t.float()).all()
    # against the oracle backward from the oracle's MXFP8 H
    x64, wr64 = O.to_f64(a["x"], "bf16"), O.to_f64(a["w_r"], "bf16")
    w1_64, w2_64 = O.to_f64(a["w1"], "bf16"), O.to_f64(a["w2"], "bf16")
    rt = O.route(x64, wr64, None, w.K)
    o = M.forward_mxfp8(x64, w1_64, w2_64, rt)
    b = O.backward(x64, wr64, w1_64, w2_64, rt, M.bf16_round(o["H"]), O.to_f64(a["d_o"], "bf16"))
    for k, t in (("dX", L.dx), ("dW1", L.dw1), ("dW2", L.dw2)):
        assert relF(host64(t), b[k]) <= TOL, k


def test_mxfp8_is_deterministic():
    w = CASES[0][0]
    a = I.draw_all(w)
    L1, _ = run_mx(w, a)
    L2, _ = run_mx(w, a)
    assert torch.equal(L1.o, L2.o) and torch.equal(L1.h_cache, L2.h_cache)


@pytest.mark.parametrize("name", ["fg7b_bf16", "olmoe_bf16"])
def test_mxfp8_full_size_expert_sample(name):
    """Full workload size, the benchmark's launch configuration: two sampled
    experts over all their rows (the GPU's routing; routing parity is tested
    elsewhere): codes and scales of their tokens' x rows and of their w1 / w2
    bit-exact, H and A against the oracle, Y against the oracle's
    down-projection of the GPU's A codes."""
    w = I.WORKLOADS[name]
    a = I.draw_all(w)
    L, _ = run_mx(w, a)
    T, d, E, n = w.T, w.d, w.E, w.n
    off = host_int(L.routing.offsets)
    P = int(off[-1])
    rng = np.random.default_rng(5)
    for e in rng.choice(E, 2, replace=False):
        s0, s1 = int(off[e]), int(off[e + 1])
        rows = np.arange(s0, s1)
        tok = host_int(L.routing.row_token[s0:s1])
        x64 = O.to_f64(a["x"][tok], "bf16")
        xq, xs = M.quantize_rows(x64)
        gx = u8(L, B.MOE_ITEM_MX_XQ, T * d).reshape(T, d)[tok]
        gs = u8(L, B.MOE_ITEM_MX_XS, T * d // 32).reshape(T, d // 32)[tok]
        assert np.array_equal(gx, xq) and np.array_equal(gs, xs)
        w1q, w1s = M.quantize_weights(O.to_f64(a["w1"][e:e + 1], "bf16"))
        w2q, w2s = M.quantize_weights(O.to_f64(a["w2"][e:e + 1], "bf16"))
        g1q = u8(L, B.MOE_ITEM_MX_W1Q, E * 2 * n * d).reshape(E, 2 * n, d)[e:e + 1]
        g1s = blocked_to_rows(u8(L, B.MOE_ITEM_MX_W1S, E * d // 32 * 2 * n), E, d, 2 * n)[e:e + 1]
        g2q = u8(L, B.MOE_ITEM_MX_W2Q, E * d * n).reshape(E, d, n)[e:e + 1]
        g2s = blocked_to_rows(u8(L, B.MOE_ITEM_MX_W2S, E * n // 32 * d), E, n, d)[e:e + 1]
        assert np.array_equal(g1q, w1q) and np.array_equal(g1s, w1s)
        assert np.array_equal(g2q, w2q) and np.array_equal(g2s, w2s)
        H = M.dequantize(xq, xs) @ np.swapaxes(M.dequantize(w1q, w1s), 1, 2)[0]
        A = O.silu(H[:, :n]) * H[:, n:]
        Hg = host64(L.h_cache[s0:s1])
        Ag = host64(L.ws_view(B.MOE_ITEM_MX_A, P * n, torch.bfloat16)).reshape(P, n)[rows]
        aq, as_ = M.quantize(Ag)
        assert np.array_equal(u8(L, B.MOE_ITEM_MX_AQ, P * n).reshape(P, n)[rows], aq)
        Y = M.dequantize(aq, as_) @ np.swapaxes(M.dequantize(w2q, w2s), 1, 2)[0]
        Yg = host64(L.ws_view(B.MOE_ITEM_MX_Y, P * d, torch.bfloat16)).reshape(P, d)[rows]
        errs = dict(H=relF(Hg, H), A=relF(Ag, A), Y=relF(Yg, Y))
        print(name, int(e), s1 - s0, {k: f"{v:.2e}" for k, v in errs.items()})
        assert all(v <= TOL for v in errs.values()), errs


BWD_CASES = [CASES[0] + (0,), CASES[1] + (0,), CASES[3] + (0,),
             # the bf16 kernels on 128-row tiles (their dH GEMM has another
             # column tile than the MXFP8 dH GEMM, so the dS partial count
             # the aggregation reads must follow the kernel launched)
             CASES[0] + (B.MOE_FLAG_GEMM_128,)]


@pytest.mark.parametrize("w,mode,tile,flags", BWD_CASES,
                         ids=[c[0].name + ("-gemm128" if c[3] else "") for c in BWD_CASES])
def test_mxfp8_backward_matches_oracle(w, mode, tile, flags):
    """moe_bwd_mxfp8 after the bf16 forward: dO, W2, dH and W1 codes
    bit-exact (dH quantized from the GPU's own bf16 dH through the oracle's
    quantizer), dH / A_s / dS and the weight and router gradients against the
    oracle's MXFP8 backward, dXt / dX against the oracle on the GPU's dH
    codes, and dX end to end against the oracle's own quantization."""
    a = I.draw_all(w)
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, "bf16", round_mode=mode, round_seed=3, tile=tile, flags=flags)
    L = B.Layer(desc)
    X, WR, W1, W2, DO = (dev(a[k], "bf16") for k in ("x", "w_r", "w1", "w2", "d_o"))
    L.route(X, WR)
    L.forward(X, W1, W2)
    L.backward_mxfp8(X, WR, W1, W2, DO)
    torch.cuda.synchronize()
    x64, wr64 = O.to_f64(a["x"], "bf16"), O.to_f64(a["w_r"], "bf16")
    w1_64, w2_64 = O.to_f64(a["w1"], "bf16"), O.to_f64(a["w2"], "bf16")
    rt = O.route(x64, wr64, None, w.K, tile, mode, 3)
    assert_routing_equal(routing_host(L, w), rt)
    fwd = O.forward(x64, w1_64, w2_64, rt)
    dO = O.to_f64(a["d_o"], "bf16")
    o = M.backward_mxfp8(x64, wr64, w1_64, w2_64, rt, M.bf16_round(fwd["H"]), dO)
    d, E, n, P = w.d, w.E, w.n, rt["n_rows"]
    T = w.T
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_DOQ, T * d).reshape(T, d), o["dOq"])
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_DOS, T * d // 32).reshape(T, d // 32), o["dOs"])
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_W2RQ, E * n * d).reshape(E, n, d), o["w2rq"])
    assert np.array_equal(blocked_to_rows(u8(L, B.MOE_ITEM_MX_W2RS, E * d // 32 * n), E, d, n), o["w2rs"])
    dH_gpu = host64(L.ws_view(B.MOE_ITEM_DH, P * 2 * n, torch.bfloat16, mx_bwd=True)).reshape(P, 2 * n)
    dhq, dhs = M.quantize(dH_gpu)
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_DHQ, P * 2 * n).reshape(P, 2 * n), dhq)
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_DHS, P * 2 * n // 32).reshape(P, 2 * n // 32), dhs)
    assert np.array_equal(u8(L, B.MOE_ITEM_MX_W1RQ, E * d * 2 * n).reshape(E, d, 2 * n), o["w1rq"])
    assert np.array_equal(blocked_to_rows(u8(L, B.MOE_ITEM_MX_W1RS, E * 2 * n // 32 * d), E, 2 * n, d), o["w1rs"])
    ref = M.dxt_from_codes(dhq, dhs, o["w1rq"], o["w1rs"], rt, o["dz"], wr64)
    dXt_gpu = host64(L.ws_view(B.MOE_ITEM_DXT, P * d, torch.bfloat16, mx_bwd=True)).reshape(P, d)
    dXt_ref = dxt_with_router_term(ref["dXt"], o["dz"][rt["row_token"], rt["row_expert"]], wr64, rt["row_expert"])
    errs = dict(dH=relF(dH_gpu, o["dH"]), dXt=relF(dXt_gpu, dXt_ref), dX=relF(host64(L.dx), ref["dX"]),
                dW1=relF(host64(L.dw1), o["dW1"]), dW2=relF(host64(L.dw2), o["dW2"]),
                dWr=relF(host64(L.dw_r), o["dWr"]), dS=relF(host64(L.ds[:P]), o["dS"]))
    e2e = relF(host64(L.dx), o["dX"])
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()}, f"dX vs independent oracle {e2e:.2e}")
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, bad
    assert e2e <= E2E_TOL


@pytest.mark.parametrize("name", ["fg7b_bf16", "olmoe_bf16"])
def test_mxfp8_backward_full_size_expert_sample(name):
    """Full size: for two sampled experts, dH and W1 codes bit-exact and their
    dXt rows against the oracle on those codes."""
    w = I.WORKLOADS[name]
    a = I.draw_all(w)
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, "bf16")
    L = B.Layer(desc)
    X, WR, W1, W2, DO = (dev(a[k], "bf16") for k in ("x", "w_r", "w1", "w2", "d_o"))
    L.route(X, WR)
    L.forward(X, W1, W2)
    L.backward_mxfp8(X, WR, W1, W2, DO)
    torch.cuda.synchronize()
    d, E, n = w.d, w.E, w.n
    off = host_int(L.routing.offsets)
    P = int(off[-1])
    dH_all = L.ws_view(B.MOE_ITEM_DH, P * 2 * n, torch.bfloat16, mx_bwd=True).view(P, 2 * n)
    dhq_all = L.ws_view(B.MOE_ITEM_MX_DHQ, P * 2 * n, torch.uint8).view(P, 2 * n)
    w1q_all = L.ws_view(B.MOE_ITEM_MX_W1RQ, E * d * 2 * n, torch.uint8).view(E, d, 2 * n)
    w1s_all = blocked_to_rows(u8(L, B.MOE_ITEM_MX_W1RS, E * 2 * n // 32 * d), E, 2 * n, d)
    dXt_all = L.ws_view(B.MOE_ITEM_DXT, P * d, torch.bfloat16, mx_bwd=True).view(P, d)
    dz_all = L.ws_view(B.MOE_ITEM_DZ, P, torch.float32, mx_bwd=True)
    wr64 = O.to_f64(a["w_r"], "bf16")
    for e in np.random.default_rng(7).choice(E, 2, replace=False):
        s0, s1 = int(off[e]), int(off[e + 1])
        dH = host64(dH_all[s0:s1])
        dhq, dhs = M.quantize(dH)
        assert np.array_equal(dhq_all[s0:s1].cpu().numpy(), dhq)
        w1q, w1s = M.quantize(O.to_f64(a["w1"][e], "bf16"))
        assert np.array_equal(w1q_all[e].cpu().numpy(), w1q) and np.array_equal(w1s_all[e], w1s)
        # plus each row's router term, from the GPU's dz (checked on whole tokens elsewhere)
        ref = M.dequantize(dhq, dhs) @ M.dequantize(w1q, w1s).T
        ref = dxt_with_router_term(ref, host64(dz_all[s0:s1]), wr64, np.full(s1 - s0, e))
        err = relF(host64(dXt_all[s0:s1]), ref)
        print(name, int(e), s1 - s0, f"dXt {err:.2e}")
        assert err <= TOL


WG_CASES = [CASES[0] + (0,), CASES[1] + (0,), CASES[3] + (0,),
            # with the bf16 kernels on 128-row tiles elsewhere in the layer
            CASES[0] + (B.MOE_FLAG_GEMM_128,)]
WG_E2E = 0.08      # MX dW against the plain bf16-operand product (E4M3 on both operands)


def seg_scales(sblk_u8, pe, kp, C):
    """stage-blocked segment scales -> [C, kp / 32] for the expert at padded row pe"""
    s = sblk_u8.reshape(-1, C, 4)[pe // 128:(pe + kp) // 128]
    return s.transpose(1, 0, 2).reshape(C, kp // 32)


def pad128(rows):
    r = rows.shape[0]
    return np.concatenate([rows, np.zeros(((-r) % 128, rows.shape[1]))], axis=0)


def mx_wgrad_layer(w, mode=0, tile=128, flags=0):
    a = I.draw_all(w)
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, "bf16", round_mode=mode, round_seed=3, tile=tile,
                       flags=B.MOE_FLAG_MXFP8_WGRAD | flags)
    L = B.Layer(desc)
    X, WR, W1, W2, DO = (dev(a[k], "bf16") for k in ("x", "w_r", "w1", "w2", "d_o"))
    L.route(X, WR)
    L.forward(X, W1, W2)
    L.backward_mxfp8(X, WR, W1, W2, DO)
    torch.cuda.synchronize()
    return a, L


def check_expert_wgrad(L, w, a, e, off, padoff, dH_all, As_all, wsq, x_rows=None):
    """One expert: its four segment operands' codes and scales bit-exact
    against the oracle's quantization of the same rows (x and dO gathered,
    dH and A_s as the GPU's dH kernel wrote them), and dW1[e], dW2[e] against
    the oracle's product of those codes.  Returns the relative errors."""
    d, n = w.d, w.n
    s0, s1 = int(off[e]), int(off[e + 1])
    pe, kp = int(padoff[e]), int(padoff[e + 1]) - int(padoff[e])
    assert kp == (s1 - s0 + 127) // 128 * 128
    tok = host_int(L.routing.row_token[s0:s1])
    x64 = O.to_f64(a["x"][tok], "bf16")
    dO = O.to_f64(a["d_o"][tok], "bf16")
    dH = host64(dH_all[s0:s1])
    As = host64(As_all[s0:s1])
    got = {}
    for key, rows, C in (("x", x64, d), ("h", dH, 2 * n), ("a", As, n), ("o", dO, d)):
        q_ref, s_ref = M.quantize_segment(pad128(rows))
        q_all, s_all = wsq[key]
        gq = q_all[C * pe:C * (pe + kp)].cpu().numpy().reshape(C, kp)
        gs = seg_scales(s_all, pe, kp, C)
        assert np.array_equal(gq, q_ref), (key, e)
        assert np.array_equal(gs, s_ref), (key, e)
        got[key] = M.dequantize(q_ref, s_ref)
    ref1 = got["x"] @ got["h"].T
    ref2 = got["a"] @ got["o"].T
    g1, g2 = host64(L.dw1[e]), host64(L.dw2[e])
    if s1 == s0:
        assert not g1.any() and not g2.any()
        return dict(dW1=0.0, dW2=0.0), None
    plain = (x64.T @ dH, As.T @ dO)
    return (dict(dW1=relF(g1, ref1), dW2=relF(g2, ref2)),
            dict(dW1=relF(g1, plain[0]), dW2=relF(g2, plain[1])))


def wgrad_views(L, w):
    d, n = w.d, w.n
    off = host_int(L.routing.offsets)
    P = int(off[-1])
    padoff = L.ws_view(B.MOE_ITEM_MX_WG_PADOFF, w.E + 1, torch.int32).cpu().numpy()
    rows = int(padoff[-1])
    wsq = {}
    for key, qi, si, C in (("x", B.MOE_ITEM_MX_WG_XQ, B.MOE_ITEM_MX_WG_XS, d),
                           ("h", B.MOE_ITEM_MX_WG_HQ, B.MOE_ITEM_MX_WG_HS, 2 * n),
                           ("a", B.MOE_ITEM_MX_WG_AQ, B.MOE_ITEM_MX_WG_AS, n),
                           ("o", B.MOE_ITEM_MX_WG_OQ, B.MOE_ITEM_MX_WG_OS, d)):
        wsq[key] = (L.ws_view(qi, C * rows, torch.uint8), u8(L, si, C * rows // 32))
    dH_all = L.ws_view(B.MOE_ITEM_DH, P * 2 * n, torch.bfloat16, mx_bwd=True).view(P, 2 * n)
    As_all = L.ws_view(B.MOE_ITEM_AS, P * n, torch.bfloat16, mx_bwd=True).view(P, n)
    return off, padoff, dH_all, As_all, wsq


@pytest.mark.parametrize("w,mode,tile,flags", WG_CASES,
                         ids=[c[0].name + ("-gemm128" if c[3] else "") for c in WG_CASES])
def test_mxfp8_weight_grads_match_oracle(w, mode, tile, flags):
    """moe_bwd_mxfp8 with MOE_FLAG_MXFP8_WGRAD, every expert: padded segment
    offsets exact, the segment operands' codes and scales bit-exact, dW1 / dW2
    against the oracle on those codes (empty experts exactly zero), the whole
    dW1 / dW2 against the oracle's weight_grads_mxfp8 on the GPU's dH and A_s,
    the rest of the backward as without the flag, and every dW against the
    plain product within the MX quantization bound."""
    a, L = mx_wgrad_layer(w, mode, tile, flags)
    off, padoff, dH_all, As_all, wsq = wgrad_views(L, w)
    cnt = np.diff(off)
    assert np.array_equal(padoff, np.concatenate([[0], np.cumsum((cnt + 127) // 128 * 128)]))
    worst, worst_e2e = {}, {}
    for e in range(w.E):
        errs, e2e = check_expert_wgrad(L, w, a, e, off, padoff, dH_all, As_all, wsq)
        for k, v in errs.items():
            worst[k] = max(worst.get(k, 0.0), v)
        for k, v in (e2e or {}).items():
            worst_e2e[k] = max(worst_e2e.get(k, 0.0), v)
    # whole tensors against the oracle's own weight-gradient routine
    x64 = O.to_f64(a["x"], "bf16")
    dO = O.to_f64(a["d_o"], "bf16")
    rt = dict(offsets=off, row_token=host_int(L.routing.row_token[:int(off[-1])]))
    o = M.weight_grads_mxfp8(x64, dO, rt, host64(dH_all), host64(As_all))
    whole = dict(dW1=relF(host64(L.dw1), o["dW1"]), dW2=relF(host64(L.dw2), o["dW2"]))
    print(w.name, "per expert", {k: f"{v:.2e}" for k, v in worst.items()},
          "whole", {k: f"{v:.2e}" for k, v in whole.items()},
          "vs plain", {k: f"{v:.2e}" for k, v in worst_e2e.items()})
    assert all(v <= TOL for v in worst.values()), worst
    assert all(v <= TOL for v in whole.values()), whole
    assert all(v <= WG_E2E for v in worst_e2e.values()), worst_e2e


def test_mxfp8_weight_grad_flag_leaves_the_rest_unchanged():
    """The flag changes dW1 / dW2 only: dX, dW_r, dS, db bit-identical to
    moe_bwd_mxfp8 without it on the same inputs."""
    w = CASES[0][0]
    a, L1 = mx_wgrad_layer(w)
    desc = B.make_desc(w.T, w.d, w.E, w.n, w.K, "bf16", round_seed=3)
    L2 = B.Layer(desc)
    X, WR, W1, W2, DO = (dev(a[k], "bf16") for k in ("x", "w_r", "w1", "w2", "d_o"))
    L2.route(X, WR)
    L2.forward(X, W1, W2)
    L2.backward_mxfp8(X, WR, W1, W2, DO)
    torch.cuda.synchronize()
    P = int(host_int(L1.routing.offsets)[-1])
    assert torch.equal(L1.dx, L2.dx) and torch.equal(L1.dw_r, L2.dw_r)
    assert torch.equal(L1.ds[:P], L2.ds[:P]) and torch.equal(L1.db, L2.db)


@pytest.mark.parametrize("name", ["fg7b_bf16", "olmoe_bf16"])
def test_mxfp8_weight_grads_full_size_expert_sample(name):
    """Full size, the benchmark's launch configuration with the flag: padded
    offsets exact and, for three sampled experts, every segment operand's
    codes and scales bit-exact and dW1[e] / dW2[e] against the oracle on
    those codes."""
    w = I.WORKLOADS[name]
    a, L = mx_wgrad_layer(w)
    off, padoff, dH_all, As_all, wsq = wgrad_views(L, w)
    cnt = np.diff(off)
    assert np.array_equal(padoff, np.concatenate([[0], np.cumsum((cnt + 127) // 128 * 128)]))
    for e in np.random.default_rng(11).choice(w.E, 3, replace=False):
        errs, e2e = check_expert_wgrad(L, w, a, int(e), off, padoff, dH_all, As_all, wsq)
        print(name, int(e), int(cnt[e]), {k: f"{v:.2e}" for k, v in errs.items()},
              "vs plain", {k: f"{v:.2e}" for k, v in (e2e or {}).items()})
        assert all(v <= TOL for v in errs.values()), errs
        assert all(v <= WG_E2E for v in (e2e or {}).values()), e2e


def bf16_pattern_blocks(seed=31):
    """Every finite bf16 bit pattern below 2^61 (zeros and subnormals too),
    shuffled into blocks of 32, each with one anchor 2^0 .. 2^12 times the
    block's largest magnitude (so the block scale sends its values to every
    code range: saturation, normal, subnormal, zero); rows of 256."""
    rng = np.random.default_rng(seed)
    p = np.arange(1 << 16, dtype=np.uint32)
    p = p[((p >> 7) & 0xFF) <= 127 + 60]
    p = rng.permutation(p)
    nb = (len(p) + 30) // 31
    p = np.concatenate([p, np.zeros(nb * 31 - len(p), dtype=np.uint32)]).reshape(nb, 31)
    ex = (p >> 7) & 0xFF
    emax = ex.max(axis=1)
    aexp = np.where(emax == 0, rng.integers(1, 21, nb), np.minimum(254, emax + rng.integers(0, 13, nb)))
    anchor = (rng.integers(0, 2, nb).astype(np.uint32) << 15) | (aexp.astype(np.uint32) << 7) | \
        rng.integers(0, 128, nb).astype(np.uint32)
    blocks = np.empty((nb, 32), dtype=np.uint32)
    pos = rng.integers(0, 32, nb)
    for b in range(nb):
        blocks[b] = np.insert(p[b], pos[b], anchor[b])
    flat = blocks.reshape(-1)
    rows = (len(flat) + 255) // 256
    flat = np.concatenate([flat, np.zeros(rows * 256 - len(flat), dtype=np.uint32)])
    return flat.astype(np.uint16).reshape(rows, 256)


def test_mxfp8_codes_of_every_bf16_pattern():
    """The quantizer's element codes and block scales, bit-exact against the
    oracle's encoder, on every finite bf16 pattern below 2^61 placed in
    blocks that send it to every code range (moe_fwd_mxfp8's x codes)."""
    x = bf16_pattern_blocks()
    T, d = x.shape
    w = W("patterns", T, d, 8, 256, 2, seed=32)
    a = I.draw_all(w)
    a["x"] = x
    L, _ = run_mx(w, a)
    xq, xs = M.quantize(O.to_f64(x, "bf16"))
    gq = u8(L, B.MOE_ITEM_MX_XQ, T * d).reshape(T, d)
    gs = u8(L, B.MOE_ITEM_MX_XS, T * d // 32).reshape(T, d // 32)
    bad = np.nonzero(gq != xq)
    assert np.array_equal(gs, xs), "scales"
    assert bad[0].size == 0, [(hex(int(x[i, j])), hex(int(gq[i, j])), hex(int(xq[i, j]))) for i, j in zip(*bad)][:10]
