"""Pins of the MXFP8 oracle (CPU): the E4M3 element codec against torch's
float8_e4m3fn conversion and against an exhaustive nearest-code search, the
format's fixed encodings, the MX block invariants (scale range, idempotence,
power-of-two equivariance, error bound, zero blocks), and the forward on
inputs that MXFP8 represents exactly, where it must equal the plain forward."""
import numpy as np
import pytest
import torch

from fine_grained_mixture_top_amd import inputs as I
from oracle import moe_oracle as O
from oracle import mx_oracle as M

ALL = np.arange(256, dtype=np.uint8)


def torch_e4m3(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def finite_values():
    vals = M.e4m3_decode(ALL)
    ok = ~np.isnan(vals)
    return ALL[ok], vals[ok]


def test_decode_matches_torch_on_every_code():
    mine = M.e4m3_decode(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])
    assert np.isnan(mine).sum() == 2  # S.1111.111 only


def test_fixed_encodings_of_the_format():
    # largest finite, smallest subnormal, smallest normal, one, a negative
    for v, c in ((448.0, 0x7E), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (1.0, 0x38), (-1.5, 0xBC),
                 (0.0, 0x00), (-0.0, 0x80), (240.0, 0x77), (2.0 ** -7, 0x04)):
        assert int(M.e4m3_encode(np.array([v]))[0]) == c, v


def test_encode_matches_torch_including_ties():
    rng = np.random.default_rng(0)
    _, fin = finite_values()
    fin = np.unique(fin)
    mids = (fin[1:] + fin[:-1]) / 2
    v = np.concatenate([rng.uniform(-448, 448, 50000),
                        rng.uniform(-1, 1, 50000) * 2.0 ** rng.integers(-14, 9, 50000), mids, fin])
    v32 = v.astype(np.float32)
    assert np.array_equal(M.e4m3_encode(v32.astype(np.float64)), torch_e4m3(v32))


def test_encode_is_the_nearest_code_ties_to_even():
    codes, vals = finite_values()
    rng = np.random.default_rng(1)
    _, fin = finite_values()
    fin = np.unique(fin)
    v = np.concatenate([rng.uniform(-448, 448, 3000), (fin[1:] + fin[:-1])[::3] / 2,
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000)])
    got = M.e4m3_encode(v)
    for x, c in zip(v, got):
        dist = np.abs(vals - x)
        best = np.nonzero(dist == dist.min())[0]
        # same sign as x among equal magnitudes (zero keeps the sign of x)
        cand = [int(codes[i]) for i in best if (codes[i] >> 7) == (1 if np.signbit(x) else 0) or vals[i] != 0]
        cand = [k for k in cand if (k >> 7) == (1 if np.signbit(x) else 0)] or cand
        if len(cand) > 1:
            cand = [k for k in cand if k & 1 == 0]
        assert int(c) in cand, (x, int(c), cand)


def test_saturation_beyond_448():
    v = np.array([448.0001, 464.0, 479.99, 500.0, 511.99, -470.0, 1e6])
    assert list(M.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E]


def rand_blocks(seed, nblk=400):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((nblk, 32)) * 2.0 ** rng.integers(-20, 20, (nblk, 1))
    v[::7, 3] *= 300.0  # outliers
    return v


def test_block_scale_puts_the_max_in_256_512():
    v = rand_blocks(2)
    q, sc = M.quantize(v)
    amax = np.abs(v).max(axis=1)
    r = amax / np.exp2(sc[:, 0].astype(np.float64) - 127)
    assert np.all((r >= 256) & (r < 512))


def test_quantize_of_dequantized_is_identity():
    v = rand_blocks(3)
    q, sc = M.quantize(v)
    q2, sc2 = M.quantize(M.dequantize(q, sc))
    assert np.array_equal(sc, sc2)
    assert np.array_equal(q, q2)


def test_power_of_two_equivariance():
    v = rand_blocks(4)
    q, sc = M.quantize(v)
    for j in (-5, 1, 7):
        q2, sc2 = M.quantize(v * 2.0 ** j)
        assert np.array_equal(q, q2)
        assert np.array_equal(sc2.astype(int), sc.astype(int) + j)


def test_error_bound_per_element():
    v = rand_blocks(5)
    q, sc = M.quantize(v)
    d = M.dequantize(q, sc)
    s = np.exp2(sc.astype(np.float64) - 127)  # [blocks, 1]
    a = np.abs(v) / s
    sat = a > 448
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_ulp = np.exp2(e - 4) * s  # 3 fraction bits: ulp = 2^(e-3)
    err = np.abs(d - v)
    assert np.all(err[~sat] <= half_ulp[~sat] * (1 + 1e-12))
    assert np.all(np.abs(d[sat]) == 448 * np.broadcast_to(s, d.shape)[sat])


def test_zero_blocks_and_row_axis():
    v = np.zeros((3, 64))
    v[1, 40] = -3.0
    q, sc = M.quantize(v)
    assert sc.shape == (3, 2)
    assert list(sc[0]) == [0, 0] and sc[1, 0] == 0 and sc[1, 1] == 1 - 8 + 127
    assert np.all(q[0] == 0) and np.all(q[1, :32] == 0)
    assert M.dequantize(q, sc)[1, 40] == -3.0


def test_weights_are_quantized_along_k_and_transposed():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((2, 64, 96))  # [E, K, N]
    q, sc = M.quantize_weights(w)
    assert q.shape == (2, 96, 64) and sc.shape == (2, 96, 2)
    for e in range(2):
        for col in (0, 5, 95):
            qc, sc_c = M.quantize(w[e, :, col][None, :])
            assert np.array_equal(q[e, col], qc[0]) and np.array_equal(sc[e, col], sc_c[0])


def test_bf16_round():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -9])
    assert list(M.bf16_round(v)) == [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 1.0]


def exact_inputs(T, d, E, n, K, seed):
    """Integer-valued x, W1, W2 in [-14, 14] with an element of magnitude >= 8
    in every 32-block along the reductions: MXFP8 represents them exactly."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-7, 8, (T, d)).astype(np.float64)
    x[:, ::32] = 8 + rng.integers(0, 7, (T, d // 32))
    w1 = rng.integers(-7, 8, (E, d, 2 * n)).astype(np.float64)
    w1[:, ::32, :] = -(8 + rng.integers(0, 7, (E, d // 32, 2 * n)))
    w2 = rng.integers(-7, 8, (E, n, d)).astype(np.float64)
    w2[:, ::32, :] = 9
    # keep the SwiGLU inputs moderate: scale the weights by powers of two
    return x, w1 / 64.0, w2 / 64.0


@pytest.mark.parametrize("seed", [0, 1])
def test_forward_equals_plain_forward_on_exact_inputs(seed):
    T, d, E, n, K = 40, 64, 4, 64, 2
    x, w1, w2 = exact_inputs(T, d, E, n, K, seed)
    wr = np.random.default_rng(seed + 10).standard_normal((d, E))
    rt = O.route(x, wr, None, K)
    xq, xs = M.quantize_rows(x)
    assert np.array_equal(M.dequantize(xq, xs), x)
    f = M.forward_mxfp8(x, w1, w2, rt)
    p = O.forward(x, w1, w2, rt)
    assert np.allclose(f["H"], p["H"], rtol=0, atol=1e-12 * np.abs(p["H"]).max())
    assert np.allclose(f["A"], p["A"], rtol=0, atol=1e-12 * np.abs(p["A"]).max())
    # A itself is rounded to MXFP8: Y and O stay within its error
    for k in ("Y", "O"):
        rel = np.linalg.norm(f[k] - p[k]) / np.linalg.norm(p[k])
        assert 0 < rel < 0.05, (k, rel)


def test_forward_on_random_inputs_is_close_to_plain():
    w = I.Workload("mx_small", T=64, d=128, E=8, n=64, K=2, dtype="bf16", seed=4)
    a = I.draw_all(w)
    o = M.layer_fwd_mxfp8(a["x"], a["w_r"], a["w1"], a["w2"], w.K)
    p = O.forward(O.to_f64(a["x"], "bf16"), O.to_f64(a["w1"], "bf16"), O.to_f64(a["w2"], "bf16"), o)
    for k in ("H", "Y", "O"):
        rel = np.linalg.norm(o[k] - p[k]) / np.linalg.norm(p[k])
        assert 1e-3 < rel < 0.08, (k, rel)


def test_backward_on_exact_inputs_equals_plain():
    """dO, W1 and W2 that MXFP8 represents exactly (integer-valued, a large
    element in every 32-block along d and along 2n): dA', dS, dH and every
    weight and router gradient equal the plain backward's, and dXt is the
    plain product of the dequantized dH (whose quantization is then the only
    rounding)."""
    T, d, E, n, K = 40, 64, 4, 64, 2
    x, w1, w2 = exact_inputs(T, d, E, n, K, 3)
    w1 = np.round(w1 * 64.0)
    w1[:, :, ::32] = 11.0
    w1 /= 64.0
    w2 = np.round(w2 * 64.0)
    w2[:, :, ::32] = -12.0          # along d (rows of W2[e]) too
    w2 /= 64.0
    rng = np.random.default_rng(14)
    dO = rng.integers(-7, 8, (T, d)).astype(np.float64)
    dO[:, ::32] = 9.0
    wr = np.random.default_rng(13).standard_normal((d, E))
    rt = O.route(x, wr, None, K)
    H = O.forward(x, w1, w2, rt)["H"]
    b = M.backward_mxfp8(x, wr, w1, w2, rt, H, dO)
    p = O.backward(x, wr, w1, w2, rt, H, dO)
    assert np.array_equal(M.dequantize(b["dOq"], b["dOs"]), dO)
    assert np.array_equal(M.dequantize(b["w2rq"], b["w2rs"]), w2)
    assert np.array_equal(M.dequantize(b["w1rq"], b["w1rs"]), w1)
    for k in ("dAp", "dS", "dH", "dW1", "dW2", "dWr", "dz", "db"):
        assert np.allclose(b[k], p[k], rtol=0, atol=1e-12 * max(1.0, np.abs(p[k]).max())), k
    dHd = M.dequantize(b["dHq"], b["dHs"])
    for e in range(E):
        s0, s1 = rt["offsets"][e], rt["offsets"][e + 1]
        assert np.allclose(b["dXt"][s0:s1], dHd[s0:s1] @ w1[e].T, rtol=0, atol=1e-12)
    rel = np.linalg.norm(b["dX"] - p["dX"]) / np.linalg.norm(p["dX"])
    assert 0 < rel < 0.05


def test_backward_on_random_inputs_is_close_to_plain():
    w = I.Workload("mx_small", T=64, d=128, E=8, n=64, K=2, dtype="bf16", seed=5)
    a = I.draw_all(w)
    x64, wr64 = O.to_f64(a["x"], "bf16"), O.to_f64(a["w_r"], "bf16")
    w1, w2, dO = (O.to_f64(a[k], "bf16") for k in ("w1", "w2", "d_o"))
    rt = O.route(x64, wr64, None, w.K)
    H = O.forward(x64, w1, w2, rt)["H"]
    b = M.backward_mxfp8(x64, wr64, w1, w2, rt, H, dO)
    p = O.backward(x64, wr64, w1, w2, rt, H, dO)
    for k in ("dAp", "dH", "dXt", "dX", "dW1", "dWr"):
        rel = np.linalg.norm(b[k] - p[k]) / np.linalg.norm(p[k])
        assert 1e-3 < rel < 0.08, (k, rel)
    assert np.array_equal(b["dW2"], p["dW2"])  # A and the unquantized dO only


# ----------------------------------------------------------------------------
# weight gradients on operands quantized along each expert's segment of rows
# ----------------------------------------------------------------------------

def exact_rows(rng, shape):
    """Values MXFP8 represents exactly whatever block they fall in: every
    magnitude in {256, 288, ..., 448} (1.0 .. 1.75 times 2^8), so every block
    maximum is in [256, 448], the block scale is 2^0 and each value is its own
    E4M3 code."""
    mag = 256.0 + 32.0 * rng.integers(0, 7, shape)
    return np.where(rng.random(shape) < 0.5, -mag, mag)


def test_segment_quantization_layout_and_padding():
    """A segment of r rows becomes [C, r rounded up to 32]: the first block
    starts at the segment's first row, padding rows are zero codes, a block of
    padding only has scale code 0, and quantizing rows 40.. of a longer array
    as their own segment equals quantizing them alone."""
    rng = np.random.default_rng(21)
    v = rng.standard_normal((100, 6))
    q, s = M.quantize_segment(v[40:77])          # 37 rows -> 64
    assert q.shape == (6, 64) and s.shape == (6, 2)
    q2, s2 = M.quantize(np.concatenate([v[40:77].T, np.zeros((6, 27))], axis=1))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.all(q[:, 37:] == 0)
    # block 0 = rows 40..71 of v, block 1 = rows 72..76 plus zeros
    assert np.array_equal(s[:, 0], M.shared_exponent(np.abs(v[40:72]).max(axis=0)))
    assert np.array_equal(s[:, 1], M.shared_exponent(np.abs(v[72:77]).max(axis=0)))
    qz, sz = M.quantize_segment(np.zeros((3, 4)))
    assert np.all(qz == 0) and np.all(sz == 0)


def test_segment_blocks_follow_the_segment_not_the_global_row_index():
    """With segments [0, 40) and [40, 80) the second segment's blocks are rows
    40..71 and 72..79, not the global blocks 32..63 and 64..95: its codes equal
    those of the same rows quantized with no first segment in front."""
    rng = np.random.default_rng(22)
    T, d, E, n = 80, 64, 2, 32
    x = rng.standard_normal((T, d))
    x[45, 3] = 1000.0                      # a large value in global block 32..63, segment block 0
    rt = dict(offsets=np.array([0, 40, 80]), row_token=np.arange(T))
    dH = rng.standard_normal((T, 2 * n))
    As = rng.standard_normal((T, n))
    dO = rng.standard_normal((T, d))
    w = M.weight_grads_mxfp8(x, dO, rt, dH, As)
    alone = M.weight_grads_mxfp8(x[40:], dO[40:], dict(offsets=np.array([0, 40]), row_token=np.arange(40)),
                                 dH[40:], As[40:])
    for k in ("xq", "xs", "hq", "hs", "aq", "as_", "oq", "os"):
        assert np.array_equal(w["codes"][1][k], alone["codes"][0][k]), k
    assert np.array_equal(w["dW1"][1], alone["dW1"][0]) and np.array_equal(w["dW2"][1], alone["dW2"][0])
    # the large value shares its scale with rows 40..71 of column 3 only
    assert int(w["codes"][1]["xs"][3, 0]) == int(M.shared_exponent(np.array([1000.0]))[0])
    assert int(w["codes"][0]["xs"][3, 1]) == int(M.shared_exponent(np.abs(x[32:40, 3]).max()[None])[0])


def test_weight_grads_equal_plain_products_on_exact_inputs():
    """Operands MXFP8 represents exactly (exact_rows), gathered and ragged
    segments with partial last blocks and an empty expert: dW1 = X_g^T dH and
    dW2 = A_s^T dO_g exactly, dH and A_s entering through their bf16 value
    (exact here too)."""
    rng = np.random.default_rng(23)
    T, d, E, n, K = 70, 64, 5, 32, 2
    x = exact_rows(rng, (T, d))
    dO = exact_rows(rng, (T, d))
    member = np.zeros((T, E), dtype=bool)
    for t in range(T):
        member[t, rng.choice(4, K, replace=False)] = True   # expert 4 stays empty
    rt = O.segments(member, 128)
    P = rt["n_rows"]
    dH = exact_rows(rng, (P, 2 * n))
    As = exact_rows(rng, (P, n))
    w = M.weight_grads_mxfp8(x, dO, rt, dH, As)
    off, tok = rt["offsets"], rt["row_token"]
    assert off[4] == off[5] and w["codes"][4] is None
    assert any((off[e + 1] - off[e]) % 32 for e in range(4))   # partial last blocks occur
    for e in range(E):
        s, t = off[e], off[e + 1]
        assert np.array_equal(w["dW1"][e], x[tok[s:t]].T @ dH[s:t])
        assert np.array_equal(w["dW2"][e], As[s:t].T @ dO[tok[s:t]])


def test_weight_grads_on_random_inputs_are_close_to_plain():
    rng = np.random.default_rng(24)
    T, d, E, n, K = 200, 128, 4, 64, 2
    x, dO = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    member = np.zeros((T, E), dtype=bool)
    for t in range(T):
        member[t, rng.choice(E, K, replace=False)] = True
    rt = O.segments(member, 128)
    P = rt["n_rows"]
    dH, As = rng.standard_normal((P, 2 * n)), rng.standard_normal((P, n))
    w = M.weight_grads_mxfp8(x, dO, rt, dH, As)
    off, tok = rt["offsets"], rt["row_token"]
    for e in range(E):
        s, t = off[e], off[e + 1]
        for k, ref in (("dW1", x[tok[s:t]].T @ dH[s:t]), ("dW2", As[s:t].T @ dO[tok[s:t]])):
            rel = np.linalg.norm(w[k][e] - ref) / np.linalg.norm(ref)
            assert 1e-3 < rel < 0.08, (k, e, rel)
