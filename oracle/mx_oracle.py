"""fp64 CPU oracle of the MoE layer's forward with MXFP8 grouped GEMMs.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the tests use it.  It shares no code with the HIP path.

Sources.  The pages name MXFP8 (and FP4) as the method's next precision step
and say no more ([A] closing "未来展望" paragraph of "DeepSeek做大→Mega MoE，
Tri Dao团队加快→SonicMoE"); the format itself is the OCP Microscaling (MX)
Formats specification v1.0 (section 5: MX block of 32 elements sharing one
E8M0 scale; section 6.3: converting a block of higher-precision values) and
the OCP 8-bit floating point specification (E4M3: bias 7, no infinities,
S.1111.111 the only NaN, largest finite 448).  Readings taken where the
specification leaves a choice:

  * element type E4M3 (the "MXFP8" the pages name; E5M2 is the other MX
    8-bit type and is not used);
  * shared exponent = floor(log2(amax of the block)) - 8, 8 being the E4M3
    exponent of its largest normal (448 = 1.75 * 2^8), clamped to E8M0's
    finite range; a block of zeros gets scale code 0 and zero elements;
  * elements are v / 2^shared rounded to nearest, ties to even, and values
    beyond 448 in magnitude saturate to +-448 (the specification leaves
    overflow to the implementation; saturation keeps the block finite);
  * blocks run along the reduction (k) axis of each GEMM: x rows along d,
    W1 along d (each column of an expert's [d, 2n] matrix), the SwiGLU
    output A rows along n, W2 along n;
  * A is quantized from its bf16 value, the precision the forward stores it
    in; H is returned in fp64 (the kernels store it in bf16 as in the plain
    layer);
  * in the backward, the activation-gradient GEMMs take MXFP8 operands:
    dA' = dO W2^T with dO and W2 quantized along d (W2 by the rows of each
    expert's [n, d] matrix), dXt = dH W1^T with dH quantized along 2n from
    its bf16 value and W1 along 2n (rows of each expert's [d, 2n] matrix);
  * the weight-gradient GEMMs reduce over an expert's rows, so their blocks
    run along the rows of each expert's segment: block b of expert e holds
    segment rows 32 b .. 32 b + 31 (counted from the segment's first row,
    so no block holds rows of two experts), the last block of a segment
    zero-padded (zeros change no block maximum and add nothing to a sum);
    dW1[e] = X_g^T dH with X_g (the expert's gathered x rows) and dH (from
    its bf16 value) quantized that way, dW2[e] = A_s^T dO_g with A_s (the
    gate-scaled A, from its bf16 value) and dO_g likewise.

The forward itself is the plain layer forward (moe_oracle.forward) on the
dequantized operands: H = deq(x_q)[tok] deq(W1_q), A = silu(G) * U,
Y = deq(A_q) deq(W2_q), O = sum over a token's rows of gate * Y.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O

BLOCK = 32
E4M3_EMAX = 8          # exponent of 448 = 1.75 * 2^8
E4M3_MAX = 448.0
E8M0_BIAS = 127


# ----------------------------------------------------------------------------
# E4M3 elements (OCP 8-bit floating point specification)
# ----------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), magnitudes
    beyond 448 saturating to 448.  Zero and negative zero map to 0x00 / 0x80
    by the sign bit of the value."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    out = np.zeros(a.shape, dtype=np.int64)
    # normal range: a >= 2^-6, exponent E in [-6, 8], 3 fraction bits
    normal = a >= 2.0 ** -6
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(normal, a, 1.0))).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    E = np.where(np.exp2(E.astype(np.float64)) > a, E - 1, E)
    E = np.where(np.exp2(E.astype(np.float64) + 1) <= a, E + 1, E)
    m = np.rint(a / np.exp2(E.astype(np.float64)) * 8.0).astype(np.int64)  # 8..16, ties to even
    carry = m == 16
    E = np.where(carry, E + 1, E)
    m = np.where(carry, 8, m)
    out = np.where(normal, ((E + 7) << 3) | (m - 8), out)
    # subnormals and zero: multiples of 2^-9; rounding up to 8 gives the
    # smallest normal (code 0x08), which the same formula produces
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    out = np.where(normal, out, sub)
    out = np.where(neg, out | 0x80, out)
    return out.astype(np.uint8)


# ----------------------------------------------------------------------------
# MX blocks (OCP MX specification, sections 5 and 6.3)
# ----------------------------------------------------------------------------

def shared_exponent(amax) -> np.ndarray:
    """E8M0 code of the block scale: floor(log2 amax) - 8 + 127, clamped to
    0..254; 0 for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(pos, amax, 1.0))).astype(np.int64)
    e = np.where(np.exp2(e.astype(np.float64)) > amax, e - 1, e)
    e = np.where(pos & (np.exp2(e.astype(np.float64) + 1) <= amax), e + 1, e)
    code = np.clip(e - E4M3_EMAX + E8M0_BIAS, 0, 254)
    return np.where(pos, code, 0).astype(np.uint8)


def quantize(v) -> tuple:
    """MXFP8 quantization along the last axis (length a multiple of 32):
    returns (codes uint8 of v's shape, scale codes uint8 [..., L/32])."""
    v = np.asarray(v, dtype=np.float64)
    L = v.shape[-1]
    assert L % BLOCK == 0, "block length"
    b = v.reshape(v.shape[:-1] + (L // BLOCK, BLOCK))
    sc = shared_exponent(np.abs(b).max(axis=-1))
    scale = np.exp2(sc.astype(np.float64) - E8M0_BIAS)
    q = e4m3_encode(b / scale[..., None])
    q = np.where((sc == 0)[..., None] & (np.abs(b).max(axis=-1) == 0)[..., None], np.uint8(0), q)
    return q.reshape(v.shape).astype(np.uint8), sc


def dequantize(q, sc) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8)
    L = q.shape[-1]
    vals = e4m3_decode(q).reshape(q.shape[:-1] + (L // BLOCK, BLOCK))
    scale = np.exp2(np.asarray(sc, dtype=np.float64) - E8M0_BIAS)
    return (vals * scale[..., None]).reshape(q.shape)


def bf16_round(v) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each float64 value, as float64."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# operands of the two forward GEMMs, quantized along their reductions
# ----------------------------------------------------------------------------

def quantize_rows(x64) -> tuple:
    """x [T, d] along d: (codes [T, d], scales [T, d/32])."""
    return quantize(x64)


def quantize_weights(w64) -> tuple:
    """An expert weight stack w [E, K, N] along K, returned k-contiguous:
    (codes [E, N, K], scales [E, N, K/32]) of w[e]^T."""
    return quantize(np.swapaxes(w64, 1, 2))


def forward_mxfp8(x64, w1_64, w2_64, rt) -> dict:
    """The layer forward with MXFP8 GEMM operands (routing rt as given)."""
    xq, xs = quantize_rows(x64)
    w1q, w1s = quantize_weights(w1_64)
    w2q, w2s = quantize_weights(w2_64)
    xd = dequantize(xq, xs)
    w1d = np.swapaxes(dequantize(w1q, w1s), 1, 2)   # [E, d, 2n]
    w2d = np.swapaxes(dequantize(w2q, w2s), 1, 2)   # [E, n, d]
    T = x64.shape[0]
    E, d, n2 = w1_64.shape
    n = n2 // 2
    P = rt["n_rows"]
    off, tok = rt["offsets"], rt["row_token"]
    H = np.zeros((P, 2 * n))
    A = np.zeros((P, n))
    Aq = np.zeros((P, n), dtype=np.uint8)
    As = np.zeros((P, n // BLOCK), dtype=np.uint8)
    Y = np.zeros((P, d))
    for e in range(E):
        s, t = off[e], off[e + 1]
        if s == t:
            continue
        H[s:t] = xd[tok[s:t]] @ w1d[e]
        A[s:t] = O.silu(H[s:t, :n]) * H[s:t, n:]
        Aq[s:t], As[s:t] = quantize(bf16_round(A[s:t]))
        Y[s:t] = dequantize(Aq[s:t], As[s:t]) @ w2d[e]
    Out = np.zeros((T, d))
    np.add.at(Out, tok, rt["row_gate"][:, None] * Y)
    return dict(H=H, A=A, Y=Y, O=Out, xq=xq, xs=xs, w1q=w1q, w1s=w1s, w2q=w2q, w2s=w2s, Aq=Aq, As=As)


def backward_mxfp8(x64, wr64, w1_64, w2_64, rt, H, dO) -> dict:
    """The backward with both activation-gradient GEMMs on MXFP8 operands:
    dA' = dO W2^T with dO quantized along d and each expert's W2 quantized
    along d (rows of its [n, d] matrix), and dXt = dH W1^T with dH quantized
    along 2n from its bf16 value and W1 along 2n.  The dH epilogue (A
    recomputed from H, dS, the SwiGLU backward, A_s) and the weight and router
    gradients follow the plain backward (moe_oracle.backward) from that dA':
    dW1 = X_g^T dH, dW2 = A^T (gate dO_g) with the unquantized dO."""
    T, d = x64.shape
    E = w1_64.shape[0]
    n = w1_64.shape[2] // 2
    P = rt["n_rows"]
    off, tok, rg = rt["offsets"], rt["row_token"], rt["row_gate"]
    dOq, dOs = quantize(dO)                          # [T, d] along d
    w2q, w2s = quantize(w2_64)                       # [E, n, d] along d
    dOd = dequantize(dOq, dOs)
    w2d = dequantize(w2q, w2s)
    dAp = np.zeros((P, n))
    dS = np.zeros(P)
    dH = np.zeros((P, 2 * n))
    dW1 = np.zeros_like(w1_64)
    dW2 = np.zeros_like(w2_64)
    for e in range(E):
        s, t = off[e], off[e + 1]
        if s == t:
            continue
        G, U = H[s:t, :n], H[s:t, n:]
        sg = O.sigmoid(G)
        A = G * sg * U
        dAp[s:t] = dOd[tok[s:t]] @ w2d[e].T
        dS[s:t] = np.sum(dAp[s:t] * A, axis=1)
        dA = rg[s:t, None] * dAp[s:t]
        dH[s:t, :n] = dA * U * sg * (1.0 + G * (1.0 - sg))
        dH[s:t, n:] = dA * G * sg
        dW1[e] = x64[tok[s:t]].T @ dH[s:t]
        dW2[e] = A.T @ (rg[s:t, None] * dO[tok[s:t]])
    # router: softmax-over-set backward per token, as in the plain backward
    dSte = np.zeros((T, E))
    dSte[tok, rt["row_expert"]] = dS
    Gt = rt["gate"]
    mean = np.sum(Gt * dSte, axis=1, keepdims=True)
    dz = np.where(rt["member"], Gt * (dSte - mean), 0.0)
    dHq, dHs = quantize(bf16_round(dH))
    w1q, w1s = quantize(w1_64)                       # [E, d, 2n] along 2n
    out = dict(dAp=dAp, dS=dS, dH=dH, dW1=dW1, dW2=dW2, dz=dz, dWr=x64.T @ dz, db=dz.sum(axis=0),
               dOq=dOq, dOs=dOs, w2rq=w2q, w2rs=w2s, dHq=dHq, dHs=dHs, w1rq=w1q, w1rs=w1s)
    out.update(dxt_from_codes(dHq, dHs, w1q, w1s, rt, dz, wr64))
    return out


def dxt_from_codes(dHq, dHs, w1q, w1s, rt, dz, wr64) -> dict:
    """dXt per row from the quantized dH rows and W1 rows, and the dX it
    aggregates to (plus the router's dz W_r^T)."""
    off, tok = rt["offsets"], rt["row_token"]
    dHd = dequantize(dHq, dHs)
    w1d = dequantize(w1q, w1s)                       # [E, d, 2n]
    E, d = w1d.shape[0], w1d.shape[1]
    dXt = np.zeros((dHd.shape[0], d))
    for e in range(E):
        s, t = off[e], off[e + 1]
        if s < t:
            dXt[s:t] = dHd[s:t] @ w1d[e].T
    dX = dz @ wr64.T
    np.add.at(dX, tok, dXt)
    return dict(dXt=dXt, dX=dX)


# ----------------------------------------------------------------------------
# weight gradients: operands quantized along each expert's segment of rows
# ----------------------------------------------------------------------------

def quantize_segment(rows64) -> tuple:
    """One expert's rows [r, C] quantized along the rows: the matrix is
    transposed to [C, r], zero-padded along the rows to a multiple of 32 and
    quantized in blocks of 32 rows.  Returns (codes [C, r_pad], scales
    [C, r_pad / 32])."""
    v = np.asarray(rows64, dtype=np.float64)
    r, C = v.shape
    pad = (-r) % BLOCK
    vt = np.concatenate([v.T, np.zeros((C, pad))], axis=1)
    return quantize(vt)


def weight_grads_mxfp8(x64, dO, rt, dH, As) -> dict:
    """dW1[e] = X_g^T dH and dW2[e] = A_s^T dO_g with every operand quantized
    along the expert's rows (quantize_segment): X_g = x[row_token] and dO_g =
    dO[row_token] over the expert's segment, dH and A_s (per routed row, in
    the expert-sorted order of rt) from their bf16 values.  Also returns each
    expert's codes and scales (None for an expert without rows)."""
    off, tok = rt["offsets"], rt["row_token"]
    E = len(off) - 1
    d, n2 = x64.shape[1], dH.shape[1]
    n = As.shape[1]
    dW1 = np.zeros((E, d, n2))
    dW2 = np.zeros((E, n, d))
    codes = []
    for e in range(E):
        s, t = off[e], off[e + 1]
        if s == t:
            codes.append(None)
            continue
        xq, xs = quantize_segment(x64[tok[s:t]])
        hq, hs = quantize_segment(bf16_round(dH[s:t]))
        aq, as_ = quantize_segment(bf16_round(As[s:t]))
        oq, os_ = quantize_segment(dO[tok[s:t]])
        dW1[e] = dequantize(xq, xs) @ dequantize(hq, hs).T
        dW2[e] = dequantize(aq, as_) @ dequantize(oq, os_).T
        codes.append(dict(xq=xq, xs=xs, hq=hq, hs=hs, aq=aq, as_=as_, oq=oq, os=os_))
    return dict(dW1=dW1, dW2=dW2, codes=codes)


def layer_fwd_mxfp8(x, w_r, w1, w2, K, bias=None, tile=128, round_mode=0, round_seed=0) -> dict:
    """Route (as the plain layer) and run the MXFP8 forward from raw bf16
    inputs (uint16 bit patterns)."""
    x64, wr64 = O.to_f64(x, "bf16"), O.to_f64(w_r, "bf16")
    w1_64, w2_64 = O.to_f64(w1, "bf16"), O.to_f64(w2, "bf16")
    rt = O.route(x64, wr64, bias, K, tile, round_mode, round_seed)
    out = dict(rt)
    out.update(forward_mxfp8(x64, w1_64, w2_64, rt))
    return out
