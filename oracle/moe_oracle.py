"""fp64 CPU oracle of one fine-grained MoE layer (routing, forward, backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the tests, the smoke check of the entry script and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP path.

Sources (web pages about SonicMoE; cited by title and section):
  [A] "DeepSeek做大→Mega MoE，Tri Dao团队加快→SonicMoE" -- news article that
      summarises the authors' Blackwell blog.  Sections used: "MoE 与它的隐患"
      (figure captions of the standard MoE forward / backward workflow, the
      routing metadata pi as a binary mask), "核心创新：一次算法级的重新设计"
      (first point: no cached tensor that scales with expert granularity, via a
      reordered contraction, no extra matmul recompute; second point: gather
      fusion, SwiGLU in the epilogue, the dH kernel).
  [B] "SonicMoE：突破细粒度MoE硬件效率瓶颈，实现高稀疏性下的极致训练加速" --
      summary of the arXiv paper.  Paragraphs used: the algorithm-level
      paragraph (router gradient without caching activations, mathematically
      equivalent to the original MoE), the scheduling paragraph (token
      rounding to multiples of the grouped-GEMM tile, deviation at most one
      tile per expert, total preserved in expectation), and the kernel-list
      paragraph (forward: up-proj A, down-proj Y, aggregation O; backward: dH,
      the up-proj activation gradient, dX aggregation, two weight gradients).

Notation (the pages'): T tokens, d hidden size, n expert intermediate size,
E experts, K experts per token, M grouped-GEMM tile of token rounding.

Everything is computed in float64.  Integer decisions that float values take
(top-K selection, token-rounding rank order) are made on float32 scores, the
precision the kernels decide in; the oracle rounds its own fp64 logits to
float32 for that.  The plain definition written out here is:

  z[t,e]    = sum_i X[t,i] W_r[i,e] + b[e]
  S_t       = K experts with largest z[t,.]  (ties: smaller expert id first)
  gate[t,e] = softmax of z[t,S_t] (e in S_t)
  rows of expert e: its tokens in ascending token id; offsets = exclusive scan
  H_r = X[tok_r] W1[e_r];  G_r = H_r[:n], U_r = H_r[n:];  A_r = silu(G_r)*U_r
  Y_r = A_r W2[e_r];       O_t = sum_{r of t} gate_r Y_r
  dA'_r = dO[tok_r] W2[e_r]^T;  dS_r = <dA'_r, A_r>   (= <dO[tok_r], Y_r>)
  dA_r  = gate_r dA'_r;  dG = dA*U*s*(1+G*(1-s)), dU = dA*silu(G), s = sigmoid(G)
  dH_r  = [dG | dU];  dXt_r = dH_r W1[e_r]^T
  dW1[e] = sum_r X[tok_r]^T dH_r;   dW2[e] = sum_r A_r^T (gate_r dO[tok_r])
  dz[t,e] = gate[t,e] (dS[t,e] - sum_{e' in S_t} gate[t,e'] dS[t,e'])
  dW_r = X^T dz;  db = sum_t dz[t,.];  dX_t = sum_{r of t} dXt_r + dz[t,.] W_r^T

Parity pins (tests/test_oracle_*.py): central finite differences, the naive
activation-caching backward below, dense special cases (E=1,K=1 is a dense
SwiGLU MLP; K=E is a dense softmax mixture), symmetry and invariants, a
brute-force routing checker, hand-worked routing / token-rounding fixtures
under tests/golden/, and the token-rounding invariants.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


# ----------------------------------------------------------------------------
# scalar conversions
# ----------------------------------------------------------------------------

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Input tensor to float64.  bf16 tensors arrive as uint16 bit patterns;
    a bf16 value is the float32 whose upper 16 bits are those bits."""
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def sigmoid(g: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-g))


def silu(g: np.ndarray) -> np.ndarray:
    return g * sigmoid(g)


# ----------------------------------------------------------------------------
# routing  ([A] "MoE 与它的隐患": routing metadata; [B] scheduling paragraph)
# ----------------------------------------------------------------------------

def router_logits(x64: np.ndarray, wr64: np.ndarray, bias=None) -> np.ndarray:
    """z = X W_r (+ b), float64."""
    z = x64 @ wr64
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    return z


def decision_scores(z64: np.ndarray) -> np.ndarray:
    """The float32 scores every integer routing decision is taken on."""
    return z64.astype(np.float32)


def topk(z32: np.ndarray, K: int) -> np.ndarray:
    """Per token, the K experts of largest score; equal scores go to the
    smaller expert id first.  Returned in that order (slot order)."""
    # A stable sort of -z keeps ascending expert id among equal scores.
    return np.argsort(-z32, axis=1, kind="stable")[:, :K].astype(np.int32)


def membership(idx: np.ndarray, E: int) -> np.ndarray:
    T = idx.shape[0]
    m = np.zeros((T, E), dtype=bool)
    m[np.arange(T)[:, None], idx] = True
    return m


def splitmix64(x: int) -> int:
    """SplitMix64 output function (Steele, Lea & Flood 2014; Vigna's C code):
    add the golden gamma, then two xor-shift-multiply rounds and a final
    xor-shift, all modulo 2^64."""
    z = (x + GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def round_uniform(seed: int, e: int, M: int) -> int:
    """Integer uniform u_e in [0, M) for stochastic rounding of expert e
    (M a power of two): the top log2(M) bits of splitmix64(seed ^ e*gamma)."""
    bits = M.bit_length() - 1
    return splitmix64((seed ^ (e * GOLDEN_GAMMA)) & MASK64) >> (64 - bits)


def rounded_count(c: int, T: int, M: int, mode: int, u: int = 0) -> int:
    """Token-rounded count of one expert ([B] scheduling paragraph).

    mode 1 (nearest): up when the remainder is at least M/2.
    mode 2 (unbiased): up when the remainder exceeds the uniform u in [0, M),
            i.e. with probability remainder/M, so the expected count is c.
    A rounded-up count larger than T (more rows than tokens) rounds down
    instead.  A multiple of M is unchanged; c = 0 stays 0.
    """
    rem = c % M
    down = c - rem
    if rem == 0:
        return c
    up = (rem >= M // 2) if mode == 1 else (rem > u)
    r = down + M if up else down
    if r > T:
        r = down
    return r


def token_round(z32: np.ndarray, member: np.ndarray, M: int, mode: int, seed: int):
    """Token rounding: make every expert's row count a multiple of M.

    Candidates are ranked by (score descending, token id ascending).  An
    expert rounded down keeps its best-ranked routed tokens; an expert rounded
    up keeps all routed tokens and adds the best-ranked tokens not routed to
    it.  Returns (new membership, raw counts c, rounded counts r).
    """
    T, E = member.shape
    out = member.copy()
    c = member.sum(axis=0).astype(np.int64)
    r = np.zeros(E, dtype=np.int64)
    tok = np.arange(T)
    for e in range(E):
        u = round_uniform(seed, e, M) if mode == 2 else 0
        r[e] = rounded_count(int(c[e]), T, M, mode, u)
        col = z32[:, e]
        if r[e] < c[e]:
            cand = tok[member[:, e]]
            order = np.lexsort((cand, -col[cand]))  # score desc, token asc
            drop = cand[order[r[e]:]]
            out[drop, e] = False
        elif r[e] > c[e]:
            cand = tok[~member[:, e]]
            order = np.lexsort((cand, -col[cand]))
            add = cand[order[: r[e] - c[e]]]
            out[add, e] = True
    return out, c, r


def segments(member: np.ndarray, tile: int) -> dict:
    """Expert-sorted row layout of a membership mask.

    counts[e], offsets (exclusive scan, E+1), tile_offsets (exclusive scan of
    ceil(counts/tile)), row_token / row_expert per row (rows of an expert in
    ascending token id), and the per-token CSR tok_ptr / tok_row listing the
    rows of each token in ascending row index.
    """
    T, E = member.shape
    counts = member.sum(axis=0).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    tiles = (counts + tile - 1) // tile
    tile_offsets = np.zeros(E + 1, dtype=np.int64)
    tile_offsets[1:] = np.cumsum(tiles)
    P = int(offsets[-1])
    row_token = np.zeros(P, dtype=np.int64)
    row_expert = np.zeros(P, dtype=np.int64)
    for e in range(E):
        tks = np.nonzero(member[:, e])[0]
        row_token[offsets[e]:offsets[e + 1]] = tks
        row_expert[offsets[e]:offsets[e + 1]] = e
    per_tok = member.sum(axis=1).astype(np.int64)
    tok_ptr = np.zeros(T + 1, dtype=np.int64)
    tok_ptr[1:] = np.cumsum(per_tok)
    # rows in ascending order, bucketed by token: a stable sort by token keeps
    # ascending row index inside each bucket
    tok_row = np.argsort(row_token, kind="stable").astype(np.int64)
    return dict(counts=counts, offsets=offsets, tile_offsets=tile_offsets,
                row_token=row_token, row_expert=row_expert, tok_ptr=tok_ptr,
                tok_row=tok_row, n_rows=P)


def gates(zval: np.ndarray, member: np.ndarray) -> np.ndarray:
    """Softmax of each token's logits over its selected set (0 elsewhere);
    a token with an empty set has all-zero gates.  ``zval`` holds the logit
    values (float64 when the oracle computed them itself)."""
    z = np.asarray(zval, dtype=np.float64)
    zm = np.where(member, z, -np.inf)
    m = zm.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    ex = np.where(member, np.exp(zm - m), 0.0)
    s = ex.sum(axis=1, keepdims=True)
    return np.divide(ex, s, out=np.zeros_like(ex), where=s > 0)


def route_scores(z32: np.ndarray, K: int, tile: int = 128, round_mode: int = 0,
                 round_seed: int = 0, zval=None) -> dict:
    """Routing from float32 scores: top-K, optional token rounding, segments,
    gates.  Everything integer is exact.  Decisions use ``z32``; gate values
    use ``zval`` (float64 logits) when given, else ``z32``."""
    if zval is None:
        zval = z32
    idx = topk(z32, K)
    member = membership(idx, z32.shape[1])
    counts_raw = member.sum(axis=0).astype(np.int64)
    if round_mode:
        member, _, _ = token_round(z32, member, tile, round_mode, round_seed)
    seg = segments(member, tile)
    G = gates(zval, member)
    seg.update(topk_idx=idx, member=member, counts_raw=counts_raw, gate=G,
               topk_gate=np.take_along_axis(gates(zval, membership(idx, z32.shape[1])), idx, 1),
               row_gate=G[seg["row_token"], seg["row_expert"]], scores=z32)
    return seg


def route(x64, wr64, bias, K, tile=128, round_mode=0, round_seed=0) -> dict:
    z64 = router_logits(x64, wr64, bias)
    r = route_scores(decision_scores(z64), K, tile, round_mode, round_seed, zval=z64)
    r["logits64"] = z64
    return r


# ----------------------------------------------------------------------------
# forward  ([B] kernel-list paragraph: up-proj A, down-proj Y, aggregation O;
#           [A] second point: SwiGLU after the up-projection)
# ----------------------------------------------------------------------------

def forward(x64, w1, w2, rt) -> dict:
    """H, A, Y per row (expert-sorted order) and the layer output O."""
    T = x64.shape[0]
    E, d, n2 = w1.shape
    n = n2 // 2
    P = rt["n_rows"]
    off, tok = rt["offsets"], rt["row_token"]
    H = np.zeros((P, 2 * n))
    A = np.zeros((P, n))
    Y = np.zeros((P, d))
    for e in range(E):
        s, t = off[e], off[e + 1]
        if s == t:
            continue
        H[s:t] = x64[tok[s:t]] @ w1[e]
        A[s:t] = silu(H[s:t, :n]) * H[s:t, n:]
        Y[s:t] = A[s:t] @ w2[e]
    O = np.zeros((T, d))
    np.add.at(O, tok, rt["row_gate"][:, None] * Y)
    return dict(H=H, A=A, Y=Y, O=O)


# ----------------------------------------------------------------------------
# backward  ([A] first point: the reordered contraction, only H cached;
#            [B] algorithm paragraph: router gradient without cached Y;
#            [B] kernel-list paragraph: dH, up-proj gradient, dX, dW1, dW2)
# ----------------------------------------------------------------------------

def backward(x64, wr64, w1, w2, rt, H, dO) -> dict:
    """Gradients of L = <dO, O> from the cached H and the routing only."""
    T, d = x64.shape
    E = w1.shape[0]
    n = w1.shape[2] // 2
    P = rt["n_rows"]
    off, tok, rg = rt["offsets"], rt["row_token"], rt["row_gate"]
    dAp = np.zeros((P, n))
    dS = np.zeros(P)
    dH = np.zeros((P, 2 * n))
    dXt = np.zeros((P, d))
    dW1 = np.zeros_like(w1)
    dW2 = np.zeros_like(w2)
    for e in range(E):
        s, t = off[e], off[e + 1]
        if s == t:
            continue
        G, U = H[s:t, :n], H[s:t, n:]
        sg = sigmoid(G)
        A = G * sg * U                      # recomputed from H, no matmul
        dAp[s:t] = dO[tok[s:t]] @ w2[e].T
        dS[s:t] = np.sum(dAp[s:t] * A, axis=1)
        dA = rg[s:t, None] * dAp[s:t]
        dH[s:t, :n] = dA * U * sg * (1.0 + G * (1.0 - sg))
        dH[s:t, n:] = dA * G * sg
        dXt[s:t] = dH[s:t] @ w1[e].T
        dW1[e] = x64[tok[s:t]].T @ dH[s:t]
        dW2[e] = A.T @ (rg[s:t, None] * dO[tok[s:t]])
    # router: softmax-over-set backward, per token
    dz = np.zeros((T, E))
    dSte = np.zeros((T, E))
    dSte[tok, rt["row_expert"]] = dS
    Gt = rt["gate"]
    mean = np.sum(Gt * dSte, axis=1, keepdims=True)
    dz = np.where(rt["member"], Gt * (dSte - mean), 0.0)
    dWr = x64.T @ dz
    db = dz.sum(axis=0)
    dX = dz @ wr64.T
    np.add.at(dX, tok, dXt)
    return dict(dAp=dAp, dS=dS, dH=dH, dXt=dXt, dW1=dW1, dW2=dW2, dz=dz, dWr=dWr,
                db=db, dX=dX)


def backward_naive(x64, wr64, w1, w2, rt, dO) -> dict:
    """The standard activation-caching backward ([A] "MoE 与它的隐患" figure
    captions): the forward caches the gathered X, H, A and Y; the gate
    gradient is <dO, Y> and the router gradient goes through the explicit
    softmax Jacobian diag(g) - g g^T of each token's set."""
    T, d = x64.shape
    E = w1.shape[0]
    n = w1.shape[2] // 2
    off, tok, rg = rt["offsets"], rt["row_token"], rt["row_gate"]
    P = rt["n_rows"]
    # forward with caches
    Xg = x64[tok]
    Hc = np.zeros((P, 2 * n))
    Ac = np.zeros((P, n))
    Yc = np.zeros((P, d))
    for e in range(E):
        s, t = off[e], off[e + 1]
        Hc[s:t] = Xg[s:t] @ w1[e]
        Ac[s:t] = silu(Hc[s:t, :n]) * Hc[s:t, n:]
        Yc[s:t] = Ac[s:t] @ w2[e]
    # backward
    dY = rg[:, None] * dO[tok]
    dgate = np.sum(dO[tok] * Yc, axis=1)
    dXg = np.zeros((P, d))
    dW1 = np.zeros_like(w1)
    dW2 = np.zeros_like(w2)
    dHc = np.zeros((P, 2 * n))
    for e in range(E):
        s, t = off[e], off[e + 1]
        if s == t:
            continue
        dA = dY[s:t] @ w2[e].T
        G, U = Hc[s:t, :n], Hc[s:t, n:]
        sg = sigmoid(G)
        dsilu = sg + G * sg * (1.0 - sg)        # d/dG of G*sigmoid(G)
        dHc[s:t, :n] = dA * U * dsilu
        dHc[s:t, n:] = dA * silu(G)
        dXg[s:t] = dHc[s:t] @ w1[e].T
        dW1[e] = Xg[s:t].T @ dHc[s:t]
        dW2[e] = Ac[s:t].T @ dY[s:t]
    dz = np.zeros((T, E))
    member, Gt = rt["member"], rt["gate"]
    rows_of = [[] for _ in range(T)]
    for r in range(P):
        rows_of[tok[r]].append(r)
    for t in range(T):
        rs = rows_of[t]
        if not rs:
            continue
        es = rt["row_expert"][rs]
        g = Gt[t, es]
        J = np.diag(g) - np.outer(g, g)      # d gate_i / d z_j over the set
        dz[t, es] = J.T @ dgate[rs]
    dX = np.zeros((T, d))
    for r in range(P):
        dX[tok[r]] += dXg[r]
    dX += dz @ wr64.T
    return dict(dS=dgate, dH=dHc, dXt=dXg, dW1=dW1, dW2=dW2, dz=dz, dWr=x64.T @ dz,
                dX=dX, Y=Yc)


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def layer(x, w_r, w1, w2, d_o, dtype, K, bias=None, tile=128, round_mode=0, round_seed=0,
          scores=None) -> dict:
    """Route, forward and backward one layer from raw inputs (bf16 as uint16
    bits).  With ``scores`` (float32 T x E) routing uses those scores in place
    of the router logits (gradients still flow through z = X W_r + b)."""
    x64, wr64 = to_f64(x, dtype), to_f64(w_r, dtype)
    w1_64, w2_64, dO = to_f64(w1, dtype), to_f64(w2, dtype), to_f64(d_o, dtype)
    if scores is None:
        rt = route(x64, wr64, bias, K, tile, round_mode, round_seed)
    else:
        rt = route_scores(np.asarray(scores, dtype=np.float32), K, tile, round_mode, round_seed)
    f = forward(x64, w1_64, w2_64, rt)
    b = backward(x64, wr64, w1_64, w2_64, rt, f["H"], dO)
    out = dict(rt)
    out.update(f)
    out.update(b)
    return out
