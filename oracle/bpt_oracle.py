"""fp64 CPU oracle of the Blockwise Parallel Transformer (BPT) layer forward.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import this module. The GPU
path never calls it and it never calls the GPU path; the two share no code.

What it computes is the plain definition, not the blockwise schedule: the BPT
paper review ("Blockwise Parallel Transformer for Large Context Models",
sections 三 "核心公式" and 四 "无近似计算") states that the blockwise
computation is exact, i.e. it yields the result of standard softmax attention
followed by the FFN. So the oracle materialises each row's full score vector,
takes a two-pass softmax, and applies the output projection, the residual,
the ReLU FFN and the second residual:

    QKV = x W_qkv + b_qkv,    Q|K|V column blocks, head n at columns n*d..   (1)
    S   = Q_n K_n^T / sqrt(d) per head, masked to key <= query if causal     (2)
    A_n = softmax_rows(S) V_n,  heads concatenated back to [b, s, h]         (3)
    y   = x + A W_o + b_o                                                    (4)
    out = y + max(0, y W_1 + b_1) W_2 + b_2                                  (5)

Sources for each step:
  (1) fused projection of x into Q, K, V: "Transformer QKV 矩阵计算…3 种并行化
      策略对比" §1 and §2; the BPT review's Algorithm 1, step 1 (the whole
      sequence is projected before the block loops). Column blocks [Q|K|V]
      follow "PyTorch 2.3 实现多头自注意力…" §6 (in_proj = cat of q, k, v);
      head n = columns n*d..n*d+d-1 follows the same page's §2 (view then
      transpose).
  (2) scale 1/sqrt(d), d = h / heads: BPT review §三 "核心公式" (standard
      attention) and the PyTorch 2.3 MHSA page §3. Causal: keep key j for query
      i iff j <= i; masked weights are exactly zero (the MHSA page §3 fills
      masked scores with -inf before the softmax).
  (3) merge heads: PyTorch 2.3 MHSA page §4.
  (4) output projection: PyTorch 2.3 MHSA page §4 (out_proj) and the QKV page
      §2 (output_linear); residual: BPT review §三, blockwise FFN with residual
      connection, where the residual operand is read as the query block's
      input x_i (the block of x that Figure 2's caption says is projected as
      query).
  (5) FFN(x) = max(0, x W1 + b1) W2 + b2 and the second residual: BPT review
      §三 "核心公式" (standard FFN, and blockwise FFN with residual).

Precision: every product and sum in float64; inputs are the exact float32 /
bf16 values the GPU receives, widened. Nothing is rounded in between.

Row sampling: ``rows`` restricts the evaluated query rows. K and V are still
projected for every token, and each evaluated row still sees its full key
range, so the result is exact for those rows. The per-row work is done in
chunks of rows only to bound memory; every chunk holds complete score rows.
"""
from __future__ import annotations

import time
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "project_qkv",
    "attention_probs",
    "attention",
    "merge_heads",
    "layer_forward",
    "stack_forward",
    "philox4x64_10",
    "dropout_keep",
    "layer_backward",
    "layer_backward_causal_tail",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _split_heads(t: np.ndarray, heads: int) -> np.ndarray:
    """[b, r, h] -> [b, heads, r, d] (PyTorch 2.3 MHSA page §2: view, transpose)."""
    b, r, h = t.shape
    d = h // heads
    return t.reshape(b, r, heads, d).transpose(0, 2, 1, 3)


def merge_heads(t: np.ndarray) -> np.ndarray:
    """[b, heads, r, d] -> [b, r, heads*d] (PyTorch 2.3 MHSA page §4)."""
    b, nh, r, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(b, r, nh * d)


def project_qkv(x, Wqkv, bqkv, heads: int, rows: Optional[np.ndarray] = None):
    """Step (1). Returns Q [b, nh, r, d] for the evaluated rows and K, V
    [b, nh, s, d] for every token."""
    x = _f64(x)
    Wqkv = _f64(Wqkv)
    bqkv = _f64(bqkv)
    b, s, h = x.shape
    if h % heads != 0:
        raise ValueError("hidden size must be divisible by the number of heads")
    xq = x if rows is None else x[:, rows, :]
    Q = xq @ Wqkv[:, 0:h] + bqkv[0:h]
    K = x @ Wqkv[:, h:2 * h] + bqkv[h:2 * h]
    V = x @ Wqkv[:, 2 * h:3 * h] + bqkv[2 * h:3 * h]
    return _split_heads(Q, heads), _split_heads(K, heads), _split_heads(V, heads)


def attention_probs(Qn: np.ndarray, Kn: np.ndarray, causal: bool,
                    qpos: np.ndarray) -> np.ndarray:
    """Step (2) and the softmax of step (3) for one (batch, head).

    Qn [r, d] holds the queries at sequence positions ``qpos``; Kn [s, d].
    Returns P [r, s]: rows of the softmax of Qn Kn^T / sqrt(d), with keys
    after the query's position given weight exactly 0 when ``causal``.
    Two passes: row maximum, then exponentials normalised by their sum.
    """
    d = Qn.shape[1]
    S = (Qn @ Kn.T) / np.sqrt(float(d))
    if causal:
        kpos = np.arange(Kn.shape[0])
        S = np.where(kpos[None, :] <= qpos[:, None], S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=1, keepdims=True)


def attention(Q, K, V, causal: bool, qpos: Optional[np.ndarray] = None,
              row_chunk: int = 512) -> np.ndarray:
    """Steps (2)-(3) per head: A_n = softmax(Q_n K_n^T / sqrt d) V_n.

    Q [b, nh, r, d] at positions ``qpos`` (default 0..r-1), K, V [b, nh, s, d].
    Returns the head outputs [b, nh, r, d].
    """
    b, nh, r, d = Q.shape
    if qpos is None:
        qpos = np.arange(r)
    out = np.empty((b, nh, r, d), dtype=np.float64)
    for bi in range(b):
        for n in range(nh):
            for r0 in range(0, r, row_chunk):
                r1 = min(r, r0 + row_chunk)
                P = attention_probs(Q[bi, n, r0:r1], K[bi, n], causal, qpos[r0:r1])
                out[bi, n, r0:r1] = P @ V[bi, n]
    return out


# ---------------------------------------------------------------------------
# Training-mode dropout on the two residual branches.
#
# The BPT review's memory analysis (section 三, FFN memory of the blockwise
# layer) counts a dropout mask of b·c·h elements per chunk, i.e. dropout on
# the FFN's h-wide output, and its JAX listing gives every FFN chunk its own
# dropout RNG stream; the PyTorch 2.3 MHSA page (§5) applies dropout to the
# projected attention output before the residual. Reading: with rate p,
#     y   = x + D0 ∘ (A W_o + b_o) / (1 - p)
#     out = y + D1 ∘ (max(0, y W_1 + b_1) W_2 + b_2) / (1 - p)
# with D0, D1 independent keep masks. Attention probabilities are not
# dropped (neither page drops them).
#
# The masks come from a counter-based generator so that they do not depend on
# block sizes or on how the FFN is chunked: element (token t, channel j) of
# site z (0: attention branch, 1: FFN branch) under a 64-bit seed uses
# Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
# easy as 1, 2, 3", SC 2011) with key (seed, z) and counter (t, j // 16, 0, 0),
# where t = batch·s + position. The four 64-bit output words hold sixteen
# 16-bit uniforms; channel j takes number j % 16 (word (j % 16) // 4, bits
# 16·(j % 4) upwards). The element is dropped iff its uniform is below
# T = round(p·65536), so the drop probability is T/65536 and kept values are
# scaled by 65536 / (65536 - T).

_U = np.uint64
_M32 = _U(0xFFFFFFFF)
# Philox4x64 multipliers and Weyl key increments, from the paper above.
_PHILOX_M0, _PHILOX_M1 = _U(0xD2E7470EE14C6C93), _U(0xCA5A826395121157)
_PHILOX_W0, _PHILOX_W1 = _U(0x9E3779B97F4A7C15), _U(0xBB67AE8584CAA73B)


def _mulhilo64(a: np.ndarray, b: np.ndarray):
    """High and low 64-bit halves of the 128-bit products a·b (uint64 arrays),
    from four 32×32-bit partial products."""
    a0, a1 = a & _M32, a >> _U(32)
    b0, b1 = b & _M32, b >> _U(32)
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _U(32)) + (p01 & _M32) + (p10 & _M32)
    lo = (p00 & _M32) | ((mid & _M32) << _U(32))
    hi = p11 + (p01 >> _U(32)) + (p10 >> _U(32)) + (mid >> _U(32))
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds (the paper above), elementwise over arrays.

    counter: four uint64 arrays (c0, c1, c2, c3) of one shape; key: two uint64
    values or arrays. A round maps (c0, c1, c2, c3) to
    (hi(M1·c2) ^ c1 ^ k0, lo(M1·c2), hi(M0·c0) ^ c3 ^ k1, lo(M0·c0)); the key
    is bumped by the Weyl constants (W0, W1) between rounds. Returns the four
    output words as uint64 arrays.
    """
    c0, c1, c2, c3 = (np.array(v, dtype=np.uint64) for v in counter)
    k0 = np.array(key[0], dtype=np.uint64).reshape(-1)
    k1 = np.array(key[1], dtype=np.uint64).reshape(-1)
    for r in range(10):
        if r:
            k0 = k0 + _PHILOX_W0
            k1 = k1 + _PHILOX_W1
        hi0, lo0 = _mulhilo64(_PHILOX_M0, c0)
        hi1, lo1 = _mulhilo64(_PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def dropout_threshold(p: float) -> int:
    """T = round(p·65536): an element is dropped iff its 16-bit uniform < T."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout rate must lie in [0, 1)")
    return int(round(p * 65536.0))


def dropout_keep(tokens, channels: int, p: float, seed: int, site: int) -> np.ndarray:
    """Keep mask [len(tokens), channels] (bool) of dropout site ``site`` for
    the given global token indices, per the definition above."""
    tok = np.asarray(tokens, dtype=np.uint64).reshape(-1, 1)
    j = np.arange(channels, dtype=np.uint64).reshape(1, -1)
    c0 = np.broadcast_to(tok, (tok.shape[0], channels))
    c1 = np.broadcast_to(j >> _U(4), c0.shape)
    zero = np.zeros(c0.shape, dtype=np.uint64)
    words = philox4x64_10((c0, c1, zero, zero), (_U(seed), _U(site)))
    i = (j & _U(15)).astype(np.int64)
    w = np.choose(np.broadcast_to(i >> 2, c0.shape), words)
    u = (w >> (_U(16) * (np.broadcast_to(i & 3, c0.shape)).astype(np.uint64))) & _U(0xFFFF)
    return u >= _U(dropout_threshold(p))


def _dropout(v: np.ndarray, tokens, p: float, seed: int, site: int) -> np.ndarray:
    """v [r, h] with dropout site ``site`` applied at the given tokens."""
    T = dropout_threshold(p)
    if T == 0:
        return v
    keep = dropout_keep(tokens, v.shape[-1], p, seed, site)
    return np.where(keep, v * (65536.0 / (65536.0 - T)), 0.0)


def layer_forward(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, heads: int, causal: bool,
                  rows: Optional[Sequence[int]] = None,
                  row_chunk: int = 512, timings: Optional[dict] = None,
                  dropout_p: float = 0.0, seed: int = 0) -> Dict[str, np.ndarray]:
    """One BPT layer forward, steps (1)-(5), in float64.

    x [b, s, h]; weights in [in, out] layout. ``rows`` (optional) selects the
    query rows to evaluate (the same rows in every batch). Returns a dict with
    ``out`` [b, r, h], ``y`` [b, r, h] (after the first residual) and ``A``
    [b, r, h] (attention output with heads merged, before W_o). If
    ``timings`` is a dict, the wall-clock seconds of step (1) and of steps
    (2)-(5) are stored in it under "projection" and "rows". ``dropout_p`` > 0
    selects training mode: both residual branches go through the dropout
    defined above, with masks keyed by ``seed``.
    """
    t0 = time.perf_counter()
    x = _f64(x)
    b, s, h = x.shape
    rws = None if rows is None else np.asarray(rows, dtype=np.int64)
    Q, K, V = project_qkv(x, Wqkv, bqkv, heads, rws)
    t1 = time.perf_counter()
    qpos = np.arange(s) if rws is None else rws
    A = merge_heads(attention(Q, K, V, causal, qpos, row_chunk))
    xr = x if rws is None else x[:, rws, :]
    attn_out = A @ _f64(Wo) + _f64(bo)
    if dropout_p > 0.0:
        pos = np.arange(s) if rws is None else rws
        for bi in range(b):
            attn_out[bi] = _dropout(attn_out[bi], bi * s + pos, dropout_p, seed, 0)
    y = xr + attn_out
    H = np.maximum(0.0, y @ _f64(W1) + _f64(b1))
    ffn_out = H @ _f64(W2) + _f64(b2)
    if dropout_p > 0.0:
        for bi in range(b):
            ffn_out[bi] = _dropout(ffn_out[bi], bi * s + pos, dropout_p, seed, 1)
    out = y + ffn_out
    if timings is not None:
        timings["projection"] = t1 - t0
        timings["rows"] = time.perf_counter() - t1
    return {"out": out, "y": y, "A": A}


def stack_forward(x, layers, heads: int, causal: bool) -> np.ndarray:
    """A stack of layers, each the layer above applied to the previous
    layer's output. ``layers`` is a sequence of 8-tuples of weights."""
    cur = _f64(x)
    for wts in layers:
        cur = layer_forward(cur, *wts, heads=heads, causal=causal)["out"]
    return cur



# ---------------------------------------------------------------------------
# Backward of the inference forward (dropout off): the gradients of
# sum(out ∘ G) for an upstream gradient G = dL/d out, by the chain rule of
# steps (1)-(5) written out term by term. The BPT review (section 三, memory
# of the blockwise layer, and its remark that the method composes with
# rematerialisation) trains this layer by recomputing each block's forward in
# the backward pass; the oracle instead materialises everything, since the
# gradients are the same. With Z = Q K^T / sqrt(d) and P = softmax_rows(Z):
#
#   (5)  dW2 = H^T G,  db2 = sum_t G,  dHpre = (G W2^T) ∘ [y W1 + b1 > 0],
#        dW1 = y^T dHpre,  db1 = sum_t dHpre,  dy = G + dHpre W1^T
#   (4)  dWo = A^T dy,  dbo = sum_t dy,  dA = dy Wo^T
#   (3)  per head: dV = P^T dO,  dP = dO V^T
#   (2)  dZ = P ∘ (dP - rowsum(dP ∘ P)),  dQ = dZ K / sqrt(d),
#        dK = dZ^T Q / sqrt(d)   (masked entries have P = 0, so dZ = 0)
#   (1)  dQKV = [dQ | dK | dV] (heads merged),  dWqkv = x^T dQKV,
#        dbqkv = sum_t dQKV,  dx = dy + dQKV Wqkv^T
#
# The derivative of max(0, v) at v = 0 is taken as 0. Weights are in the
# oracle's [in, out] layout, so each weight gradient has its weight's shape.
# The ReLU's on/off decisions are the oracle's own, taken in float64.
#
# Training mode (dropout_p > 0): the forward drops the two residual branches
# with fixed masks (they depend on seed, site, token and channel only), so
# each branch is multiplied elementwise by a constant M_z = keep_z · 65536 /
# (65536 - T) and the chain rule passes the upstream gradient of a branch
# through the same constant:
#
#   (5')  G is replaced by G ∘ M_1 in dW2, db2 and dHpre (dy = G + dHpre W1^T
#         keeps the unmasked G of the residual path)
#   (4')  dy is replaced by dy ∘ M_0 in dWo, dbo and dA (dx = dy + dQKV
#         Wqkv^T keeps the unmasked dy)


def _branch_scale(b: int, s: int, h: int, p: float, seed: int, site: int,
                  pos: Optional[np.ndarray] = None) -> np.ndarray:
    """M_z [b, r, h]: keep · 65536 / (65536 - T) of dropout site ``site`` at
    the positions ``pos`` (all s by default) of every sequence; ones when
    p = 0. The same masks as layer_forward's training mode."""
    pos = np.arange(s) if pos is None else np.asarray(pos)
    T = dropout_threshold(p)
    if T == 0:
        return np.ones((b, len(pos), h))
    scale = 65536.0 / (65536.0 - T)
    return np.stack([np.where(dropout_keep(bi * s + pos, h, p, seed, site), scale, 0.0)
                     for bi in range(b)])


def layer_backward(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, G, heads: int,
                   causal: bool, dropout_p: float = 0.0, seed: int = 0) -> Dict[str, np.ndarray]:
    """Gradients of sum(layer_forward(..., dropout_p, seed)["out"] ∘ G) in
    float64 (dropout_p = 0: the inference forward).

    Returns a dict with dx [b, s, h] and dWqkv, dbqkv, dWo, dbo, dW1, db1,
    dW2, db2 (each in its parameter's shape), plus the forward's out and y
    and the projection's upstream gradient dQKV [b, s, 3h].
    """
    x = _f64(x)
    G = _f64(G)
    Wqkv, bqkv, Wo, bo = _f64(Wqkv), _f64(bqkv), _f64(Wo), _f64(bo)
    W1, b1, W2, b2 = _f64(W1), _f64(b1), _f64(W2), _f64(b2)
    b, s, h = x.shape
    d = h // heads
    # forward, keeping what the chain rule needs
    Q, K, V = project_qkv(x, Wqkv, bqkv, heads)
    pos = np.arange(s)
    P = np.empty((b, heads, s, s))
    for bi in range(b):
        for n in range(heads):
            P[bi, n] = attention_probs(Q[bi, n], K[bi, n], causal, pos)
    O = P @ V
    A = merge_heads(O)
    M0 = _branch_scale(b, s, h, dropout_p, seed, 0)
    M1 = _branch_scale(b, s, h, dropout_p, seed, 1)
    y = x + M0 * (A @ Wo + bo)
    Hpre = y @ W1 + b1
    H = np.maximum(0.0, Hpre)
    out = y + M1 * (H @ W2 + b2)
    flat = lambda t: t.reshape(-1, t.shape[-1])
    # (5) FFN and second residual
    Gf = G * M1
    dW2 = flat(H).T @ flat(Gf)
    db2 = flat(Gf).sum(axis=0)
    dHpre = (Gf @ W2.T) * (Hpre > 0.0)
    dW1 = flat(y).T @ flat(dHpre)
    db1 = flat(dHpre).sum(axis=0)
    dy = G + dHpre @ W1.T
    # (4) output projection and first residual
    da = dy * M0
    dWo = flat(A).T @ flat(da)
    dbo = flat(da).sum(axis=0)
    dO = _split_heads(da @ Wo.T, heads)
    # (3), (2) attention
    dV = np.swapaxes(P, 2, 3) @ dO
    dP = dO @ np.swapaxes(V, 2, 3)
    dZ = P * (dP - np.sum(dP * P, axis=3, keepdims=True))
    dQ = (dZ @ K) / np.sqrt(float(d))
    dK = (np.swapaxes(dZ, 2, 3) @ Q) / np.sqrt(float(d))
    # (1) projection
    dQKV = np.concatenate([merge_heads(dQ), merge_heads(dK), merge_heads(dV)], axis=2)
    dWqkv = flat(x).T @ flat(dQKV)
    dbqkv = flat(dQKV).sum(axis=0)
    dx = dy + dQKV @ Wqkv.T
    return {"dx": dx, "dWqkv": dWqkv, "dbqkv": dbqkv, "dWo": dWo, "dbo": dbo,
            "dW1": dW1, "db1": db1, "dW2": dW2, "db2": db2, "out": out, "y": y,
            "dQKV": dQKV}


def layer_backward_causal_tail(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, G, heads: int,
                               tail: int, dropout_p: float = 0.0,
                               seed: int = 0) -> Dict[str, np.ndarray]:
    """dx of sum(layer_forward(..., causal=True)["out"] ∘ G) for the last
    ``tail`` positions of every sequence, exactly, without the full backward.

    The same chain rule as ``layer_backward``, restricted by the causal
    structure: for a position t in the tail T = {s-tail, ..., s-1},
      * dy[t], dO[t] and the ReLU branch involve row t only (steps (4)-(5)
        are position-wise);
      * dQ[t] needs the score row of query t, over keys <= t;
      * dK[t] and dV[t] take contributions from the queries q >= t only,
        all of which lie in T.
    So the score rows of the tail queries (each over its full causal key
    range) and K, V for every token determine dx[T]. Returns {"dx": [b, tail,
    h], "rows": the positions}.
    """
    x = _f64(x)
    G = _f64(G)
    Wqkv, bqkv, Wo, bo = _f64(Wqkv), _f64(bqkv), _f64(Wo), _f64(bo)
    W1, b1, W2 = _f64(W1), _f64(b1), _f64(W2)
    b, s, h = x.shape
    d = h // heads
    if not 0 < tail <= s:
        raise ValueError("tail must be in [1, s]")
    rows = np.arange(s - tail, s)
    Q, K, V = project_qkv(x, Wqkv, bqkv, heads, rows)       # Q of the tail rows only
    P = np.empty((b, heads, tail, s))
    for bi in range(b):
        for n in range(heads):
            P[bi, n] = attention_probs(Q[bi, n], K[bi, n], True, rows)
    A = merge_heads(P @ V)
    xr, Gr = x[:, rows, :], G[:, rows, :]
    M0 = _branch_scale(b, s, h, dropout_p, seed, 0, rows)
    M1 = _branch_scale(b, s, h, dropout_p, seed, 1, rows)
    y = xr + M0 * (A @ Wo + bo)
    Hpre = y @ W1 + b1
    dy = Gr + ((Gr * M1 @ W2.T) * (Hpre > 0.0)) @ W1.T
    dO = _split_heads((dy * M0) @ Wo.T, heads)               # [b, nh, tail, d]
    dP = dO @ np.swapaxes(V, 2, 3)                           # [b, nh, tail, s]
    dZ = P * (dP - np.sum(dP * P, axis=3, keepdims=True))
    dQ = (dZ @ K) / np.sqrt(float(d))
    # key t in T: only tail queries see it; columns s-tail.. of the tail rows
    dK = (np.swapaxes(dZ[..., s - tail:], 2, 3) @ Q) / np.sqrt(float(d))
    dV = np.swapaxes(P[..., s - tail:], 2, 3) @ dO
    dQKV = np.concatenate([merge_heads(dQ), merge_heads(dK), merge_heads(dV)], axis=2)
    return {"dx": dy + dQKV @ Wqkv.T, "rows": rows}
