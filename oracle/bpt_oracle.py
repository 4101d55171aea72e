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


def layer_forward(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, heads: int, causal: bool,
                  rows: Optional[Sequence[int]] = None,
                  row_chunk: int = 512, timings: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """One BPT layer forward, steps (1)-(5), in float64.

    x [b, s, h]; weights in [in, out] layout. ``rows`` (optional) selects the
    query rows to evaluate (the same rows in every batch). Returns a dict with
    ``out`` [b, r, h], ``y`` [b, r, h] (after the first residual) and ``A``
    [b, r, h] (attention output with heads merged, before W_o). If
    ``timings`` is a dict, the wall-clock seconds of step (1) and of steps
    (2)-(5) are stored in it under "projection" and "rows".
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
    y = xr + A @ _f64(Wo) + _f64(bo)
    H = np.maximum(0.0, y @ _f64(W1) + _f64(b1))
    out = y + H @ _f64(W2) + _f64(b2)
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

