"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each ``pin_*`` takes a layer function with the oracle's signature
``fn(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, heads=, causal=) -> {"out", "y", "A"}``
and raises AssertionError when the function disagrees with what the pages
and the mathematics fix. The oracle must pass all of them; the mutation test
checks that each plausible slip in a layer function fails at least one.

Sources of the pins:
  * hand-worked closed forms (tests/golden/hand_worked.json);
  * the library special case of the PyTorch 2.3 MHSA page §6: torch's own
    nn.MultiheadAttention with synchronised weights (float64, CPU), plus
    torch's Linear/ReLU layers for the FFN;
  * the BPT review's Algorithm 1 transcribed here as an independent blockwise
    computation (per-block statistics rescaled at the end), which the review
    (§四, exact computation) says must equal standard attention, for every
    block size dividing the sequence;
  * invariants: causality, constant V, uniform attention, key-bias shift,
    permutation equivariance, zero weights, a single token;
  * brute force with scalar Python loops on tiny shapes;
  * large logits (numerical stability of the blockwise softmax, BPT review
    §三 scaling, and the tutorial's note on per-block statistics).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")

RTOL = 1e-12


def rand_layer(rng, b, s, h, f, wstd=0.3, bstd=0.1):
    x = rng.standard_normal((b, s, h))
    W = dict(
        Wqkv=rng.standard_normal((h, 3 * h)) * wstd, bqkv=rng.standard_normal(3 * h) * bstd,
        Wo=rng.standard_normal((h, h)) * wstd, bo=rng.standard_normal(h) * bstd,
        W1=rng.standard_normal((h, f)) * wstd, b1=rng.standard_normal(f) * bstd,
        W2=rng.standard_normal((f, h)) * wstd, b2=rng.standard_normal(h) * bstd,
    )
    return x, W


def _call(fn, x, W, heads, causal):
    return fn(x, W["Wqkv"], W["bqkv"], W["Wo"], W["bo"], W["W1"], W["b1"], W["W2"],
              W["b2"], heads=heads, causal=causal)


def _close(a, b, rtol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    scale = max(1.0, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b))) / scale
    assert err <= rtol, f"{what}: max error {err:.3e} > {rtol:.1e}"


# ---------------------------------------------------------------------------
def pin_hand_worked(fn):
    with open(GOLDEN) as fh:
        cases = json.load(fh)["cases"]
    env = {"exp": math.exp, "sqrt": math.sqrt, "__builtins__": {}}
    for c in cases:
        arr = lambda k: np.asarray(c[k], dtype=np.float64)
        x = arr("x")[None]
        W = {k: arr(k) for k in ("Wqkv", "bqkv", "Wo", "bo", "W1", "b1", "W2", "b2")}
        got = _call(fn, x, W, c["heads"], c["causal"])["out"][0]
        want = np.array([[eval(e, env) for e in row] for row in c["out"]], dtype=np.float64)
        _close(got, want, 1e-14, c["name"])


# ---------------------------------------------------------------------------
def _torch_layer(x, W, heads, causal):
    """The layer assembled from torch's own modules in float64 on the CPU:
    nn.MultiheadAttention with the weights synchronised as the PyTorch 2.3
    MHSA page §6 does, then nn.Linear / ReLU / nn.Linear for the FFN."""
    import torch
    b, s, h = x.shape
    f = W["W1"].shape[1]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    mha = torch.nn.MultiheadAttention(h, heads, bias=True, batch_first=True,
                                      dtype=torch.float64)
    lin1 = torch.nn.Linear(h, f, dtype=torch.float64)
    lin2 = torch.nn.Linear(f, h, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(t(W["Wqkv"].T))
        mha.in_proj_bias.copy_(t(W["bqkv"]))
        mha.out_proj.weight.copy_(t(W["Wo"].T))
        mha.out_proj.bias.copy_(t(W["bo"]))
        lin1.weight.copy_(t(W["W1"].T))
        lin1.bias.copy_(t(W["b1"]))
        lin2.weight.copy_(t(W["W2"].T))
        lin2.bias.copy_(t(W["b2"]))
        xt = t(x)
        mask = None
        if causal:
            mask = torch.triu(torch.ones(s, s, dtype=torch.bool), diagonal=1)
        att, _ = mha(xt, xt, xt, need_weights=False, attn_mask=mask)
        y = xt + att
        out = y + lin2(torch.relu(lin1(y)))
    return out.numpy(), y.numpy()


def pin_library(fn, seed=11):
    rng = np.random.default_rng(seed)
    for (b, s, h, heads, f, causal) in [(2, 9, 8, 2, 12, False), (1, 13, 12, 3, 8, True),
                                        (2, 7, 8, 1, 16, True), (1, 16, 16, 4, 32, False)]:
        x, W = rand_layer(rng, b, s, h, f)
        got = _call(fn, x, W, heads, causal)
        want_out, want_y = _torch_layer(x, W, heads, causal)
        _close(got["y"], want_y, 1e-12, f"library y b{b} s{s} h{h} nh{heads} causal={causal}")
        _close(got["out"], want_out, 1e-12, f"library out b{b} s{s} h{h} nh{heads} causal={causal}")


# ---------------------------------------------------------------------------
def blockwise_algorithm1(x, W, heads, causal, B_q, B_kv):
    """Independent fp64 transcription of the BPT review's Algorithm 1.

    Project the whole sequence; for each query block, walk the key/value
    blocks recording each block's row maximum m_j, the block's unnormalised
    exponentials' row sums l_j and partial products with V_j; then rescale
    all blocks by exp(m_j - max_j m_j) (the review's "Scaling", Eq. 3) and
    normalise; then apply the output projection, residual, FFN and second
    residual to that query block alone.
    """
    b, s, h = x.shape
    d = h // heads
    qkv = x @ W["Wqkv"] + W["bqkv"]
    out = np.empty_like(x)
    for bi in range(b):
        for q0 in range(0, s, B_q):
            q1 = q0 + B_q
            A_blk = np.empty((B_q, h))
            for n in range(heads):
                q = qkv[bi, q0:q1, n * d:(n + 1) * d]
                stats = []
                for k0 in range(0, s, B_kv):
                    k1 = k0 + B_kv
                    k = qkv[bi, k0:k1, h + n * d:h + (n + 1) * d]
                    v = qkv[bi, k0:k1, 2 * h + n * d:2 * h + (n + 1) * d]
                    sc = (q @ k.T) / math.sqrt(d)
                    if causal:
                        keep = np.arange(k0, k1)[None, :] <= np.arange(q0, q1)[:, None]
                        if not keep.any():
                            continue
                        sc = np.where(keep, sc, -np.inf)
                    mj = sc.max(axis=1, keepdims=True)
                    # rows whose keys in this block are all masked contribute nothing
                    mj_safe = np.where(np.isfinite(mj), mj, 0.0)
                    e = np.exp(sc - mj_safe)
                    stats.append((mj, e.sum(axis=1, keepdims=True), e @ v))
                m_all = np.max(np.concatenate([st[0] for st in stats], axis=1), axis=1,
                               keepdims=True)
                num = np.zeros((B_q, d))
                den = np.zeros((B_q, 1))
                for mj, lj, pv in stats:
                    w = np.where(np.isfinite(mj), np.exp(np.where(np.isfinite(mj), mj, 0) - m_all), 0.0)
                    num += w * pv
                    den += w * lj
                A_blk[:, n * d:(n + 1) * d] = num / den
            y = x[bi, q0:q1] + A_blk @ W["Wo"] + W["bo"]
            out[bi, q0:q1] = y + np.maximum(0.0, y @ W["W1"] + W["b1"]) @ W["W2"] + W["b2"]
    return out


def pin_blockwise(fn, seed=12):
    rng = np.random.default_rng(seed)
    b, s, h, heads, f = 2, 24, 8, 2, 16
    x, W = rand_layer(rng, b, s, h, f, wstd=0.6)
    divisors = [B for B in range(1, s + 1) if s % B == 0]
    for causal in (False, True):
        ref = _call(fn, x, W, heads, causal)["out"]
        for B_q in divisors:
            for B_kv in divisors:
                got = blockwise_algorithm1(x, W, heads, causal, B_q, B_kv)
                _close(ref, got, 1e-12, f"blockwise B_q={B_q} B_kv={B_kv} causal={causal}")


# ---------------------------------------------------------------------------
def brute_force_layer(x, W, heads, causal):
    """Scalar Python loops over lists; only for tiny shapes."""
    b, s, h = len(x), len(x[0]), len(x[0][0])
    f = len(W["b1"])
    d = h // heads
    Wqkv, bqkv = W["Wqkv"].tolist(), W["bqkv"].tolist()
    Wo, bo, W1, b1, W2, b2 = (W[k].tolist() for k in ("Wo", "bo", "W1", "b1", "W2", "b2"))
    res = []
    for bi in range(b):
        xs = x[bi].tolist()
        proj = [[sum(xs[t][k] * Wqkv[k][c] for k in range(h)) + bqkv[c] for c in range(3 * h)]
                for t in range(s)]
        out_rows = []
        for i in range(s):
            A = [0.0] * h
            for n in range(heads):
                keys = [j for j in range(s) if (not causal or j <= i)]
                sc = [sum(proj[i][n * d + e] * proj[j][h + n * d + e] for e in range(d)) / math.sqrt(d)
                      for j in keys]
                m = max(sc)
                w = [math.exp(v - m) for v in sc]
                Z = sum(w)
                for e in range(d):
                    A[n * d + e] = sum(w[t] * proj[keys[t]][2 * h + n * d + e] for t in range(len(keys))) / Z
            y = [xs[i][c] + sum(A[k] * Wo[k][c] for k in range(h)) + bo[c] for c in range(h)]
            H = [max(0.0, sum(y[c] * W1[c][g] for c in range(h)) + b1[g]) for g in range(f)]
            out_rows.append([y[c] + sum(H[g] * W2[g][c] for g in range(f)) + b2[c] for c in range(h)])
        res.append(out_rows)
    return np.array(res)


def pin_brute_force(fn, seed=13):
    rng = np.random.default_rng(seed)
    for (b, s, h, heads, f, causal) in [(1, 5, 4, 1, 6, False), (2, 6, 6, 2, 4, True),
                                        (1, 8, 8, 2, 8, True), (1, 3, 2, 2, 3, False)]:
        x, W = rand_layer(rng, b, s, h, f, wstd=0.8)
        _close(_call(fn, x, W, heads, causal)["out"], brute_force_layer(x, W, heads, causal),
               1e-12, f"brute force s{s} h{h} nh{heads} causal={causal}")


# ---------------------------------------------------------------------------
def pin_causality(fn, seed=14):
    """Perturbing tokens after position i leaves outputs 0..i unchanged."""
    rng = np.random.default_rng(seed)
    b, s, h, heads, f = 1, 20, 8, 2, 8
    x, W = rand_layer(rng, b, s, h, f, wstd=0.5)
    ref = _call(fn, x, W, heads, True)["out"]
    for i in (0, 7, 18):
        xp = x.copy()
        xp[:, i + 1:] += rng.standard_normal(xp[:, i + 1:].shape) * 3.0
        got = _call(fn, xp, W, heads, True)["out"]
        assert np.array_equal(got[:, :i + 1], ref[:, :i + 1]), f"causality broken at row {i}"
        if i + 1 < s:
            assert not np.allclose(got[:, i + 1:], ref[:, i + 1:]), "perturbation had no effect"


def pin_constant_v(fn, seed=15):
    """W_v = 0 and b_v = c make every attention output row equal c."""
    rng = np.random.default_rng(seed)
    b, s, h, heads, f = 2, 11, 8, 2, 8
    for causal in (False, True):
        x, W = rand_layer(rng, b, s, h, f, wstd=0.5)
        W["Wqkv"][:, 2 * h:] = 0.0
        c = rng.standard_normal(h)
        W["bqkv"][2 * h:] = c
        r = _call(fn, x, W, heads, causal)
        _close(r["A"], np.broadcast_to(c, (b, s, h)), 1e-14, "constant V: A")
        _close(r["y"], x + c @ W["Wo"] + W["bo"], 1e-13, "constant V: y")


def pin_uniform_attention(fn, seed=16):
    """W_q = 0, b_q = 0: every score is 0, so attention is the (prefix) mean of V."""
    rng = np.random.default_rng(seed)
    b, s, h, heads, f = 2, 10, 6, 3, 8
    x, W = rand_layer(rng, b, s, h, f, wstd=0.5)
    W["Wqkv"][:, :h] = 0.0
    W["bqkv"][:h] = 0.0
    V = x @ W["Wqkv"][:, 2 * h:] + W["bqkv"][2 * h:]
    prefix = np.cumsum(V, axis=1) / np.arange(1, s + 1)[None, :, None]
    _close(_call(fn, x, W, heads, True)["A"], prefix, 1e-13, "uniform causal")
    _close(_call(fn, x, W, heads, False)["A"], np.broadcast_to(V.mean(axis=1, keepdims=True), V.shape),
           1e-13, "uniform non-causal")


def pin_key_bias_shift(fn, seed=17):
    """Changing b_k adds q_i . b_k to every score of row i: softmax unchanged."""
    rng = np.random.default_rng(seed)
    b, s, h, heads, f = 1, 12, 8, 2, 8
    x, W = rand_layer(rng, b, s, h, f, wstd=0.5)
    for causal in (False, True):
        ref = _call(fn, x, W, heads, causal)["A"]
        W2_ = {k: v.copy() for k, v in W.items()}
        W2_["bqkv"][h:2 * h] += rng.standard_normal(h) * 2.0
        _close(_call(fn, x, W2_, heads, causal)["A"], ref, 1e-12, "key-bias shift")


def pin_permutation(fn, seed=18):
    """Non-causal attention and the position-wise FFN commute with token permutations."""
    rng = np.random.default_rng(seed)
    b, s, h, heads, f = 1, 9, 8, 2, 8
    x, W = rand_layer(rng, b, s, h, f, wstd=0.5)
    perm = rng.permutation(s)
    ref = _call(fn, x, W, heads, False)["out"]
    got = _call(fn, x[:, perm], W, heads, False)["out"]
    _close(got, ref[:, perm], 1e-12, "permutation equivariance")


def pin_zero_weights(fn):
    rng = np.random.default_rng(19)
    x = rng.standard_normal((2, 7, 8))
    W = dict(Wqkv=np.zeros((8, 24)), bqkv=np.zeros(24), Wo=np.zeros((8, 8)), bo=np.zeros(8),
             W1=np.zeros((8, 16)), b1=np.zeros(16), W2=np.zeros((16, 8)), b2=np.zeros(8))
    for causal in (False, True):
        assert np.array_equal(_call(fn, x, W, 2, causal)["out"], x), "zero weights: out != x"


def pin_single_token(fn, seed=20):
    """s = 1: the only key is the query's own, so A = V."""
    rng = np.random.default_rng(seed)
    x, W = rand_layer(rng, 3, 1, 8, 8)
    V = x @ W["Wqkv"][:, 16:] + W["bqkv"][16:]
    for causal in (False, True):
        _close(_call(fn, x, W, 2, causal)["A"], V, 1e-14, "single token")


def pin_large_logits(fn, seed=21):
    """x scaled by 50 drives the scores far past exp's range; the result must
    stay finite and agree with torch's float64 layer."""
    rng = np.random.default_rng(seed)
    x, W = rand_layer(rng, 1, 16, 16, 16, wstd=0.3)
    x = x * 50.0
    for causal in (False, True):
        got = _call(fn, x, W, 2, causal)
        want_out, _ = _torch_layer(x, W, 2, causal)
        _close(got["out"], want_out, 1e-10, f"large logits causal={causal}")


ALL_PINS = [pin_hand_worked, pin_library, pin_blockwise, pin_brute_force, pin_causality,
            pin_constant_v, pin_uniform_attention, pin_key_bias_shift, pin_permutation,
            pin_zero_weights, pin_single_token, pin_large_logits]
