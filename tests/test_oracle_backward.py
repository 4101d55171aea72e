"""The oracle's backward (layer_backward) against pins that do not use it.

* Central finite differences of the oracle's own forward (float64): for every
  parameter and for x, the directional derivative of sum(out ∘ G) along a
  random direction, and single elements of each gradient.
* Closed forms: db2 is the column sum of G; with W2 = 0 the FFN branch has no
  gradient (dW1 = db1 = 0) and dx reduces to the attention path; causality:
  an upstream gradient on token 0 alone gives no gradient to later tokens.
"""
import numpy as np
import pytest

from oracle import bpt_oracle as O
from tests import oracle_pins as pins

NAMES = ["Wqkv", "bqkv", "Wo", "bo", "W1", "b1", "W2", "b2"]


def _f(x, W, G, heads, causal):
    out = O.layer_forward(x, *[W[k] for k in NAMES], heads=heads, causal=causal)["out"]
    return float(np.sum(out * G))


def _grads(x, W, G, heads, causal):
    return O.layer_backward(x, *[W[k] for k in NAMES], G, heads=heads, causal=causal)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("b,s,h,f,heads", [(2, 6, 8, 12, 2), (1, 9, 12, 8, 3)])
def test_directional_derivatives(b, s, h, f, heads, causal):
    rng = np.random.default_rng(81 + s)
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = rng.standard_normal((b, s, h))
    g = _grads(x, W, G, heads, causal)
    eps = 1e-6
    for name in ["x"] + NAMES:
        base = x if name == "x" else W[name]
        V = rng.standard_normal(base.shape)
        def at(t):
            if name == "x":
                return _f(base + t * V, W, G, heads, causal)
            W2 = dict(W)
            W2[name] = base + t * V
            return _f(x, W2, G, heads, causal)
        fd = (at(eps) - at(-eps)) / (2 * eps)
        an = float(np.sum(g["d" + name] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_single_elements():
    rng = np.random.default_rng(90)
    b, s, h, f, heads = 1, 5, 8, 8, 2
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = rng.standard_normal((b, s, h))
    g = _grads(x, W, G, heads, True)
    eps = 1e-6
    for name in ["x"] + NAMES:
        base = x if name == "x" else W[name]
        for _ in range(3):
            idx = tuple(rng.integers(0, n) for n in base.shape)
            E = np.zeros_like(base)
            E[idx] = 1.0
            def at(t):
                if name == "x":
                    return _f(base + t * E, W, G, heads, True)
                W2 = dict(W)
                W2[name] = base + t * E
                return _f(x, W2, G, heads, True)
            fd = (at(eps) - at(-eps)) / (2 * eps)
            an = float(g["d" + name][idx])
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


def test_closed_forms():
    rng = np.random.default_rng(91)
    b, s, h, f, heads = 2, 7, 8, 16, 2
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = rng.standard_normal((b, s, h))
    g = _grads(x, W, G, heads, False)
    np.testing.assert_allclose(g["db2"], G.reshape(-1, h).sum(axis=0), rtol=0, atol=1e-12)
    # out is linear in b2 and in bo through y, so db2 and the identity path of
    # dy are exact sums; with W2 = 0 the FFN contributes nothing else
    W0 = dict(W)
    W0["W2"] = np.zeros_like(W["W2"])
    g0 = _grads(x, W0, G, heads, False)
    assert np.all(g0["dW1"] == 0.0) and np.all(g0["db1"] == 0.0)
    np.testing.assert_allclose(g0["dbo"], G.reshape(-1, h).sum(axis=0), rtol=0, atol=1e-12)


def test_causal_gradient_stays_in_the_past():
    rng = np.random.default_rng(92)
    b, s, h, f, heads = 1, 8, 8, 8, 2
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = np.zeros((b, s, h))
    G[:, 3, :] = rng.standard_normal(h)
    g = _grads(x, W, G, heads, True)
    assert np.all(g["dx"][:, 4:, :] == 0.0)
    assert np.any(g["dx"][:, :4, :] != 0.0)


@pytest.mark.parametrize("b1_shift", [100.0, -100.0])
def test_relu_branch_closed_forms(b1_shift):
    """Every pre-activation on (b1 shifted far up): the FFN is the affine map
    y -> (y W1 + b1) W2 + b2, whose gradients are dy = G + G W2^T W1^T,
    dW1 = y^T (G W2^T), db1 = sum_t G W2^T, dW2 = H^T G with H = y W1 + b1.
    Every one off (b1 shifted far down): H = 0, so dW1 = db1 = dW2 = 0 and
    dy = G. Both against the chain rule written out here, per token."""
    rng = np.random.default_rng(93)
    b, s, h, f, heads = 1, 6, 8, 12, 2
    x, W = pins.rand_layer(rng, b, s, h, f)
    W = dict(W)
    W["b1"] = W["b1"] + b1_shift
    G = rng.standard_normal((b, s, h))
    g = _grads(x, W, G, heads, True)
    y = g["y"][0]
    on = b1_shift > 0
    gw2 = G[0] @ W["W2"].T
    if on:
        np.testing.assert_allclose(g["dW1"], y.T @ gw2, rtol=0, atol=1e-10)
        np.testing.assert_allclose(g["db1"], gw2.sum(axis=0), rtol=0, atol=1e-10)
        np.testing.assert_allclose(g["dW2"], (y @ W["W1"] + W["b1"]).T @ G[0], rtol=0, atol=1e-9)
        dy = G[0] + gw2 @ W["W1"].T
    else:
        assert np.all(g["dW1"] == 0.0) and np.all(g["db1"] == 0.0) and np.all(g["dW2"] == 0.0)
        dy = G[0]
    # dy reaches dbo = sum_t dy and dWo = A^T dy
    np.testing.assert_allclose(g["dbo"], dy.sum(axis=0), rtol=0, atol=1e-9)


@pytest.mark.parametrize("b,s,h,f,heads,tail", [(2, 11, 8, 12, 2, 1), (1, 24, 12, 8, 3, 7),
                                                (2, 16, 8, 8, 2, 16)])
def test_causal_tail_against_finite_differences(b, s, h, f, heads, tail):
    """layer_backward_causal_tail (dx of the last positions, computed from the
    tail rows alone) against central differences of the causal forward, along
    random directions supported on the tail rows and on single elements."""
    rng = np.random.default_rng(300 + s)
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = rng.standard_normal((b, s, h))
    r = O.layer_backward_causal_tail(x, *[W[k] for k in NAMES], G, heads=heads, tail=tail)
    assert list(r["rows"]) == list(range(s - tail, s))
    dx = np.zeros_like(x)
    dx[:, s - tail:] = r["dx"]
    eps = 1e-6
    for _ in range(3):
        V = np.zeros_like(x)
        V[:, s - tail:] = rng.standard_normal((b, tail, h))
        fd = (_f(x + eps * V, W, G, heads, True) - _f(x - eps * V, W, G, heads, True)) / (2 * eps)
        an = float(np.sum(dx * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
    for _ in range(4):
        idx = (int(rng.integers(0, b)), int(rng.integers(s - tail, s)), int(rng.integers(0, h)))
        E = np.zeros_like(x)
        E[idx] = 1.0
        fd = (_f(x + eps * E, W, G, heads, True) - _f(x - eps * E, W, G, heads, True)) / (2 * eps)
        assert abs(fd - dx[idx]) <= 1e-6 * max(1.0, abs(dx[idx])), (idx, fd, dx[idx])


def test_causal_tail_equals_the_full_backward():
    """The tail function returns the full backward's dx rows (a consistency
    check on top of the finite-difference pins above)."""
    rng = np.random.default_rng(310)
    b, s, h, f, heads = 2, 40, 16, 24, 4
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = rng.standard_normal((b, s, h))
    full = _grads(x, W, G, heads, True)["dx"]
    for tail in (1, 9, 40):
        t = O.layer_backward_causal_tail(x, *[W[k] for k in NAMES], G, heads=heads, tail=tail)["dx"]
        assert np.abs(t - full[:, s - tail:]).max() <= 1e-12 * np.abs(full).max()


# ---------------------------------------------------------------------------
# Training mode: the backward through both dropout masks, against central
# differences of the training-mode forward (the masks are fixed by the seed,
# so the forward is a smooth function of x and the weights between ReLU
# switches).
def _f_train(x, W, G, heads, causal, p, seed):
    out = O.layer_forward(x, *[W[k] for k in NAMES], heads=heads, causal=causal,
                          dropout_p=p, seed=seed)["out"]
    return float(np.sum(out * G))


@pytest.mark.parametrize("p,seed", [(0.25, 3), (0.5, 11)])
@pytest.mark.parametrize("causal", [True, False])
def test_training_mode_directional_derivatives(p, seed, causal):
    b, s, h, f, heads = 2, 7, 16, 12, 2
    rng = np.random.default_rng(400 + seed)
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = rng.standard_normal((b, s, h))
    g = O.layer_backward(x, *[W[k] for k in NAMES], G, heads=heads, causal=causal,
                         dropout_p=p, seed=seed)
    # the masks are not all ones or all zeros, so both branches are exercised
    for site in (0, 1):
        keep = O.dropout_keep(np.arange(b * s), h, p, seed, site)
        assert 0 < keep.mean() < 1
    eps = 1e-6
    for name in ["x"] + NAMES:
        base = x if name == "x" else W[name]
        V = rng.standard_normal(base.shape)

        def at(t):
            if name == "x":
                return _f_train(base + t * V, W, G, heads, causal, p, seed)
            W2 = dict(W)
            W2[name] = base + t * V
            return _f_train(x, W2, G, heads, causal, p, seed)
        fd = (at(eps) - at(-eps)) / (2 * eps)
        an = float(np.sum(g["d" + name] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    # and the forward it differentiates is layer_forward's training mode
    out = O.layer_forward(x, *[W[k] for k in NAMES], heads=heads, causal=causal,
                          dropout_p=p, seed=seed)["out"]
    assert np.array_equal(g["out"], out)


def test_training_mode_rate_zero_is_the_inference_backward():
    rng = np.random.default_rng(420)
    x, W = pins.rand_layer(rng, 1, 6, 8, 8)
    G = rng.standard_normal((1, 6, 8))
    a = _grads(x, W, G, 2, True)
    b = O.layer_backward(x, *[W[k] for k in NAMES], G, heads=2, causal=True, dropout_p=0.0,
                         seed=99)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_training_mode_causal_tail_equals_the_full_backward():
    rng = np.random.default_rng(430)
    b, s, h, f, heads = 2, 24, 16, 24, 4
    x, W = pins.rand_layer(rng, b, s, h, f)
    G = rng.standard_normal((b, s, h))
    full = O.layer_backward(x, *[W[k] for k in NAMES], G, heads=heads, causal=True,
                            dropout_p=0.3, seed=5)["dx"]
    for tail in (1, 8, 24):
        t = O.layer_backward_causal_tail(x, *[W[k] for k in NAMES], G, heads=heads, tail=tail,
                                         dropout_p=0.3, seed=5)["dx"]
        assert np.abs(t - full[:, s - tail:]).max() <= 1e-12 * np.abs(full).max()
