"""The oracle's training-mode dropout against its pins (CPU only).

* The generator: the oracle's own Philox4x64-10 against numpy's independent
  implementation (numpy.random.Philox), whose counter is advanced once before
  each block of four words.
* The mask: the drop fraction T/65536 within binomial bounds, no correlation
  between channels of one 16-channel group or between the two sites, and a
  pure function of (token, channel), so row sampling and chunking cannot
  change it.
* The layer: rate 0 is the inference forward exactly; with W_o = 0 and b_o = c
  (or W_2 = 0 and b_2 = c) a residual branch is the constant c, so each
  output element is x + c·keep·65536/(65536 - T) in closed form.
"""
import numpy as np
import pytest

import oracle
from oracle import bpt_oracle as O
from tests import oracle_pins as pins


def _numpy_philox_block(counter, key):
    """First block of numpy's Philox4x64-10 started one below ``counter``."""
    c = sum(int(v) << (64 * i) for i, v in enumerate(counter)) - 1
    c %= 1 << 256
    start = np.array([(c >> (64 * i)) & (2 ** 64 - 1) for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=start)
    return [int(v) for v in g.random_raw(4)]


@pytest.mark.parametrize("counter,key", [
    ((1, 0, 0, 0), (5, 7)),
    ((0, 1, 0, 0), (0, 0)),  # the reference counter borrows across words
    ((2 ** 64 - 1, 2 ** 64 - 1, 0, 5), (2 ** 64 - 1, 3)),
    ((123, 456, 789, 2 ** 63), (0x0123456789ABCDEF, 1)),
    ((0, 0, 0, 0), (42, 1)),  # wraps to the all-ones reference counter
])
def test_philox_matches_numpy(counter, key):
    mine = O.philox4x64_10([np.uint64(c) for c in counter], key)
    assert [int(np.asarray(w).reshape(-1)[0]) for w in mine] == _numpy_philox_block(counter, key)


def test_philox_is_elementwise():
    rng = np.random.default_rng(70)
    c = [rng.integers(0, 2 ** 63, 50, dtype=np.uint64) for _ in range(4)]
    vec = O.philox4x64_10(c, (9, 1))
    for i in (0, 17, 49):
        one = O.philox4x64_10([ci[i] for ci in c], (9, 1))
        assert [int(np.asarray(v).reshape(-1)[0]) for v in one] == [int(w[i]) for w in vec]


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_drop_fraction(p):
    keep = O.dropout_keep(np.arange(4096), 256, p, seed=11, site=1)
    n = keep.size
    q = O.dropout_threshold(p) / 65536.0
    frac = 1.0 - keep.mean()
    assert abs(frac - q) < 5.0 * np.sqrt(q * (1 - q) / n)
    assert abs(q - p) <= 0.5 / 65536


def test_channels_and_sites_uncorrelated():
    keep0 = O.dropout_keep(np.arange(2048), 64, 0.5, seed=3, site=0).astype(np.float64)
    keep1 = O.dropout_keep(np.arange(2048), 64, 0.5, seed=3, site=1).astype(np.float64)
    lim = 5.0 / np.sqrt(keep0.shape[0])
    # neighbours inside a 16-channel group come from different 16-bit fields
    for a, b in ((0, 1), (3, 4), (0, 15), (15, 16)):
        assert abs(np.corrcoef(keep0[:, a], keep0[:, b])[0, 1]) < lim
    assert abs(np.corrcoef(keep0.ravel(), keep1.ravel())[0, 1]) < 5.0 / np.sqrt(keep0.size)
    other_seed = O.dropout_keep(np.arange(2048), 64, 0.5, seed=4, site=0).astype(np.float64)
    assert abs(np.corrcoef(keep0.ravel(), other_seed.ravel())[0, 1]) < 5.0 / np.sqrt(keep0.size)


def test_mask_is_a_function_of_token_and_channel():
    full = O.dropout_keep(np.arange(300), 96, 0.2, seed=8, site=0)
    tok = np.array([299, 0, 17, 160])
    np.testing.assert_array_equal(O.dropout_keep(tok, 96, 0.2, seed=8, site=0), full[tok])
    np.testing.assert_array_equal(O.dropout_keep(np.arange(300), 48, 0.2, seed=8, site=0),
                                  full[:, :48])


def test_rate_zero_is_the_inference_forward():
    rng = np.random.default_rng(71)
    x, W = pins.rand_layer(rng, 2, 24, 16, 32)
    a = oracle.layer_forward(x, *W.values(), heads=2, causal=True)
    b = oracle.layer_forward(x, *W.values(), heads=2, causal=True, dropout_p=0.0, seed=5)
    for k in ("out", "y", "A"):
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("p", [0.1, 0.37])
def test_closed_form_branches(p):
    rng = np.random.default_rng(72)
    b_, s, h, f = 2, 20, 32, 48
    x, W = pins.rand_layer(rng, b_, s, h, f)
    c_o = rng.standard_normal(h)
    c_2 = rng.standard_normal(h)
    W["Wo"] = np.zeros_like(W["Wo"])
    W["bo"] = c_o
    W["W2"] = np.zeros_like(W["W2"])
    W["b2"] = c_2
    seed = 12345
    r = oracle.layer_forward(x, *W.values(), heads=4, causal=False, dropout_p=p, seed=seed)
    tok = np.arange(b_ * s)
    scale = 65536.0 / (65536.0 - O.dropout_threshold(p))
    k0 = O.dropout_keep(tok, h, p, seed, 0).reshape(b_, s, h)
    k1 = O.dropout_keep(tok, h, p, seed, 1).reshape(b_, s, h)
    y = x + np.where(k0, c_o * scale, 0.0)
    np.testing.assert_allclose(r["y"], y, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["out"], y + np.where(k1, c_2 * scale, 0.0), rtol=0, atol=1e-13)
    # a wrong scale, 1/(1-p) instead of 65536/(65536-T), would miss this
    assert abs(scale - 1.0 / (1.0 - p)) > 1e-9


def test_dropout_row_sampling_is_exact():
    rng = np.random.default_rng(73)
    x, W = pins.rand_layer(rng, 2, 30, 16, 16)
    full = oracle.layer_forward(x, *W.values(), heads=2, causal=True, dropout_p=0.25, seed=9)
    rows = np.array([0, 7, 29])
    part = oracle.layer_forward(x, *W.values(), heads=2, causal=True, dropout_p=0.25, seed=9,
                                rows=rows)
    for k in ("out", "y"):
        np.testing.assert_allclose(part[k], full[k][:, rows], rtol=0, atol=1e-13)


def test_dropout_is_unbiased_on_average():
    # E[D ∘ v / (1 - q)] = v: the mean over many seeds approaches the
    # inference branch (only the branches carry dropout)
    rng = np.random.default_rng(74)
    x, W = pins.rand_layer(rng, 1, 8, 16, 16)
    W["W2"] = np.zeros_like(W["W2"])
    W["b2"] = np.zeros(16)
    ref = oracle.layer_forward(x, *W.values(), heads=2, causal=False)["y"]
    n = 400
    acc = np.zeros_like(ref)
    for seed in range(n):
        acc += oracle.layer_forward(x, *W.values(), heads=2, causal=False, dropout_p=0.3,
                                    seed=seed)["y"]
    branch = ref - x
    err = np.abs(acc / n - ref)
    # per element the estimator's standard deviation is |branch|·sqrt(q/(1-q)/n)
    q = O.dropout_threshold(0.3) / 65536.0
    assert np.all(err <= 6.0 * np.abs(branch) * np.sqrt(q / (1 - q) / n) + 1e-12)


def test_rate_out_of_range_is_rejected():
    with pytest.raises(ValueError):
        O.dropout_threshold(1.0)
    with pytest.raises(ValueError):
        O.dropout_threshold(-0.1)
