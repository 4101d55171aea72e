"""The fp64 oracle against its pins (CPU only).

The oracle must pass every pin in tests/oracle_pins.py. The mutation tests
plant one plausible slip at a time in a layer function written here (never in
the GPU path) and check that some pin catches it, so the pins are known to
bite on a dropped term, a wrong sign or index, or a transposed operand.
"""
import math

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def oracle_fn(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, heads, causal):
    return oracle.layer_forward(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, heads=heads, causal=causal)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_fn)


def test_rows_sum_to_one_and_causal_zeros():
    # debug checklist of the PyTorch 2.3 MHSA page §8: attention weights sum to 1
    rng = np.random.default_rng(30)
    Q = rng.standard_normal((17, 8)) * 3
    K = rng.standard_normal((17, 8)) * 3
    for causal in (False, True):
        P = oracle.attention_probs(Q, K, causal, np.arange(17))
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-14
        assert np.all(P >= 0)
        if causal:
            assert np.all(P[np.triu_indices(17, 1)] == 0.0)
            assert P[0, 0] == 1.0


def test_row_sampling_is_exact():
    rng = np.random.default_rng(31)
    x, W = pins.rand_layer(rng, 2, 40, 8, 8)
    rows = np.array([0, 1, 13, 39])
    for causal in (False, True):
        full = oracle_fn(x, **W, heads=2, causal=causal)
        part = oracle.layer_forward(x, *W.values(), heads=2, causal=causal, rows=rows, row_chunk=3)
        for k in ("out", "y", "A"):
            np.testing.assert_allclose(part[k], full[k][:, rows], rtol=0, atol=1e-13)


def test_stack_of_two_closed_form():
    """Two layers whose composition has a closed form:
    layer 1 is FFN-only (Wqkv = Wo = 0, bo = 0), so out1 = x + relu(x W1 + b1) W2 + b2;
    layer 2 has constant values (V = c for every token, Wo = I) and an FFN
    that is off (W1 = 0, b1 = -1), so out2 = out1 + c + b2'. A stack that fed
    layer 2 the input x instead of out1 would give x + c + b2'."""
    rng = np.random.default_rng(33)
    b, s, h, f, heads = 2, 7, 8, 12, 2
    x = rng.standard_normal((b, s, h))
    W1 = rng.standard_normal((h, f)) * 0.5
    b1 = rng.standard_normal(f) * 0.3
    W2 = rng.standard_normal((f, h)) * 0.5
    b2 = rng.standard_normal(h) * 0.3
    l1 = (np.zeros((h, 3 * h)), np.zeros(3 * h), np.zeros((h, h)), np.zeros(h), W1, b1, W2, b2)
    c = rng.standard_normal(h)
    bqkv2 = np.concatenate([rng.standard_normal(2 * h), c])  # Q, K biases arbitrary; V = c
    Wqkv2 = np.concatenate([rng.standard_normal((h, 2 * h)), np.zeros((h, h))], axis=1)
    b2b = rng.standard_normal(h)
    l2 = (Wqkv2, bqkv2, np.eye(h), np.zeros(h), np.zeros((h, f)), -np.ones(f),
          rng.standard_normal((f, h)), b2b)
    want = x + np.maximum(0.0, x @ W1 + b1) @ W2 + b2 + c + b2b
    for causal in (True, False):
        got = oracle.stack_forward(x, [l1, l2], heads=heads, causal=causal)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # and the slip this pins: layer 2 applied to x
    slip = oracle.layer_forward(x, *l2, heads=heads, causal=True)["out"]
    assert np.max(np.abs(slip - want)) > 0.1


def test_stack_of_one_is_the_layer():
    rng = np.random.default_rng(32)
    x, W = pins.rand_layer(rng, 1, 6, 4, 4)
    one = oracle.stack_forward(x, [tuple(W.values())], heads=2, causal=True)
    np.testing.assert_array_equal(one, oracle_fn(x, **W, heads=2, causal=True)["out"])


# ---------------------------------------------------------------------------
# mutation tests: each slip must fail at least one pin
# ---------------------------------------------------------------------------
def _slipped_layer(slip):
    def fn(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, heads, causal):
        x = np.asarray(x, dtype=np.float64)
        b, s, h = x.shape
        d = h // heads
        qkv = x @ Wqkv + bqkv
        q, k, v = qkv[..., :h], qkv[..., h:2 * h], qkv[..., 2 * h:]
        if slip == "swap_k_v":
            k, v = v, k
        split = lambda t: t.reshape(b, s, heads, d).transpose(0, 2, 1, 3)
        Q, K, V = split(q), split(k), split(v)
        scale = {"no_scale": 1.0, "scale_by_h": 1 / math.sqrt(h)}.get(slip, 1 / math.sqrt(d))
        S = np.einsum("bnid,bnjd->bnij", Q, K) * scale
        if causal:
            i = np.arange(s)[:, None]
            j = np.arange(s)[None, :]
            keep = (j < i) if slip == "mask_off_by_one" else (j >= i) if slip == "mask_flipped" else (j <= i)
            S = np.where(keep, S, -np.inf)
        if slip == "no_max_subtraction":
            E = np.exp(S)
        else:
            E = np.exp(S - S.max(axis=-1, keepdims=True))
        P = E / E.sum(axis=-1, keepdims=True)
        Ah = P @ V
        if slip == "merge_without_transpose":
            A = Ah.reshape(b, s, h)
        else:
            A = Ah.transpose(0, 2, 1, 3).reshape(b, s, h)
        Wo_ = Wo.T if slip == "wo_transposed" else Wo
        resid = q if slip == "residual_is_query" else x
        y = resid + A @ Wo_ + (0 if slip == "drop_bo" else bo)
        pre = y @ W1 + b1
        H = pre if slip == "no_relu" else np.maximum(0.0, pre)
        f_out = H @ W2 + (0 if slip == "drop_b2" else b2)
        out = f_out if slip == "no_second_residual" else y + f_out
        if slip == "ffn_on_x":
            out = y + np.maximum(0.0, x @ W1 + b1) @ W2 + b2
        return {"out": out, "y": y, "A": A}
    return fn


SLIPS = ["swap_k_v", "no_scale", "scale_by_h", "mask_off_by_one", "mask_flipped",
         "no_max_subtraction", "merge_without_transpose", "wo_transposed", "residual_is_query",
         "drop_bo", "no_relu", "drop_b2", "no_second_residual", "ffn_on_x"]


def test_unslipped_variant_passes_all_pins():
    fn = _slipped_layer(None)
    for pin in pins.ALL_PINS:
        pin(fn)


@pytest.mark.parametrize("slip", SLIPS)
def test_pins_catch_slip(slip):
    fn = _slipped_layer(slip)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the slip {slip!r}"
