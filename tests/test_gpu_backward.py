"""The layer backward on the GPU (bpt_layer_bwd, bf16) against the oracle.

Every gradient (dx and the fp32 gradients of the eight parameters, in the
library's [out, in] weight layout) is compared element by element with the
oracle's float64 layer_backward on the same bf16 inputs: max|gpu - oracle| /
max|oracle| within 2e-2, the bar of the bf16 forward. The shapes cover head
dims 32, 64 and 128, both causal modes, sequence lengths that are not a
multiple of 32 (zero-padded token axes), several FFN groups (the weight
gradients accumulate across groups) and ragged GEMM tiles.

ReLU decisions. The FFN's on/off decision [y·W1 + b1 > 0] is a
floating-point decision, so the inputs settle every one of them by
construction and the oracle takes them all by itself, in float64; no GPU
value reaches an oracle call:

* feature 0 of x is ±3 (seeded signs); the attention neither reads it (row 0
  of Wqkv, in the oracle's [in, out] layout, is zero) nor writes it (column 0
  of Wo and bo[0] are zero), so y[:, 0] = x[:, 0] exactly on both sides;
* row 0 of W1 is λ·v with v = ±1 (seeded), so every pre-activation carries a
  term ±3λ. y does not depend on W1, so λ is chosen from the oracle's y.

The forward gate holds the GPU's y within E = 2e-2·max|y_oracle| of the
oracle's (checked here too, through bpt_debug_intermediates), so the GPU's
pre-activation differs from the oracle's by at most
    δ[t, j] = E·Σ_{i>=1} |W1[i, j]| + (h+1)·2^-24·((|y[t]| + E)·|W1[:, j]| + |b1[j]|)
(the second term bounds the fp32 accumulation of bf16 products). Each test
asserts min(|pre_oracle| - δ) > 0 over the rows it checks before comparing;
then both sides take every decision alike and the gradients are compared with
no slack. The large feature reaches dy[:, 0] (so dx[:, 0], the gradient of
Wo's output row 0 and dbo[0]) but not the attention, since Wo's column 0 is
zero; such parts are compared on their own scale, the rest on theirs.
"""
import numpy as np
import pytest

from oracle import bpt_oracle as O
from tests.gpu_helpers import TOL, make, rel_inf, say

pytestmark = pytest.mark.gpu

# gradients in the library's layout, and the parts compared on their own
# scale (index expressions into the library-layout array)
GRADS = [("dWqkv", True), ("dbqkv", False), ("dWo", True), ("dbo", False), ("dW1", True),
         ("db1", False), ("dW2", True), ("db2", False)]
PARTS = {
    "dx": [(np.s_[..., :1], "[:, 0]"), (np.s_[..., 1:], "[:, 1:]")],
    "dWqkv": [(np.s_[:, :1], "[:, 0]"), (np.s_[:, 1:], "[:, 1:]")],
    "dWo": [(np.s_[:1, :], "[0, :]"), (np.s_[1:, :], "[1:, :]")],
    "dbo": [(np.s_[:1], "[0]"), (np.s_[1:], "[1:]")],
    "dW1": [(np.s_[:, :1], "[:, 0]"), (np.s_[:, 1:], "[:, 1:]")],
}


def _bf16(a):
    import torch
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def decided_inputs(x, lw, heads, causal, seed, rows=None, dropout_p=0.0, drop_seed=0):
    """The inputs described above: x and the weights with feature 0 isolated
    and a ±λ row 0 of W1, λ the smallest integer >= 2 for which the margin
    holds with a quarter to spare. Returns (x, lw, margin report). ``rows``
    restricts the rows the margin is asserted for (the rows a test checks);
    ``dropout_p`` and ``drop_seed`` select the training-mode forward (its y
    keeps feature 0 too: the attention branch is zero there, dropped or
    not)."""
    rng = np.random.default_rng(seed)
    x = x.copy()
    b, s, h = x.shape
    x[..., 0] = np.where(rng.random((b, s)) < 0.5, -3.0, 3.0).astype(np.float32)
    Wqkv, bqkv, Wo, bo, W1, b1, W2, b2 = [a.copy() for a in lw.as_tuple()]
    Wqkv[0, :] = 0.0
    Wo[:, 0] = 0.0
    bo[0] = 0.0
    v = np.where(rng.random(W1.shape[1]) < 0.5, -1.0, 1.0)
    yref = O.layer_forward(x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, heads=heads, causal=causal,
                           rows=rows, dropout_p=dropout_p, seed=drop_seed)["y"]
    assert np.all(yref[..., 0] == x[..., 0] if rows is None else yref[..., 0] == x[:, rows, 0])
    y2 = yref.reshape(-1, h)
    E = TOL["bf16"] * float(np.max(np.abs(y2)))
    W1a, b1a = np.abs(W1.astype(np.float64)), np.abs(b1.astype(np.float64))
    rest = y2[:, 1:] @ W1[1:, :].astype(np.float64) + b1
    base = E * W1a[1:, :].sum(axis=0)

    def delta(lam):
        col = W1a.copy()
        col[0, :] = lam
        return base + (h + 1) * 2.0 ** -24 * ((np.abs(y2) + E) @ col + b1a)

    lam = 2
    while True:
        pre = 3.0 * lam * np.sign(y2[:, :1]) * v + rest
        slack = np.abs(pre) - delta(lam)
        if float(slack.min()) > 0.25 * 3.0 * lam:
            break
        lam += 1
    W1[0, :] = (lam * v).astype(np.float32)
    # y is unchanged by W1; the margin now holds for every checked (t, j)
    pre = y2 @ W1.astype(np.float64) + b1
    margin = float((np.abs(pre) - delta(lam)).min())
    assert margin > 0.0, margin
    from blockwise_attention_ffn_amd import inputs
    lw2 = inputs.LayerWeights(Wqkv, bqkv, Wo, bo, W1, b1, W2, b2)
    return x, lw2, {"lambda": lam, "margin": margin, "E": E, "yref": yref}


def _gpu_backward(x, lw, heads, ffn, causal, B_q, B_kv, G, ffn_rows=0, dropout_p=None,
                  drop_seed=0):
    """bpt_layer_bwd, or bpt_layer_bwd_train when ``dropout_p`` is given."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    xd = L.upload(x, "bf16")
    wd = L.upload_weights(lw, "bf16")
    Gd = L.upload(G, "bf16")
    sh = L.shape_for(xd, heads, ffn, "bf16")
    h = x.shape[-1]
    ws = torch.empty(B.bpt_layer_bwd_workspace_bytes(sh, B_q, B_kv, causal, ffn_rows),
                     dtype=torch.uint8, device="cuda")
    dx = torch.empty_like(xd)
    shapes = {"dWqkv": (3 * h, h), "dbqkv": (3 * h,), "dWo": (h, h), "dbo": (h,),
              "dW1": (ffn, h), "db1": (ffn,), "dW2": (h, ffn), "db2": (h,)}
    g = {k: torch.full(v, float("nan"), dtype=torch.float32, device="cuda")
         for k, v in shapes.items()}
    if dropout_p is None:
        B.bpt_layer_bwd(sh, xd, *wd.as_tuple(), B_q, B_kv, causal, ffn_rows, Gd, dx,
                        *[g[k] for k, _ in GRADS], ws)
    else:
        B.bpt_layer_bwd_train(sh, xd, *wd.as_tuple(), B_q, B_kv, causal, ffn_rows, dropout_p,
                              drop_seed, Gd, dx, *[g[k] for k, _ in GRADS], ws)
    torch.cuda.synchronize()
    out = {"dx": L.to_f64(dx)}
    out.update({k: v.double().cpu().numpy() for k, v in g.items()})
    return out


def _gpu_y_gate(tag, x, lw, heads, ffn, causal, B_q, B_kv, info, rows=None):
    """The forward gate on y that the decision margin assumes (GPU y against
    the oracle's), and y[:, 0] = x[:, 0] exactly."""
    from tests.gpu_helpers import run_gpu
    _, _, y = run_gpu(x, lw, heads, ffn, "bf16", causal, B_q, B_kv)
    if rows is not None:
        y = y[:, rows, :]
    xs = x if rows is None else x[:, rows, :]
    e = rel_inf(y, info["yref"])
    say(f"{tag}: y gate {e:.2e}; λ = {info['lambda']}, decision margin {info['margin']:.3f} "
        f"(E = {info['E']:.3f})")
    assert e <= TOL["bf16"], e
    assert np.array_equal(y[..., 0], xs[..., 0].astype(np.float64))


def _check(tag, got, ref, x):
    """Every gradient part within 2e-2 of its own largest entry, except
    dWqkv[:, 0] = Σ_t x[t, 0]·dQKV[t, :]. Feature 0 of x is ±3 with random
    signs, so that sum cancels heavily (its largest entry is ~10× below the
    other rows'), and the bf16 storage of dQKV alone (2^-9 per element)
    moves it by up to 3.6e-2 of its own largest entry at these shapes
    (rounding the oracle's dQKV to bf16 on the CPU; one training case
    cancels 180-fold). It is held instead to 2^-9 (one bf16 rounding unit)
    of max_j Σ_t |x[t, 0]|·|dQKV[t, j]|, the scale that bounds the rounding
    error of such a sum, from the oracle's dQKV: the storage rounding alone
    comes to 1.2e-4 – 4.9e-4 of it at these shapes."""
    errs = {}
    for k in ["dx"] + [g for g, _ in GRADS]:
        is_w = dict(GRADS).get(k, False)
        want = ref[k].T if is_w else ref[k]  # oracle weights are [in, out]
        for sl, name in PARTS.get(k, [(np.s_[...], "")]):
            if k == "dWqkv" and name == "[:, 0]":
                x0 = np.abs(np.asarray(x, np.float64)[..., 0]).reshape(-1)
                terms = x0 @ np.abs(ref["dQKV"]).reshape(-1, ref["dQKV"].shape[-1])
                # reported in units of the part's bar: <= 1 passes like the rest
                errs[k + name + " (/ 2^-9·Σ|terms|, x 2e-2)"] = (
                    float(np.max(np.abs(got[k][sl] - want[sl]))) / (2.0 ** -9 * float(np.max(terms)))
                    * TOL["bf16"])
                continue
            errs[k + name] = rel_inf(got[k][sl], want[sl])
    say(f"{tag}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"{tag}: {bad}"


# (b, s, h, nh, f, causal, B_q, B_kv, ffn_rows). The attention kernels walk
# their blocks of 32 four per loop iteration from block 1, so the last 0 to 3
# take one of four tail paths; with the sequence lengths from 160 on, every
# path of every kernel is taken at every head dim (test_backward_cover.py
# checks this on the CPU).
SMALL_SHAPES = [
    (1, 128, 128, 2, 256, True, 64, 64, 0),      # d = 64
    (2, 272, 256, 2, 512, True, 16, 16, 48),     # d = 128, s % 32 = 16, 12 FFN groups
    (1, 256, 128, 4, 192, False, 64, 128, 128),  # d = 32, non-causal, 2 groups
    (2, 336, 128, 4, 192, True, 48, 112, 0),     # d = 32, N and M tails
    (1, 512, 256, 2, 512, False, 128, 128, 256), # d = 128, non-causal
    (1, 1024, 512, 4, 1024, True, 256, 128, 512),
    (1, 176, 256, 2, 256, True, 16, 176, 0),     # d = 128, tails of 1 (dV, dK, dQ) and 3 (dQ)
    (1, 208, 256, 2, 256, False, 208, 16, 0),    # d = 128, tails of 2
    (1, 224, 128, 2, 256, True, 32, 112, 0),     # d = 64, tails of 2 and 3
    (1, 176, 128, 2, 192, False, 16, 16, 0),     # d = 64, tails of 1
    (1, 160, 128, 2, 192, True, 32, 80, 0),      # d = 64, tails of 0
    (1, 160, 128, 4, 192, False, 160, 32, 0),    # d = 32, tails of 0
    (1, 176, 128, 4, 192, True, 176, 16, 0),     # d = 32, tails of 1 and 3
]


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv,ffn_rows", SMALL_SHAPES)
def test_backward_small_shapes(b, s, h, nh, f, causal, B_q, B_kv, ffn_rows):
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=f, seq=s, batch=b,
                       bias_std=0.05)
    x, lw, info = decided_inputs(x, lw, nh, causal, seed=2000 + s)
    rng = np.random.default_rng(1000 + s)
    G = _bf16(rng.standard_normal(x.shape))
    tag = f"bwd b{b} s{s} h{h} nh{nh} f{f} causal={causal} B_q={B_q} B_kv={B_kv} ffn_rows={ffn_rows}"
    say(f"case {tag}")
    _gpu_y_gate(tag, x, lw, nh, f, causal, B_q, B_kv, info)
    got = _gpu_backward(x, lw, nh, f, causal, B_q, B_kv, G, ffn_rows)
    ref = O.layer_backward(x, *lw.as_tuple(), G, heads=nh, causal=causal)
    _check(tag, got, ref, x)


def test_backward_is_deterministic():
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=256, batch=2)
    G = _bf16(np.random.default_rng(5).standard_normal(x.shape))
    say("case bwd repeat")
    a = _gpu_backward(x, lw, 2, 512, True, 64, 64, G, 128)
    b = _gpu_backward(x, lw, 2, 512, True, 64, 64, G, 128)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.slow
def test_backward_c2_recipe_at_seq_1024():
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", seq=1024)
    x, lw, info = decided_inputs(x, lw, w.heads, w.causal, seed=2006)
    G = _bf16(np.random.default_rng(6).standard_normal(x.shape))
    tag = f"bwd c2 recipe {x.shape}"
    say(f"case {tag}")
    _gpu_y_gate(tag, x, lw, w.heads, w.ffn, w.causal, w.B_q, w.B_kv, info)
    got = _gpu_backward(x, lw, w.heads, w.ffn, w.causal, w.B_q, w.B_kv, G)
    ref = O.layer_backward(x, *lw.as_tuple(), G, heads=w.heads, causal=w.causal)
    _check(tag, got, ref, x)


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["c2_bf16_b2_s8k_h2048", "c3_bf16_s32k_h2048",
                                   "c4_bf16_s16k_h4096"])
def test_full_size_causal_tail_and_bias_identities(wname):
    """Full workload sizes, in the launch configuration bench.py times (the
    workload's B_q and B_kv, the default FFN group):

    * dx of the last 64 positions of every sequence, element by element,
      against the oracle's layer_backward_causal_tail (exact for those rows:
      with a causal mask only the tail queries see the tail keys, and only
      the tail rows' ReLU decisions reach their dx). These rows take the
      longest path of the dQ kernel (every key block) and the dK / dV
      kernels' last tiles.
    * Two identities that hold at any size and cover every dK and dV tile:
      softmax rows sum to one, so the K-bias gradient Σ_t dK[t] is zero and
      the V-bias gradient Σ_t dV[t] equals Σ_q dO[q] = dbo·Wo^T. The GPU's
      sums carry the bf16 rounding of each dK / dV element (relative 2^-9,
      random in sign), so db_k is held to 2e-2 of the K-weight gradient's
      scale (of the same sums weighted by x) and db_v to 2e-2 of dbo·Wo^T
      (dbo[0], large here, does not enter it: Wo's column 0 is zero).

    The inputs are the workload's with the decision construction above;
    the margin is asserted for the tail rows.
    """
    w, x, (lw,) = make(wname)
    assert w.causal
    tail = 64
    b, s, h = x.shape
    rows = np.arange(s - tail, s)
    x, lw, info = decided_inputs(x, lw, w.heads, True, seed=2100 + s, rows=rows)
    G = _bf16(np.random.default_rng(7).standard_normal(x.shape))
    tag = f"bwd full size {wname} {x.shape} B_q={w.B_q} B_kv={w.B_kv} tail={tail}"
    say(f"case {tag}")
    _gpu_y_gate(tag, x, lw, w.heads, w.ffn, True, w.B_q, w.B_kv, info, rows=rows)
    got = _gpu_backward(x, lw, w.heads, w.ffn, True, w.B_q, w.B_kv, G, 0)
    for k, v in got.items():
        assert np.all(np.isfinite(v)), f"non-finite {k}"
    ref = O.layer_backward_causal_tail(x, *lw.as_tuple(), G, heads=w.heads, tail=tail)["dx"]
    gpu = got["dx"][:, s - tail:, :]
    e0 = rel_inf(gpu[..., :1], ref[..., :1])
    e1 = rel_inf(gpu[..., 1:], ref[..., 1:])
    Wo = np.asarray(lw.Wo, np.float64)
    e_k = float(np.max(np.abs(got["dbqkv"][h:2 * h]))) / float(np.max(np.abs(got["dWqkv"][h:2 * h])))
    e_v = rel_inf(got["dbqkv"][2 * h:], Wo @ got["dbo"])
    say(f"{tag}: dx[:, 0] {e0:.2e} dx[:, 1:] {e1:.2e}; db_k / |dW_k| {e_k:.2e}; "
        f"db_v vs dbo·Wo^T {e_v:.2e}")
    assert e0 <= TOL["bf16"], e0
    assert e1 <= TOL["bf16"], e1
    assert e_k <= TOL["bf16"], e_k
    assert e_v <= TOL["bf16"], e_v


# ---------------------------------------------------------------------------
# Backward of the training-mode forward (bpt_layer_bwd_train)
def _gpu_train_y(x, lw, heads, ffn, causal, B_q, B_kv, p, seed):
    """The training-mode forward's y on the GPU: bpt_layer_fwd_train with the
    FFN switched off (W1 = W2 = b2 = 0, so the FFN branch is zero whether
    dropped or not) returns out = y."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import inputs
    from blockwise_attention_ffn_amd import layer as L
    Wqkv, bqkv, Wo, bo, W1, b1, W2, b2 = lw.as_tuple()
    lw0 = inputs.LayerWeights(Wqkv, bqkv, Wo, bo, np.zeros_like(W1), b1, np.zeros_like(W2),
                              np.zeros_like(b2))
    xd, wd = L.upload(x, "bf16"), L.upload_weights(lw0, "bf16")
    sh = L.shape_for(xd, heads, ffn, "bf16")
    ws = L.alloc_workspace(sh, B_q, B_kv, causal)
    out = torch.empty_like(xd)
    B.bpt_layer_fwd_train(sh, xd, *wd.as_tuple(), B_q, B_kv, causal, 0, p, seed, out, ws)
    torch.cuda.synchronize()
    return L.to_f64(out)


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv,ffn_rows,p,seed", [
    (1, 128, 128, 2, 256, True, 64, 64, 0, 0.1, 7),        # d = 64
    (2, 272, 256, 2, 512, True, 16, 16, 48, 0.3, 8),       # d = 128, s % 32 = 16, 12 FFN groups
    (1, 256, 128, 4, 192, False, 64, 128, 128, 0.5, 9),    # d = 32, non-causal, 2 groups
])
def test_training_backward_small_shapes(b, s, h, nh, f, causal, B_q, B_kv, ffn_rows, p, seed):
    """Every gradient of the training-mode forward against the oracle's
    layer_backward with the same dropout rate and seed, element by element;
    the decisions settled as above, for the training-mode y."""
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=f, seq=s, batch=b,
                       bias_std=0.05)
    x, lw, info = decided_inputs(x, lw, nh, causal, seed=2200 + s, dropout_p=p, drop_seed=seed)
    G = _bf16(np.random.default_rng(1200 + s).standard_normal(x.shape))
    tag = (f"bwd train p={p} seed={seed} b{b} s{s} h{h} nh{nh} f{f} causal={causal} "
           f"B_q={B_q} B_kv={B_kv} ffn_rows={ffn_rows}")
    say(f"case {tag}")
    y = _gpu_train_y(x, lw, nh, f, causal, B_q, B_kv, p, seed)
    e = rel_inf(y, info["yref"])
    say(f"{tag}: training-mode y gate {e:.2e}; λ = {info['lambda']}, margin {info['margin']:.3f}")
    assert e <= TOL["bf16"], e
    assert np.array_equal(y[..., 0], x[..., 0].astype(np.float64))
    got = _gpu_backward(x, lw, nh, f, causal, B_q, B_kv, G, ffn_rows, dropout_p=p, drop_seed=seed)
    ref = O.layer_backward(x, *lw.as_tuple(), G, heads=nh, causal=causal, dropout_p=p, seed=seed)
    _check(tag, got, ref, x)
    # the masks matter: the inference backward's gradients differ from these
    plain = O.layer_backward(x, *lw.as_tuple(), G, heads=nh, causal=causal)
    assert rel_inf(plain["dW2"], ref["dW2"]) > 10 * TOL["bf16"]


def test_training_backward_rate_zero_is_the_inference_backward():
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=256, batch=2)
    G = _bf16(np.random.default_rng(15).standard_normal(x.shape))
    say("case bwd train p=0")
    a = _gpu_backward(x, lw, 2, 512, True, 64, 64, G, 128)
    b = _gpu_backward(x, lw, 2, 512, True, 64, 64, G, 128, dropout_p=0.0, drop_seed=123)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv,ffn_rows,p", [
    (1, 512, 256, 2, 512, True, 256, 64, 0, 0.0),     # d = 128, the 256 x 64 tile
    (1, 272, 256, 2, 512, True, 16, 16, 0, 0.2),      # s = 17 x 16, 16 x 16 blocks, dropout
    (2, 192, 128, 4, 256, False, 64, 64, 128, 0.3),   # d = 32, three FFN groups, dropout
    (1, 512, 256, 4, 384, True, 256, 128, 256, 0.1),  # d = 64, two FFN groups, dropout
    (1, 32768, 2048, 16, 8192, True, 1024, 512, 0, 0.0),  # the 32K workload as bench.py times it
])
def test_backward_from_kept_activations_is_bitwise_the_recomputing_one(b, s, h, nh, f, causal,
                                                                         B_q, B_kv, ffn_rows, p):
    """bpt_layer_fwd_for_bwd followed by bpt_layer_bwd_from_fwd against
    bpt_layer_bwd_train with the same arguments: the kept activations come from
    the same kernels on the same inputs as the recomputed ones, so dx and every
    weight gradient agree bit for bit (and through bpt_layer_bwd_train, which
    the tests above hold to the oracle, with the oracle). The pair's out is
    the training-mode forward's: bit for bit at the 256-row, 64-key attention
    tile both then run, within the bf16 bar of each other otherwise."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    if (b, s, h, nh, f) == (1, 32768, 2048, 16, 8192):
        w, x, (lw,) = make("c3_bf16_s32k_h2048")  # the workload's own recipe
    else:
        w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=f, seq=s, batch=b,
                           bias_std=0.05)
    G = _bf16(np.random.default_rng(1700 + s).standard_normal(x.shape))
    seed = 31
    tag = (f"kept b{b} s{s} h{h} nh{nh} f{f} causal={causal} B_q={B_q} B_kv={B_kv} "
           f"ffn_rows={ffn_rows} p={p}")
    say(f"case {tag}")
    xd = L.upload(x, "bf16")
    wd = L.upload_weights(lw, "bf16").as_tuple()
    Gd = L.upload(G, "bf16")
    sh = L.shape_for(xd, nh, f, "bf16")
    nbytes = B.bpt_layer_bwd_workspace_bytes(sh, B_q, B_kv, causal, ffn_rows)
    shapes = [(3 * h, h), (3 * h,), (h, h), (h,), (f, h), (f,), (h, f), (h,)]

    def grads():
        return [torch.full(v, float("nan"), dtype=torch.float32, device="cuda") for v in shapes]
    ws_k = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out_k, dx_k, g_k = torch.empty_like(xd), torch.empty_like(xd), grads()
    B.bpt_layer_fwd_for_bwd(sh, xd, *wd, B_q, B_kv, causal, ffn_rows, p, seed, out_k, ws_k)
    B.bpt_layer_bwd_from_fwd(sh, xd, *wd, B_q, B_kv, causal, ffn_rows, p, seed, Gd, dx_k, *g_k,
                             ws_k)
    ws_r = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dx_r, g_r = torch.empty_like(xd), grads()
    B.bpt_layer_bwd_train(sh, xd, *wd, B_q, B_kv, causal, ffn_rows, p, seed, Gd, dx_r, *g_r, ws_r)
    ws_f = torch.empty(B.bpt_layer_workspace_bytes_ex(sh, B_q, B_kv, causal, ffn_rows),
                       dtype=torch.uint8, device="cuda")
    out_t = torch.empty_like(xd)
    B.bpt_layer_fwd_train(sh, xd, *wd, B_q, B_kv, causal, ffn_rows, p, seed, out_t, ws_f)
    torch.cuda.synchronize()
    assert torch.equal(dx_k, dx_r), tag
    for (name, _), a, r in zip(GRADS, g_k, g_r):
        assert torch.equal(a, r), (tag, name)
    assert not torch.isnan(g_k[0]).any()
    same_tile = B_q % 256 == 0 and B_kv % 64 == 0
    e = rel_inf(L.to_f64(out_k), L.to_f64(out_t))
    say(f"{tag}: gradients bitwise equal; out against the training forward {e:.2e}")
    if same_tile:
        assert torch.equal(out_k, out_t), tag
    else:
        assert e <= TOL["bf16"], e
