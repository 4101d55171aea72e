"""The layer backward on the GPU (bpt_layer_bwd, bf16) against the oracle.

Every gradient (dx and the fp32 gradients of the eight parameters, in the
library's [out, in] weight layout) is compared element by element with the
oracle's float64 layer_backward on the same bf16 inputs: max|gpu - oracle| /
max|oracle| within 2e-2, the bar of the bf16 forward. The shapes cover head
dims 32, 64 and 128, both causal modes, sequence lengths that are not a
multiple of 32 (zero-padded token axes), several FFN groups (the weight
gradients accumulate across groups) and ragged GEMM tiles.

The ReLU's on/off decision [y·W1 + b1 > 0] is taken by floating point, so
both sides take it in the GPU's precision: the oracle differentiates the branch
the GPU's own bf16 y selects (pre-activations recomputed in float64 from the
GPU forward's y). Only pre-activations within fp32-accumulation distance of
zero (|p| <= 2^-18 · Σ|y|·|W1|) remain undecided; for those few entries dW1
and db1 are allowed, per element, the largest change a flip can make.
"""
import numpy as np
import pytest

from oracle import bpt_oracle as O
from tests.gpu_helpers import TOL, make, rel_inf, say

pytestmark = pytest.mark.gpu

GRADS = [("dWqkv", True), ("dbqkv", False), ("dWo", True), ("dbo", False), ("dW1", True),
         ("db1", False), ("dW2", True), ("db2", False)]


def _bf16(a):
    import torch
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _gpu_backward(x, lw, heads, ffn, causal, B_q, B_kv, G, ffn_rows=0):
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
    B.bpt_layer_bwd(sh, xd, *wd.as_tuple(), B_q, B_kv, causal, ffn_rows, Gd, dx,
                    *[g[k] for k, _ in GRADS], ws)
    torch.cuda.synchronize()
    out = {"dx": L.to_f64(dx)}
    out.update({k: v.double().cpu().numpy() for k, v in g.items()})
    return out


def _gpu_relu_decisions(x, lw, heads, ffn, causal, B_q, B_kv, G):
    """The ReLU decisions of the GPU's precision (from the GPU forward's bf16
    y), and per-element bounds of what the still-undecided ones can change in
    dW1 (oracle [in, out] layout) and db1."""
    from tests.gpu_helpers import run_gpu
    _, _, y_gpu = run_gpu(x, lw, heads, ffn, "bf16", causal, B_q, B_kv)
    _, _, _, _, W1, b1, W2, _ = [np.asarray(a, np.float64) for a in lw.as_tuple()]
    y2 = y_gpu.reshape(-1, y_gpu.shape[-1])
    pre = y2 @ W1 + b1
    amb = np.abs(pre) <= 2.0 ** -18 * (np.abs(y2) @ np.abs(W1))
    dfull = np.abs(G.reshape(-1, G.shape[-1]) @ W2.T) * amb
    mask = (pre > 0.0).reshape(y_gpu.shape[:-1] + (W1.shape[1],))
    return mask, (np.abs(y2).T @ dfull, dfull.sum(axis=0), int(amb.sum()))


def _check(tag, got, ref, slack=None):
    errs = {}
    e = rel_inf(got["dx"], ref["dx"])
    errs["dx"] = e
    for k, is_w in GRADS:
        want = ref[k].T if is_w else ref[k]  # oracle weights are [in, out]
        if slack is not None and k in ("dW1", "db1"):
            sl = slack[0].T if k == "dW1" else slack[1]
            scale = float(np.max(np.abs(want)))
            excess = np.abs(got[k] - want) - sl
            errs[k] = max(0.0, float(np.max(excess))) / scale
        else:
            errs[k] = rel_inf(got[k], want)
    amb = "" if slack is None else f" ({slack[2]} undecided ReLU entries)"
    say(f"{tag}{amb}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"{tag}: {bad}"


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv,ffn_rows", [
    (1, 128, 128, 2, 256, True, 64, 64, 0),      # d = 64
    (2, 272, 256, 2, 512, True, 16, 16, 48),     # d = 128, s % 32 = 16, 12 FFN groups
    (1, 256, 128, 4, 192, False, 64, 128, 128),  # d = 32, non-causal, 2 groups
    (2, 336, 128, 4, 192, True, 48, 112, 0),     # d = 32, N and M tails
    (1, 512, 256, 2, 512, False, 128, 128, 256), # d = 128, non-causal
    (1, 1024, 512, 4, 1024, True, 256, 128, 512),
])
def test_backward_small_shapes(b, s, h, nh, f, causal, B_q, B_kv, ffn_rows):
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=f, seq=s, batch=b,
                       bias_std=0.05)
    rng = np.random.default_rng(1000 + s)
    G = _bf16(rng.standard_normal(x.shape))
    say(f"case bwd b{b} s{s} h{h} nh{nh} f{f} causal={causal} B_q={B_q} B_kv={B_kv} "
        f"ffn_rows={ffn_rows}")
    got = _gpu_backward(x, lw, nh, f, causal, B_q, B_kv, G, ffn_rows)
    mask, slack = _gpu_relu_decisions(x, lw, nh, f, causal, B_q, B_kv, G)
    ref = O.layer_backward(x, *lw.as_tuple(), G, heads=nh, causal=causal, relu_mask=mask)
    _check(f"bwd s{s} h{h} d{h // nh}", got, ref, slack)


def test_backward_is_deterministic():
    import torch
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
    G = _bf16(np.random.default_rng(6).standard_normal(x.shape))
    say(f"case bwd c2 recipe {x.shape}")
    got = _gpu_backward(x, lw, w.heads, w.ffn, w.causal, w.B_q, w.B_kv, G)
    mask, slack = _gpu_relu_decisions(x, lw, w.heads, w.ffn, w.causal, w.B_q, w.B_kv, G)
    ref = O.layer_backward(x, *lw.as_tuple(), G, heads=w.heads, causal=w.causal, relu_mask=mask)
    _check("bwd c2@1024", got, ref, slack)


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["c2_bf16_b2_s8k_h2048", "c3_bf16_s32k_h2048",
                                   "c4_bf16_s16k_h4096"])
def test_full_size_causal_tail_and_bias_identities(wname):
    """Full workload sizes, in the launch configuration bench.py times (the
    workload's B_q and B_kv, the default FFN group):

    * dx of the last 64 positions of every sequence, element by element,
      against the oracle's layer_backward_causal_tail (exact for those rows:
      with a causal mask only the tail queries see the tail keys). These rows
      take the longest path of the dQ kernel (every key block) and the dK / dV
      kernels' last tiles.
    * Two identities that hold at any size and cover every dK and dV tile:
      softmax rows sum to one, so the K-bias gradient Σ_t dK[t] is zero and
      the V-bias gradient Σ_t dV[t] equals Σ_q dO[q] = dbo·Wo^T. The GPU's
      sums carry the bf16 rounding of each dK / dV element (relative 2^-9,
      random in sign), so db_k is held to 2e-2 of the K-weight gradient's
      scale (of the same sums weighted by x ~ N(0,1)) and db_v to 2e-2 of
      dbo·Wo^T.
    """
    from tests.gpu_helpers import run_gpu
    w, x, (lw,) = make(wname)
    assert w.causal
    tail = 64
    b, s, h = x.shape
    G = _bf16(np.random.default_rng(7).standard_normal(x.shape))
    say(f"case bwd full size {wname} {x.shape} B_q={w.B_q} B_kv={w.B_kv} tail={tail}")
    got = _gpu_backward(x, lw, w.heads, w.ffn, True, w.B_q, w.B_kv, G, 0)
    for k, v in got.items():
        assert np.all(np.isfinite(v)), f"non-finite {k}"
    # the ReLU decisions of the tail rows in the GPU's precision (from its own
    # forward's y); an undecided entry (t, j) can move dy[t] by
    # |(G·W2^T)[t, j]|·|W1[:, j]|, twice that covers what reaches dx[t]
    # through the attention
    _, _, y_gpu = run_gpu(x, lw, w.heads, w.ffn, "bf16", True, w.B_q, w.B_kv)
    _, _, Wo, _, W1, b1, W2, _ = [np.asarray(a, np.float64) for a in lw.as_tuple()]
    yt = y_gpu[:, s - tail:, :]
    del y_gpu
    pre = yt @ W1 + b1
    amb = np.abs(pre) <= 2.0 ** -18 * (np.abs(yt) @ np.abs(W1))
    slack = 2.0 * ((np.abs(G[:, s - tail:, :] @ W2.T) * amb) @ np.abs(W1).T)
    ref = O.layer_backward_causal_tail(x, *lw.as_tuple(), G, heads=w.heads, tail=tail,
                                       relu_mask=pre > 0.0)["dx"]
    gpu = got["dx"][:, s - tail:, :]
    scale = float(np.max(np.abs(ref)))
    e_dx = max(0.0, float(np.max(np.abs(gpu - ref) - slack))) / scale
    e_k = float(np.max(np.abs(got["dbqkv"][h:2 * h]))) / float(np.max(np.abs(got["dWqkv"][h:2 * h])))
    e_v = rel_inf(got["dbqkv"][2 * h:], got["dbo"] @ Wo.T)
    say(f"bwd {wname} tail {tail} ({int(amb.sum())} undecided ReLU entries): dx {e_dx:.2e}; "
        f"db_k / |dW_k| {e_k:.2e}; db_v vs dbo·Wo^T {e_v:.2e}")
    assert e_dx <= TOL["bf16"], e_dx
    assert e_k <= TOL["bf16"], e_k
    assert e_v <= TOL["bf16"], e_v
