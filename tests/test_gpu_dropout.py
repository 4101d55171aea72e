"""Training-mode dropout on the GPU (bpt_layer_fwd_train) against the oracle.

* The keep masks, bit for bit: the GPU's generator (bpt_debug_dropout_keep,
  the same device code as the GEMM epilogues) against the oracle's
  Philox4x64-10 masks.
* The layer: max|gpu - oracle| / max|oracle| on out within 1e-4 (fp32) or
  2e-2 (bf16), on shapes with several FFN groups (so the token offset of
  each group's mask matters), ragged sequence lengths and both causal modes.
* Rate 0 is the inference forward bit for bit, and the output does not
  depend on the FFN group size.
"""
import numpy as np
import pytest

import oracle
from blockwise_attention_ffn_amd import inputs
from tests.gpu_helpers import TOL, make, rel_inf, say

pytestmark = pytest.mark.gpu


def _train(x, lw, heads, ffn, dtype, causal, B_q, B_kv, p, seed, ffn_rows=0):
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    xd = L.upload(x, dtype)
    wd = L.upload_weights(lw, dtype)
    sh = L.shape_for(xd, heads, ffn, dtype)
    ws = torch.empty(B.bpt_layer_workspace_bytes_ex(sh, B_q, B_kv, causal, ffn_rows),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(xd)
    B.bpt_layer_fwd_train(sh, xd, *wd.as_tuple(), B_q, B_kv, causal, ffn_rows, p, seed, out, ws)
    torch.cuda.synchronize()
    return out, xd, wd, sh


def _check(tag, out, ref, dtype, rows=None):
    from blockwise_attention_ffn_amd import layer as L
    got = L.to_f64(out)
    if rows is not None:
        got = got[:, rows, :]
    e = rel_inf(got, ref)
    say(f"{tag}: out {e:.2e}")
    assert e <= TOL[dtype], f"{tag}: {e:.3e} > {TOL[dtype]}"


@pytest.mark.parametrize("tokens,channels,token0,p,seed,site", [
    (1000, 256, 0, 0.1, 42, 0),
    (333, 2048, 12345, 0.5, 2 ** 64 - 1, 1),
    (64, 16, 2 ** 40, 0.9, 7, 0),
    (2048, 2048, 0, 0.1, 1, 1),
    (17, 48, 3, 0.0, 5, 0),
])
def test_mask_bit_exact(tokens, channels, token0, p, seed, site):
    import torch
    from blockwise_attention_ffn_amd import binding as B
    say(f"case mask tokens={tokens} channels={channels} token0={token0} p={p} site={site}")
    keep = torch.empty((tokens, channels), dtype=torch.uint8, device="cuda")
    B.bpt_debug_dropout_keep(tokens, channels, token0, p, seed, site, keep)
    torch.cuda.synchronize()
    got = keep.cpu().numpy()
    assert set(np.unique(got)) <= {0, 1}
    ref = oracle.dropout_keep(np.arange(token0, token0 + tokens), channels, p, seed, site)
    np.testing.assert_array_equal(got.astype(bool), ref)


def test_c1_fp32_workload_with_dropout():
    w, x, (lw,) = make("c1_fp32_s256_h64")
    say(f"case c1 fp32 train {x.shape} p=0.1")
    out, *_ = _train(x, lw, w.heads, w.ffn, "f32", w.causal, w.B_q, w.B_kv, 0.1, 2024)
    ref = oracle.layer_forward(x, *lw.as_tuple(), heads=w.heads, causal=w.causal,
                               dropout_p=0.1, seed=2024)
    _check("c1-train", out, ref["out"], "f32")


@pytest.mark.parametrize("dtype,b,s,h,nh,f,causal,B_q,B_kv,ffn_rows,p", [
    ("f32", 2, 272, 64, 2, 128, True, 16, 16, 48, 0.2),     # ragged, 12 FFN groups
    ("f32", 1, 144, 256, 2, 320, False, 144, 48, 0, 0.5),
    ("bf16", 2, 592, 256, 2, 512, True, 16, 16, 160, 0.1),  # ragged against the 256 tiles
    ("bf16", 1, 1024, 256, 4, 256, True, 64, 128, 256, 0.3),
    ("bf16", 2, 336, 128, 4, 192, False, 48, 112, 0, 0.1),  # d = 32, N and M tails
    ("bf16", 1, 592, 2048, 16, 2048, True, 16, 16, 256, 0.1),  # K = 2048, ragged rows
])
def test_train_small_shapes(dtype, b, s, h, nh, f, causal, B_q, B_kv, ffn_rows, p):
    base = "c1_fp32_s256_h64" if dtype == "f32" else "c2_bf16_b2_s8k_h2048"
    w, x, (lw,) = make(base, hidden=h, heads=nh, ffn=f, seq=s, batch=b, bias_std=0.05)
    say(f"case train {dtype} b{b} s{s} h{h} nh{nh} f{f} causal={causal} B_q={B_q} "
        f"B_kv={B_kv} ffn_rows={ffn_rows} p={p}")
    out, *_ = _train(x, lw, nh, f, dtype, causal, B_q, B_kv, p, 99, ffn_rows)
    ref = oracle.layer_forward(x, *lw.as_tuple(), heads=nh, causal=causal, dropout_p=p, seed=99)
    _check(f"train-{dtype}", out, ref["out"], dtype)


def test_rate_zero_is_the_inference_forward_bitwise():
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=512, batch=2)
    say("case train p=0 vs inference")
    out, xd, wd, sh = _train(x, lw, 2, 512, "bf16", True, 128, 128, 0.0, 5, 256)
    ws = torch.empty(B.bpt_layer_workspace_bytes_ex(sh, 128, 128, True, 256), dtype=torch.uint8,
                     device="cuda")
    ref = torch.empty_like(xd)
    B.bpt_layer_fwd_ex(sh, xd, *wd.as_tuple(), 128, 128, True, 256, ref, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_train_output_does_not_depend_on_ffn_group_size():
    import torch
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=1024, batch=2)
    first = None
    for rows in (128, 384, 2048):
        say(f"case train ffn group rows {rows}")
        out, *_ = _train(x, lw, 2, 512, "bf16", True, 128, 256, 0.1, 77, rows)
        if first is None:
            first = out
        else:
            assert torch.equal(out, first)


def test_seed_changes_the_masks():
    import torch
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=128, heads=1, ffn=128, seq=256, batch=1)
    say("case train seeds differ")
    a, *_ = _train(x, lw, 1, 128, "bf16", True, 64, 64, 0.5, 1)
    b, *_ = _train(x, lw, 1, 128, "bf16", True, 64, 64, 0.5, 2)
    assert not torch.equal(a, b)


@pytest.mark.slow
def test_c3_workload_with_dropout_sampled_rows():
    w, x, (lw,) = make("c3_bf16_s32k_h2048")
    rows = inputs.sample_rows(w.seq, w.B_q, 32)
    say(f"case c3 train {x.shape} p=0.1 rows={len(rows)}")
    out, *_ = _train(x, lw, w.heads, w.ffn, "bf16", w.causal, w.B_q, w.B_kv, 0.1, 31337)
    ref = oracle.layer_forward(x, *lw.as_tuple(), heads=w.heads, causal=w.causal, rows=rows,
                               dropout_p=0.1, seed=31337)
    _check("c3-train", out, ref["out"], "bf16", rows=rows)
