"""GPU path (HIP kernels behind the C ABI) against the fp64 oracle.

Small shapes: every output element. Full workload sizes: a row sample (rows
0, 1, s-1, both edges of every query block, seeded random rows) that the
oracle computes exactly with full keys. Bars: max|gpu-oracle|/max|oracle|
<= 1e-4 (fp32) or 2e-2 (bf16 storage, fp32 accumulation) on out, A and y.
"""
import numpy as np
import pytest

import oracle
from blockwise_attention_ffn_amd import inputs
from tests.gpu_helpers import TOL, check_against_oracle, make, rel_inf, run_gpu, say

pytestmark = pytest.mark.gpu


def _oracle(x, lw, heads, causal, rows=None):
    return oracle.layer_forward(x, *lw.as_tuple(), heads=heads, causal=causal, rows=rows)


# ---------------------------------------------------------------------------
def test_c1_fp32_exact_workload():
    w, x, (lw,) = make("c1_fp32_s256_h64")
    say(f"case c1 fp32 {x.shape} B_q={w.B_q} B_kv={w.B_kv} causal={w.causal}")
    gpu = run_gpu(x, lw, w.heads, w.ffn, "f32", w.causal, w.B_q, w.B_kv)
    check_against_oracle("c1", gpu, _oracle(x, lw, w.heads, w.causal), "f32")


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv", [
    (1, 256, 64, 2, 256, True, 64, 64),
    (2, 272, 64, 2, 128, True, 16, 16),      # ragged: s = 17 x 16
    (1, 208, 256, 4, 192, False, 16, 208),   # d = 64, single KV block
    (1, 144, 256, 2, 320, True, 144, 48),    # d = 128, single query block
])
def test_fp32_shapes(b, s, h, nh, f, causal, B_q, B_kv):
    w, x, (lw,) = make("c1_fp32_s256_h64", hidden=h, heads=nh, ffn=f, bias_std=0.05,
                       seq=s, batch=b)
    say(f"case fp32 b{b} s{s} h{h} nh{nh} f{f} causal={causal} B_q={B_q} B_kv={B_kv}")
    gpu = run_gpu(x, lw, nh, f, "f32", causal, B_q, B_kv)
    check_against_oracle("fp32", gpu, _oracle(x, lw, nh, causal), "f32")


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv", [
    (2, 592, 256, 2, 512, True, 16, 16),     # s = 37 x 16: ragged against 64/256 tiles
    (1, 592, 256, 2, 512, False, 16, 592),
    (1, 1024, 256, 4, 256, True, 64, 128),   # d = 64
    (2, 336, 128, 4, 192, True, 48, 112),    # d = 32, N and M tails in every GEMM
    (1, 512, 384, 3, 320, False, 128, 256),  # h, f not multiples of the 256 tile
    (1, 16, 128, 1, 64, True, 16, 16),       # one block of 16 tokens
])
def test_bf16_small_shapes(b, s, h, nh, f, causal, B_q, B_kv):
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=f, seq=s, batch=b)
    say(f"case bf16 b{b} s{s} h{h} nh{nh} f{f} causal={causal} B_q={B_q} B_kv={B_kv}")
    gpu = run_gpu(x, lw, nh, f, "bf16", causal, B_q, B_kv)
    check_against_oracle("bf16-small", gpu, _oracle(x, lw, nh, causal), "bf16")


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv", [
    (1, 592, 2048, 16, 2048, True, 16, 16),   # K = 2048 everywhere, ragged rows
    (2, 336, 1344, 21, 1408, False, 48, 112),  # d = 64, h = 10.5 tiles of 128, K = 1344 / 1408
    (1, 256, 1280, 10, 1280, True, 64, 64),    # K = 1280: 40 steps of 32
])
def test_bf16_long_k_shapes(b, s, h, nh, f, causal, B_q, B_kv):
    # every row of GEMMs with long K (many steps per tile) and ragged tiles
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=f, seq=s, batch=b)
    say(f"case bf16 long-K b{b} s{s} h{h} nh{nh} f{f} causal={causal} B_q={B_q} B_kv={B_kv}")
    gpu = run_gpu(x, lw, nh, f, "bf16", causal, B_q, B_kv)
    check_against_oracle("bf16-long-k", gpu, _oracle(x, lw, nh, causal), "bf16")


def test_c2_recipe_at_seq_1024_every_row():
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", seq=1024)
    say(f"case c2-recipe {x.shape} causal={w.causal}")
    gpu = run_gpu(x, lw, w.heads, w.ffn, "bf16", w.causal, w.B_q, w.B_kv)
    check_against_oracle("c2@1024", gpu, _oracle(x, lw, w.heads, w.causal), "bf16")


# (B_q, B_kv) pairs that select every attention tile: query rows per
# workgroup 16..256 x keys per stage 16, 32, 64 (bpt_layer_attention_tile)
TILE_BLOCKS = [(16, 16), (16, 32), (16, 64), (32, 16), (32, 32), (32, 64), (64, 16), (64, 32),
               (64, 64), (128, 16), (128, 32), (384, 64), (256, 16), (768, 32), (256, 256)]


@pytest.mark.parametrize("d", [32, 64, 128])
def test_every_attention_tile(d):
    """Each (query rows, keys per stage) tile of the bf16 attention, selected
    through B_q and B_kv, against the oracle's A on every element, causal and
    not, at seq 768 (3 x 256) with batch 2: the workgroups' causal ranges
    end inside and at the edges of stages, and a 16-row tile uses half of
    the 32-wide MFMA tile."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    h = 256
    nh = h // d
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=256, seq=768, batch=2)
    xd, wd = L.upload(x, "bf16"), L.upload_weights(lw, "bf16")
    sh = L.shape_for(xd, nh, 256, "bf16")
    seen = set()
    for causal in (True, False):
        ref = _oracle(x, lw, nh, causal)["A"]
        for bq, bkv in TILE_BLOCKS:
            tile = B.bpt_layer_attention_tile(sh, bq, bkv)
            seen.add(tile)
            ws = L.alloc_workspace(sh, bq, bkv, causal)
            A = torch.empty_like(xd)
            B.bpt_debug_attention(sh, xd, wd.Wqkv, wd.bqkv, bq, bkv, causal, True, A, ws)
            torch.cuda.synchronize()
            e = rel_inf(L.to_f64(A), ref)
            say(f"case tile d={d} causal={causal} B_q={bq} B_kv={bkv} -> {tile}: A {e:.2e}")
            assert e <= TOL["bf16"], (tile, e)
    assert len(seen) == 15, sorted(seen)


@pytest.mark.parametrize("b,s,h,nh,f,causal,B_q,B_kv,ffn_rows", [
    (2, 272, 256, 2, 512, True, 16, 16, 48),     # 11 full FFN groups and a 16-row last one
    (1, 592, 384, 3, 640, False, 16, 592, 0),    # one group; h, f not multiples of 256
    (1, 1024, 2048, 16, 2048, True, 512, 512, 512),  # h = 2048, K = 2048, two groups
])
def test_ffn_branch_dominates(b, s, h, nh, f, causal, B_q, B_kv, ffn_rows):
    """a4 and a5 gated on their own in bf16: W1 and W2 drawn with standard
    deviation 0.2 (ten times the recipe's), so the FFN term out - y is several
    times the residual stream y and the 2e-2 bar on out bounds the FFN's own
    error. Also the last FFN group's hidden activations H (bounded scratch)
    against the oracle's H = max(0, y W1 + b1), from the oracle's own y."""
    import torch
    from blockwise_attention_ffn_amd import layer as L
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=nh, ffn=f, seq=s, batch=b)
    lw.W1[...] = inputs.round_to_bf16(lw.W1 * np.float32(10.0))
    lw.W2[...] = inputs.round_to_bf16(lw.W2 * np.float32(10.0))
    ref = _oracle(x, lw, nh, causal)
    ratio = float(np.max(np.abs(ref["out"] - ref["y"])) / np.max(np.abs(ref["y"])))
    tag = f"ffn-dominant b{b} s{s} h{h} f{f} ffn_rows={ffn_rows}"
    say(f"case {tag}: max|out - y| / max|y| = {ratio:.1f}")
    assert ratio >= 3.0, ratio
    xd, wd = L.upload(x, "bf16"), L.upload_weights(lw, "bf16")
    sh = L.shape_for(xd, nh, f, "bf16")
    out, A, y, H = L.layer_forward_debug(sh, xd, wd, B_q, B_kv, causal, ffn_rows=ffn_rows,
                                         want_H=True)
    torch.cuda.synchronize()
    gpu = (L.to_f64(out), L.to_f64(A), L.to_f64(y))
    check_against_oracle(tag, gpu, ref, "bf16")
    n = H.shape[0]
    y2 = ref["y"].reshape(-1, h)[-n:]
    H_ref = np.maximum(0.0, y2 @ lw.W1.astype(np.float64) + lw.b1)
    e_H = rel_inf(L.to_f64(H), H_ref)
    say(f"{tag}: last group H ({n} rows) {e_H:.2e}")
    assert e_H <= TOL["bf16"], e_H


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["c2_bf16_b2_s8k_h2048", "c3_bf16_s32k_h2048",
                                   "c4_bf16_s16k_h4096"])
def test_full_size_sampled_rows(wname):
    w, x, (lw,) = make(wname)
    rows = inputs.sample_rows(w.seq, w.B_q, 48)
    say(f"case {wname} {x.shape} B_q={w.B_q} B_kv={w.B_kv} rows={len(rows)}")
    gpu = run_gpu(x, lw, w.heads, w.ffn, "bf16", w.causal, w.B_q, w.B_kv)
    ref = _oracle(x, lw, w.heads, w.causal, rows=rows)
    check_against_oracle(wname, gpu, ref, "bf16", rows=rows)


@pytest.mark.slow
def test_c3_block_sweep_agrees():
    """The 32K workload at every point of its 3 x 3 block grid and of the
    pages' grid B_q = B_kv in {16, 64, 128, 256, 512, 1024, 2048, 4096} (the
    points bench.py --sweep times; attention tiles from 16 x 16 to 256 x 64):
    sampled rows (every 512-row block edge, 24 random rows, both edges of a
    16-row tile among them) against the oracle, and every point against the
    first on every element."""
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    w, x, (lw,) = make("c3_bf16_s32k_h2048")
    rows = inputs.sample_rows(w.seq, 512, 24)
    rows = np.unique(np.concatenate([rows, [16, 31, 4096 + 47]]))
    ref = _oracle(x, lw, w.heads, w.causal, rows=rows)
    pts = [(q, k) for q in w.sweep_q for k in w.sweep_kv]
    pts += [(b, b) for b in (16, 64, 128, 256, 512, 1024, 2048, 4096) if (b, b) not in pts]
    sh = B.make_shape(1, w.seq, w.hidden, w.heads, w.ffn, "bf16")
    tiles = set()
    first = None
    for B_q, B_kv in pts:
        tile = B.bpt_layer_attention_tile(sh, B_q, B_kv)
        tiles.add(tile)
        say(f"case c3 sweep B_q={B_q} B_kv={B_kv} (attention tile {tile})")
        out, _, _ = run_gpu(x, lw, w.heads, w.ffn, "bf16", w.causal, B_q, B_kv, debug=False)
        e = rel_inf(out[:, rows], ref["out"])
        say(f"  out vs oracle {e:.2e}")
        assert e <= TOL["bf16"]
        if first is None:
            first = out
        else:
            assert rel_inf(out, first) <= TOL["bf16"]
        del out
    assert {(16, 16), (64, 64), (128, 64), (256, 64)} <= tiles


@pytest.mark.slow
def test_c5_stack_per_layer():
    import torch
    from blockwise_attention_ffn_amd import layer as L
    w, x, layers = make("c5_bf16_s128k_h2048_x4")
    rows = inputs.sample_rows(w.seq, w.B_q, 16)
    xd = L.upload(x, "bf16")
    wds = [L.upload_weights(lw, "bf16") for lw in layers]
    sh = L.shape_for(xd, w.heads, w.ffn, "bf16")
    say(f"case c5 stack {x.shape} layers={len(layers)} rows={len(rows)}")
    final, outs = L.stack_forward(sh, xd, wds, w.B_q, w.B_kv, w.causal, keep_all=True)
    torch.cuda.synchronize()
    prev = x
    for li, (lw, od) in enumerate(zip(layers, outs)):
        got = L.to_f64(od)
        ref = _oracle(prev, lw, w.heads, w.causal, rows=rows)
        e = rel_inf(got[:, rows], ref["out"])
        say(f"  layer {li}: out vs oracle(gpu layer input) {e:.2e}")
        assert e <= TOL["bf16"]
        prev = got.astype(np.float32)  # bf16 values, exact in float32
        del got


@pytest.mark.slow
def test_c5_recipe_end_to_end_at_seq_2048():
    """The 4-layer recipe (independent weights per layer, h 2048, 16 heads,
    f 8192, causal, B_q 2048, B_kv 1024) at seq 2048, every row:

    * per layer, the GPU's layer l against the oracle's layer l applied to the
      GPU's layer l-1 output, at the 2e-2 bar;
    * end to end, the GPU stack's final output against oracle.stack_forward on
      the same input. The bf16 rounding of every layer compounds here: each
      layer adds its own error and passes the earlier ones on, so the stack
      is held to the sum of the four per-layer bars, 4 x 2e-2, and the value
      is reported."""
    import torch
    from blockwise_attention_ffn_amd import layer as L
    w, x, layers = make("c5_bf16_s128k_h2048_x4", seq=2048)
    xd = L.upload(x, "bf16")
    wds = [L.upload_weights(lw, "bf16") for lw in layers]
    sh = L.shape_for(xd, w.heads, w.ffn, "bf16")
    say(f"case c5 recipe end to end {x.shape} layers={len(layers)}")
    final, outs = L.stack_forward(sh, xd, wds, w.B_q, w.B_kv, w.causal, keep_all=True)
    torch.cuda.synchronize()
    prev = x
    for li, (lw, od) in enumerate(zip(layers, outs)):
        got = L.to_f64(od)
        e = rel_inf(got, _oracle(prev, lw, w.heads, w.causal)["out"])
        say(f"  layer {li}: out vs oracle(gpu layer input) {e:.2e}")
        assert e <= TOL["bf16"], (li, e)
        prev = got.astype(np.float32)
    ref = oracle.stack_forward(x, [lw.as_tuple() for lw in layers], heads=w.heads,
                               causal=w.causal)
    e = rel_inf(L.to_f64(final), ref)
    say(f"  4-layer out vs oracle.stack_forward {e:.2e} (bar {len(layers) * TOL['bf16']:.0e})")
    assert e <= len(layers) * TOL["bf16"], e


# ---------------------------------------------------------------------------
# properties of the GPU path
def test_causality_bitwise():
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=768, batch=1)
    out0, _, _ = run_gpu(x, lw, 2, 512, "bf16", True, 128, 64, debug=False)
    for i in (0, 200, 511, 700):
        xp = x.copy()
        xp[:, i + 1:] = inputs.round_to_bf16(xp[:, i + 1:] * 3.0 + 1.0)
        out1, _, _ = run_gpu(xp, lw, 2, 512, "bf16", True, 128, 64, debug=False)
        say(f"case causality row {i}")
        assert np.array_equal(out1[:, :i + 1], out0[:, :i + 1])
        assert not np.array_equal(out1[:, i + 1:], out0[:, i + 1:])


def test_repeat_runs_are_bitwise_identical():
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=512, heads=4, ffn=1024, seq=1024, batch=2)
    a = run_gpu(x, lw, 4, 1024, "bf16", True, 256, 256)
    b = run_gpu(x, lw, 4, 1024, "bf16", True, 256, 256)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_calls_on_two_streams_with_their_own_workspaces():
    """Calls are reentrant across streams when their workspaces differ: two
    layers of different shapes (bf16 and fp32), enqueued three times each on two
    streams of default priority without waiting for each other, give the bits
    the same calls give one after the other on one stream."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    specs = [("c2_bf16_b2_s8k_h2048", "bf16", dict(hidden=512, heads=4, ffn=1024, seq=1024, batch=2),
              True, 256, 128),
             ("c1_fp32_s256_h64", "f32", dict(hidden=128, heads=4, ffn=256, seq=528, batch=1),
              False, 48, 16)]
    calls = []
    for wname, dtype, over, causal, B_q, B_kv in specs:
        w, x, (lw,) = make(wname, bias_std=0.05, **over)
        xd = L.upload(x, dtype)
        wd = L.upload_weights(lw, dtype).as_tuple()
        sh = L.shape_for(xd, over["heads"], over["ffn"], dtype)
        ws = torch.empty(B.bpt_layer_workspace_bytes(sh, B_q, B_kv, causal), dtype=torch.uint8,
                         device="cuda")
        calls.append((sh, xd, wd, B_q, B_kv, causal, ws))
    say("case two streams: bf16 b2 s1024 h512 and fp32 b1 s528 h128, three calls each")
    refs = []
    for sh, xd, wd, B_q, B_kv, causal, ws in calls:
        out = torch.empty_like(xd)
        B.bpt_layer_fwd(sh, xd, *wd, B_q, B_kv, causal, out, ws)
        torch.cuda.synchronize()
        refs.append(out)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.full_like(r, float("nan")) for _ in range(3)] for r in refs]
    torch.cuda.synchronize()
    for rep in range(3):
        for k, (sh, xd, wd, B_q, B_kv, causal, ws) in enumerate(calls):
            B.bpt_layer_fwd(sh, xd, *wd, B_q, B_kv, causal, outs[k][rep], ws, streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        for rep in range(3):
            assert torch.equal(outs[k][rep], refs[k]), (k, rep)


def test_constant_v_and_uniform_attention():
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=256, seq=512, batch=1)
    h = 256
    # constant V: W_v = 0, b_v = c
    lw.Wqkv[:, 2 * h:] = 0.0
    c = inputs.round_to_bf16(np.random.default_rng(5).standard_normal(h).astype(np.float32))
    lw.bqkv[2 * h:] = c
    for causal in (False, True):
        out, A, y = run_gpu(x, lw, 2, 256, "bf16", causal, 64, 64)
        assert rel_inf(A, np.broadcast_to(c, A.shape)) <= 4e-3
    # uniform attention: W_q = 0, b_q = 0
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=256, seq=512, batch=1)
    lw.Wqkv[:, :h] = 0.0
    lw.bqkv[:h] = 0.0
    gpu = run_gpu(x, lw, 2, 256, "bf16", True, 64, 64)
    check_against_oracle("uniform", gpu, _oracle(x, lw, 2, True), "bf16")


def test_large_logits_fp32_parity():
    # x * 20 drives the logits to O(10^2), past the float32 range of exp
    # without the running max. The fp32 path must still meet its 1e-4 bar.
    w, x, (lw,) = make("c1_fp32_s256_h64", hidden=256, heads=2, ffn=256, seq=256, batch=1)
    x = x * np.float32(20.0)
    for causal in (False, True):
        say(f"case fp32 x*20 causal={causal}")
        gpu = run_gpu(x, lw, 2, 256, "f32", causal, 64, 64)
        ref = _oracle(x, lw, 2, causal)
        assert np.max(np.abs(x)) > 60.0
        check_against_oracle("fp32 x*20", gpu, ref, "f32")


def test_large_logits_bf16():
    # At logits of O(10^3) the bf16 rounding of Q and K alone moves scores by
    # O(1), so the bf16 path is held to what holds at any precision: finite
    # results, and every attention row a convex combination of the value rows
    # it may see. A milder scale (x * 4) is held to the bf16 parity bar.
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=256, seq=512, batch=1)
    xs = inputs.round_to_bf16(x * 50.0)
    out, A, y = run_gpu(xs, lw, 2, 256, "bf16", True, 64, 64)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(A))
    h = 256
    V = xs.astype(np.float64) @ lw.Wqkv[:, 2 * h:] + lw.bqkv[2 * h:]
    lo = np.minimum.accumulate(V, axis=1)
    hi = np.maximum.accumulate(V, axis=1)
    slack = 0.01 * (np.max(np.abs(V)))
    assert np.all(A >= lo - slack) and np.all(A <= hi + slack)
    x4 = inputs.round_to_bf16(x * 4.0)
    gpu = run_gpu(x4, lw, 2, 256, "bf16", True, 64, 64)
    check_against_oracle("bf16 x*4", gpu, _oracle(x4, lw, 2, True), "bf16")


@pytest.mark.parametrize("jump,d", [(48.0, 128), (150.0, 128), (48.0, 64), (48.0, 32)])
def test_score_jump_moves_the_reference_max(jump, d):
    # Every key of the second half of the sequence gets the same extra score
    # of `jump` log2 units: feature 0 of x is 1 there and 0 elsewhere, only
    # head-dim 0 of K reads it (K0 = B exactly), and head-dim 0 of Q is the
    # constant bias A (Q0 = A exactly). The running reference max, set by the
    # first stage, must then move past a weight of 2^jump (jump 150 overflows
    # exp2 in fp32) in the middle of the key walk, in bulk and diagonal
    # stages, causal and not. The offset is one number per query row, so its
    # bf16 rounding cancels in the softmax and the bf16 parity bar applies.
    h = 256
    heads = h // d
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=h, heads=heads, ffn=256, seq=1024, batch=1)
    s = x.shape[1]
    x[:, :, 0] = 0.0
    x[:, s // 2:, 0] = 1.0
    lw.Wqkv[0, :] = 0.0
    A_q = 16.0
    B_k = float(inputs.round_to_bf16(np.array([jump * np.sqrt(d) / np.log2(np.e) / A_q],
                                                dtype=np.float32))[0])
    for n in range(heads):
        lw.Wqkv[:, n * d] = 0.0           # Q dim 0 = bias only
        lw.bqkv[n * d] = A_q
        lw.Wqkv[:, h + n * d] = 0.0       # K dim 0 = B * feature 0 only
        lw.Wqkv[0, h + n * d] = B_k
        lw.bqkv[h + n * d] = 0.0
    for causal in (False, True):
        say(f"case score jump {jump} d={d} causal={causal}")
        gpu = run_gpu(x, lw, heads, 256, "bf16", causal, 64, 128)
        check_against_oracle(f"jump {jump}", gpu, _oracle(x, lw, heads, causal), "bf16")


def test_in_place_equals_out_of_place_and_no_stray_writes():
    import torch
    from blockwise_attention_ffn_amd import layer as L
    from blockwise_attention_ffn_amd import binding as B
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=528, batch=2)
    xd = L.upload(x, "bf16")
    wd = L.upload_weights(lw, "bf16")
    sh = L.shape_for(xd, 2, 512, "bf16")
    ref = L.layer_forward(sh, xd, wd, 48, 176, True)
    # guard bands around out and the workspace
    n = xd.numel()
    pad = 4096
    big = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[pad:pad + n].view_as(xd)
    wsn = B.bpt_layer_workspace_bytes(sh, 48, 176, True)
    wsbig = torch.full((wsn + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = wsbig[pad:pad + wsn]
    L.layer_forward(sh, xd, wd, 48, 176, True, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.all(big[:pad] == 7.0) and torch.all(big[pad + n:] == 7.0)
    assert torch.all(wsbig[:pad] == 0x5A) and torch.all(wsbig[pad + wsn:] == 0x5A)
    # in place: out is x
    xi = xd.clone()
    B.bpt_layer_fwd(sh, xi, *wd.as_tuple(), 48, 176, True, xi, ws)
    torch.cuda.synchronize()
    assert torch.equal(xi, ref)


def test_debug_attention_matches_layer_A():
    import torch
    from blockwise_attention_ffn_amd import layer as L
    from blockwise_attention_ffn_amd import binding as B
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=512, heads=4, ffn=512, seq=1024, batch=1)
    xd = L.upload(x, "bf16")
    wd = L.upload_weights(lw, "bf16")
    sh = L.shape_for(xd, 4, 512, "bf16")
    _, A, _ = L.layer_forward_debug(sh, xd, wd, 256, 256, True)
    ws = L.alloc_workspace(sh, 256, 256, True)
    A2 = torch.empty_like(xd)
    B.bpt_debug_attention(sh, xd, wd.Wqkv, wd.bqkv, 256, 256, True, True, A2, ws)
    A3 = torch.empty_like(xd)
    B.bpt_debug_attention(sh, xd, wd.Wqkv, wd.bqkv, 256, 256, True, False, A3, ws)
    torch.cuda.synchronize()
    assert torch.equal(A, A2) and torch.equal(A2, A3)


def test_ffn_group_size_does_not_change_the_result():
    import torch
    from blockwise_attention_ffn_amd import layer as L
    from blockwise_attention_ffn_amd import binding as B
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=1024, batch=2)
    xd = L.upload(x, "bf16")
    wd = L.upload_weights(lw, "bf16")
    sh = L.shape_for(xd, 2, 512, "bf16")
    ref = L.layer_forward(sh, xd, wd, 128, 256, True)
    for rows in (128, 384, 1024, 2048):
        ws = torch.empty(B.bpt_layer_workspace_bytes_ex(sh, 128, 256, True, rows),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty_like(xd)
        B.bpt_layer_fwd_ex(sh, xd, *wd.as_tuple(), 128, 256, True, rows, out, ws)
        torch.cuda.synchronize()
        say(f"case ffn group rows {rows}")
        assert torch.equal(out, ref)
