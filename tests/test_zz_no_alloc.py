"""bpt_layer_fwd_noalloc (the layer with its workspace in the library's fixed
scratch) against bpt_layer_fwd_ex with a caller workspace, through the C ABI.

Same kernels and schedule, so the outputs must be bitwise equal. Two calls in
a row, the second with a smaller input (the scratch keeps the first call's
contents), for bf16 and fp32; the smaller case is also held to the oracle's
bar. A call whose workspace would exceed the scratch is rejected with
BPT_ERR_SCRATCH before anything runs.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import TOL, make, rel_inf, say

pytestmark = pytest.mark.gpu


def _both(x, lw, heads, ffn, dtype, causal, B_q, B_kv, ffn_rows):
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    xd = L.upload(x, dtype)
    wd = L.upload_weights(lw, dtype)
    sh = L.shape_for(xd, heads, ffn, dtype)
    need = B.bpt_layer_workspace_bytes_ex(sh, B_q, B_kv, causal, ffn_rows)
    assert need <= B.NOALLOC_SCRATCH_BYTES, need
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(xd)
    B.bpt_layer_fwd_ex(sh, xd, *wd.as_tuple(), B_q, B_kv, causal, ffn_rows, ref, ws)
    got = torch.full_like(xd, float("nan"))
    B.bpt_layer_fwd_noalloc(sh, xd, *wd.as_tuple(), B_q, B_kv, causal, ffn_rows, got)
    torch.cuda.synchronize()
    return L.to_f64(got), L.to_f64(ref), need


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_entry_point(dtype):
    wname = "c2_bf16_b2_s8k_h2048" if dtype == "bf16" else "c1_fp32_s256_h64"
    cases = [  # (b, s, h, heads, f, causal, B_q, B_kv, ffn_rows): larger first, then smaller
        (2, 1024, 512, 4, 1024, True, 128, 256, 0),
        (1, 272, 256, 2, 512, False, 16, 16, 48),
    ]
    for i, (b, s, h, nh, f, causal, B_q, B_kv, ffn_rows) in enumerate(cases):
        w, x, (lw,) = make(wname, hidden=h, heads=nh, ffn=f, seq=s, batch=b, bias_std=0.05)
        say(f"case noalloc {dtype} call {i}: b{b} s{s} h{h} nh{nh} f{f} causal={causal} "
            f"B_q={B_q} B_kv={B_kv} ffn_rows={ffn_rows}")
        got, ref, need = _both(x, lw, nh, f, dtype, causal, B_q, B_kv, ffn_rows)
        say(f"  workspace {need} bytes; bitwise equal: {np.array_equal(got, ref)}")
        assert np.array_equal(got, ref)
        if i == 1:
            o = oracle.layer_forward(x, *lw.as_tuple(), heads=nh, causal=causal)["out"]
            e = rel_inf(got, o)
            say(f"  vs oracle {e:.2e}")
            assert e <= TOL[dtype]


def test_noalloc_rejects_calls_beyond_the_scratch():
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    sh = B.make_shape(1, 8192, 2048, 16, 8192, "bf16")
    need = B.bpt_layer_workspace_bytes_ex(sh, 512, 512, True, 0)
    assert need > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, 8192, 2048), dtype=torch.bfloat16, device="cuda")
    h, f = 2048, 8192
    wts = [torch.zeros(n, dtype=torch.bfloat16, device="cuda")
           for n in (3 * h * h, 3 * h, h * h, h, f * h, f, h * f, h)]
    out = torch.empty_like(x)
    with pytest.raises(B.BptError) as ei:
        B.bpt_layer_fwd_noalloc(sh, x, *wts, 512, 512, True, 0, out)
    assert ei.value.name == "BPT_ERR_SCRATCH"
    say(f"case noalloc too large: {need} bytes > {B.NOALLOC_SCRATCH_BYTES}: {ei.value.name}")


def test_noalloc_under_graph_capture():
    """The callers the entry point is for: bpt_layer_fwd_noalloc captured into a
    HIP graph (through torch.cuda.graph, on its capture stream) and replayed
    four times. Between replays the program does its own eager work: it
    poisons the graph's output and runs an eager call of another shape, which
    overwrites the shared scratch. Every replay must still give the eager
    call's bits, since the layer reads nothing from the scratch that it did
    not write first. The captured path records kernel launches only (no
    memset, no copy, no allocation)."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import layer as L
    w, x, (lw,) = make("c2_bf16_b2_s8k_h2048", hidden=256, heads=2, ffn=512, seq=512, batch=2,
                       bias_std=0.05)
    w2, x2, (lw2,) = make("c2_bf16_b2_s8k_h2048", hidden=512, heads=4, ffn=1024, seq=272, batch=1,
                          bias_std=0.05)
    say("case noalloc graph: bf16 b2 s512 h256 captured; eager b1 s272 h512 between replays")
    xd, xd2 = L.upload(x, "bf16"), L.upload(x2, "bf16")
    wd, wd2 = L.upload_weights(lw, "bf16").as_tuple(), L.upload_weights(lw2, "bf16").as_tuple()
    sh, sh2 = L.shape_for(xd, 2, 512, "bf16"), L.shape_for(xd2, 4, 1024, "bf16")
    eager = torch.empty_like(xd)
    B.bpt_layer_fwd_noalloc(sh, xd, *wd, 128, 64, True, 0, eager)
    other = torch.empty_like(xd2)
    out = torch.empty_like(xd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        B.bpt_layer_fwd_noalloc(sh, xd, *wd, 128, 64, True, 0, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.bpt_layer_fwd_noalloc(sh, xd, *wd, 128, 64, True, 0, out)
    for rep in range(4):
        out.fill_(float("nan"))
        B.bpt_layer_fwd_noalloc(sh2, xd2, *wd2, 16, 16, False, 0, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
    assert not torch.isnan(other.float()).any()
