"""The C-ABI library on the host: it loads, exports every declared symbol,
plans workspaces, counts FLOPs, and rejects bad arguments before touching a
device. No kernel is launched here (fake, never-dereferenced addresses)."""
import os
import re

import pytest

from blockwise_attention_ffn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bpt.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from blockwise_attention_ffn_amd import build
        build.build(verbose=False)
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bpt_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert "bpt_layer_fwd" in names and len(names) >= 8
    for n in names:
        assert hasattr(L, n), f"{n} declared in bpt.h but not exported"
    assert set(names) == set(B.EXPORTED)


def test_status_strings(L):
    for code in range(0, 12):
        s = B.bpt_status_string(code)
        assert s and s != "unknown status"
    assert B.bpt_status_string(99) == "unknown status"
    assert B.bpt_version().startswith("bpt-gfx950")


# algorithmic FLOPs per layer: 6bsh^2 + 2bsh^2 + 4bshf + attention
@pytest.mark.parametrize("dims,causal,want", [
    ((1, 256, 64, 2, 256, "f32"), False, 41.94e6),
    ((2, 8192, 2048, 16, 8192, "bf16"), True, 2.199e12),
    ((1, 32768, 2048, 16, 8192, "bf16"), True, 7.697e12),
    ((1, 16384, 4096, 32, 16384, "bf16"), True, 8.796e12),
    ((1, 131072, 2048, 16, 8192, "bf16"), True, 83.56e12),
])
def test_algorithmic_flops(L, dims, causal, want):
    f = B.bpt_layer_algorithmic_flops(B.make_shape(*dims), causal)
    assert abs(f - want) / want < 1e-3


def test_flops_exact_small(L):
    b, s, h, f = 1, 16, 64, 64
    sh = B.make_shape(b, s, h, 2, f, "bf16")
    dense = 8 * b * s * h * h + 4 * b * s * h * f
    # causal: 4*d per kept (query, key) pair per head: pairs = s(s+1)/2
    assert B.bpt_layer_algorithmic_flops(sh, True) == dense + 4 * h * s * (s + 1) // 2
    assert B.bpt_layer_algorithmic_flops(sh, False) == dense + 4 * h * s * s
    assert B.bpt_layer_algorithmic_flops(B.make_shape(1, 16, 64, 3, 64, "bf16"), True) < 0


def _align(v):
    return (v + 255) // 256 * 256


def test_workspace_plan_bf16(L):
    b, s, h, nh, f = 1, 32768, 2048, 16, 8192
    sh = B.make_shape(b, s, h, nh, f, "bf16")
    for B_q in (512, 1024, 2048):
        rows = B.bpt_layer_epilogue_rows(sh, B_q)
        assert rows == 8192 and rows % B_q == 0
        want = 4 * _align(b * s * h * 2) + _align(rows * f * 2)
        assert B.bpt_layer_workspace_bytes(sh, B_q, 512, True) == want
    # the FFN scratch does not grow with s: linear slope of 4*h*e bytes per token
    w1 = B.bpt_layer_workspace_bytes(B.make_shape(1, 65536, h, nh, f, "bf16"), 2048, 1024, True)
    w2 = B.bpt_layer_workspace_bytes(B.make_shape(1, 131072, h, nh, f, "bf16"), 2048, 1024, True)
    assert w2 - w1 == 4 * 65536 * h * 2


def test_workspace_plan_f32_small(L):
    sh = B.make_shape(1, 256, 64, 2, 256, "f32")
    assert B.bpt_layer_epilogue_rows(sh, 64) == 256
    assert B.bpt_layer_workspace_bytes(sh, 64, 64, False) == 4 * _align(256 * 64 * 4) + _align(256 * 256 * 4)


# ---------------------------------------------------------------------------
BASE = 0x7f0000000000


def _layout(sh, esize):
    """Disjoint fake device addresses for every argument."""
    b, s, h, f = sh.batch, sh.seq, sh.hidden, sh.ffn
    sizes = [b * s * h, 3 * h * h, 3 * h, h * h, h, h * f, f, f * h, h]
    addrs, a = [], BASE
    for n in sizes:
        addrs.append(a)
        a += _align(n * esize) + 4096
    out = a
    ws = out + _align(b * s * h * esize) + 4096
    return addrs, out, ws


def _call(sh, ptrs, out, ws, ws_bytes, B_q=64, B_kv=64):
    return B.bpt_layer_fwd_raw(sh, ptrs, B_q, B_kv, 0, out, ws, ws_bytes, None)


def test_argument_errors_are_reported_before_any_launch(L):
    sh = B.make_shape(1, 256, 64, 2, 256, "f32")
    ptrs, out, ws = _layout(sh, 4)
    need = B.bpt_layer_workspace_bytes(sh, 64, 64, False)
    E = {v: k for k, v in B.STATUS_NAMES.items()}

    assert L.bpt_layer_fwd(None, *ptrs, 64, 64, 0, out, ws, need, None) == E["BPT_ERR_NULL"]
    assert _call(B.make_shape(1, 256, 64, 2, 256, 7), ptrs, out, ws, need) == E["BPT_ERR_DTYPE"]
    for bad in [(1, 256, 64, 3, 256), (1, 256, 64, 4, 256), (1, 256, 96, 3, 256),
                (1, 256, 64, 2, 100), (0, 256, 64, 2, 256), (1, 250, 64, 2, 256),
                (1, 256, 1024, 4, 256)]:
        assert _call(B.make_shape(*bad, "f32"), ptrs, out, ws, need) == E["BPT_ERR_SHAPE"], bad
    for bq, bkv in [(8, 64), (64, 8), (48, 64), (64, 48), (512, 64), (64, 0), (24, 64)]:
        assert _call(sh, ptrs, out, ws, need, bq, bkv) == E["BPT_ERR_BLOCK"], (bq, bkv)
    for i in range(9):
        p = list(ptrs)
        p[i] = None
        assert _call(sh, p, out, ws, need) == E["BPT_ERR_NULL"], i
    assert _call(sh, ptrs, None, ws, need) == E["BPT_ERR_NULL"]
    assert _call(sh, ptrs, out, None, need) == E["BPT_ERR_NULL"]
    for i in range(9):
        p = list(ptrs)
        p[i] += 8
        assert _call(sh, p, out, ws, need) == E["BPT_ERR_ALIGN"], i
    assert _call(sh, ptrs, out + 4, ws, need) == E["BPT_ERR_ALIGN"]
    assert _call(sh, ptrs, out, ws, need - 1) == E["BPT_ERR_WORKSPACE"]
    # out overlapping a weight, partially overlapping x, or the workspace
    assert _call(sh, ptrs, ptrs[3], ws, need) == E["BPT_ERR_ALIAS"]
    assert _call(sh, ptrs, ptrs[0] + 256, ws, need) == E["BPT_ERR_ALIAS"]
    assert _call(sh, ptrs, ws + 4096, ws, need) == E["BPT_ERR_ALIAS"]
    # the workspace overlapping an input
    assert _call(sh, ptrs, out, ptrs[5], need) == E["BPT_ERR_ALIAS"]


def test_block_sizes_accepted_by_plan(L):
    sh = B.make_shape(1, 32768, 2048, 16, 8192, "bf16")
    for Bsz in (16, 64, 128, 256, 512, 1024, 2048, 4096, 32768):
        assert B.bpt_layer_workspace_bytes(sh, Bsz, Bsz, True) > 0
    with pytest.raises(B.BptError):
        B.bpt_layer_workspace_bytes(sh, 3000, 512, True)


def test_ffn_group_rows_ex(L):
    sh = B.make_shape(1, 32768, 2048, 16, 8192, "bf16")
    base = B.bpt_layer_workspace_bytes(sh, 1024, 512, True)
    assert B.bpt_layer_workspace_bytes_ex(sh, 1024, 512, True, 0) == base
    whole = B.bpt_layer_workspace_bytes_ex(sh, 1024, 512, True, 32768)
    # the whole-sequence FFN holds s x f of hidden activations instead of 8192 x f
    assert whole - base == (32768 - 8192) * 8192 * 2
    for bad in (1000, 2 * 32768, -1024, 512):
        with pytest.raises(B.BptError) as e:
            B.bpt_layer_workspace_bytes_ex(sh, 1024, 512, True, bad)
        assert e.value.name == "BPT_ERR_BLOCK"


def test_training_mode_argument_errors(L):
    """Dropout arguments are checked before anything else is touched."""
    E = {v: k for k, v in B.STATUS_NAMES.items()}
    sh = B.make_shape(1, 256, 64, 2, 256, "f32")
    base = 0x7f0000000000
    ptrs = [base + i * (1 << 24) for i in range(9)]
    out, ws = base + 9 * (1 << 24), base + 10 * (1 << 24)
    need = B.bpt_layer_workspace_bytes(sh, 64, 64, False)
    for p in (1.0, -0.1, float("nan"), float("inf"), 2.0):
        st = L.bpt_layer_fwd_train(B.ctypes.byref(sh), *ptrs, 64, 64, 0, 0, p, 7, out, ws, need,
                                   None)
        assert st == E["BPT_ERR_DROPOUT"], p
    # the mask hook: rate, channel multiple of 16, ranges, pointer
    keep = base + 11 * (1 << 24)
    assert L.bpt_debug_dropout_keep(4, 32, 0, 1.0, 1, 0, keep, None) == E["BPT_ERR_DROPOUT"]
    assert L.bpt_debug_dropout_keep(4, 24, 0, 0.1, 1, 0, keep, None) == E["BPT_ERR_DROPOUT"]
    assert L.bpt_debug_dropout_keep(-1, 32, 0, 0.1, 1, 0, keep, None) == E["BPT_ERR_SHAPE"]
    assert L.bpt_debug_dropout_keep(4, 32, -5, 0.1, 1, 0, keep, None) == E["BPT_ERR_SHAPE"]
    assert L.bpt_debug_dropout_keep(4, 32, 0, 0.1, 1, 2, keep, None) == E["BPT_ERR_SHAPE"]
    assert L.bpt_debug_dropout_keep(4, 32, 0, 0.1, 1, 0, None, None) == E["BPT_ERR_NULL"]
    assert L.bpt_debug_dropout_keep(4, 32, 0, 0.1, 1, 0, keep + 8, None) == E["BPT_ERR_ALIGN"]
    assert L.bpt_debug_dropout_keep(0, 32, 0, 0.1, 1, 0, None, None) == E["BPT_OK"]
    assert L.bpt_status_string(E["BPT_ERR_DROPOUT"]).startswith(b"dropout rate")
    # the training-mode backward checks its rate first too
    shb = B.make_shape(1, 256, 128, 2, 256, "bf16")
    needb = B.bpt_layer_bwd_workspace_bytes(shb, 64, 64, True)
    grads = [base + (12 + i) * (1 << 24) for i in range(10)]  # dout, dx, 8 gradients
    for p in (1.0, -0.1, float("nan"), 1.5):
        st = L.bpt_layer_bwd_train(B.ctypes.byref(shb), *ptrs, 64, 64, 1, 0, p, 7, *grads, ws,
                                   needb, None)
        assert st == E["BPT_ERR_DROPOUT"], p
    # and rejects fp32 shapes as the inference backward does
    st = L.bpt_layer_bwd_train(B.ctypes.byref(sh), *ptrs, 64, 64, 1, 0, 0.1, 7, *grads, ws,
                               needb, None)
    assert st == E["BPT_ERR_DTYPE"]


def test_backward_plan_and_argument_errors(L):
    """The backward's plan (bf16 only) and its argument checks, which all come
    before the device is queried."""
    E = {v: k for k, v in B.STATUS_NAMES.items()}
    sh = B.make_shape(1, 256, 128, 2, 256, "bf16")
    need = B.bpt_layer_bwd_workspace_bytes(sh, 64, 64, True)
    assert need > B.bpt_layer_workspace_bytes(sh, 64, 64, True)
    # FFN groups of 64 rows hold 64 x f of hidden activations instead of 256 x f
    assert B.bpt_layer_bwd_workspace_bytes(sh, 64, 64, True, 64) < need
    with pytest.raises(B.BptError) as e:
        B.bpt_layer_bwd_workspace_bytes(B.make_shape(1, 256, 128, 2, 256, "f32"), 64, 64, True)
    assert e.value.name == "BPT_ERR_DTYPE"
    with pytest.raises(B.BptError) as e:
        B.bpt_layer_bwd_workspace_bytes(sh, 48, 64, True)
    assert e.value.name == "BPT_ERR_BLOCK"
    base = 0x7f0000000000
    step = 1 << 24
    ins = [base + i * step for i in range(10)]        # x, 8 weights, dout
    outs = [base + (10 + i) * step for i in range(9)]  # dx and 8 gradients
    ws = base + 19 * step

    def call(ins_, outs_, ws_, nbytes=need, B_q=64):
        return L.bpt_layer_bwd(B.ctypes.byref(sh), *ins_[:9], B_q, 64, 1, 0, ins_[9], *outs_, ws_,
                               nbytes, None)
    assert call(ins, outs, ws, B_q=40) == E["BPT_ERR_BLOCK"]
    for i in range(10):
        bad = list(ins)
        bad[i] = None
        assert call(bad, outs, ws) == E["BPT_ERR_NULL"], i
    for i in range(9):
        bad = list(outs)
        bad[i] = None
        assert call(ins, bad, ws) == E["BPT_ERR_NULL"], i
    assert call(ins, outs, None) == E["BPT_ERR_NULL"]
    bad = list(outs)
    bad[3] += 8
    assert call(ins, bad, ws) == E["BPT_ERR_ALIGN"]
    assert call(ins, outs, ws, need - 256) == E["BPT_ERR_WORKSPACE"]
    bad = list(outs)
    bad[0] = ins[0]  # dx over x
    assert call(ins, bad, ws) == E["BPT_ERR_ALIAS"]
    bad = list(outs)
    bad[2] = bad[1]  # two gradients on one buffer
    assert call(ins, bad, ws) == E["BPT_ERR_ALIAS"]
    assert call(ins, outs, outs[4]) == E["BPT_ERR_ALIAS"]  # workspace over a gradient


def test_kept_activation_pair_argument_errors(L):
    """bpt_layer_fwd_for_bwd and bpt_layer_bwd_from_fwd check rate, dtype,
    blocks, pointers, alignment, workspace size and overlaps before the device
    is queried; out may not be x, which the backward reads again."""
    E = {v: k for k, v in B.STATUS_NAMES.items()}
    sh = B.make_shape(1, 256, 128, 2, 256, "bf16")
    need = B.bpt_layer_bwd_workspace_bytes(sh, 64, 64, True)
    base = 0x7f0000000000
    step = 1 << 24
    ins = [base + i * step for i in range(9)]  # x and 8 weights
    out, ws = base + 9 * step, base + 10 * step

    def fwd(ins_=ins, out_=out, ws_=ws, nbytes=need, p=0.1, shape=sh, B_q=64):
        return L.bpt_layer_fwd_for_bwd(B.ctypes.byref(shape), *ins_, B_q, 64, 1, 0, p, 7, out_,
                                       ws_, nbytes, None)
    for p in (1.0, -0.1, float("nan")):
        assert fwd(p=p) == E["BPT_ERR_DROPOUT"], p
    assert fwd(shape=B.make_shape(1, 256, 128, 2, 256, "f32")) == E["BPT_ERR_DTYPE"]
    assert fwd(B_q=40) == E["BPT_ERR_BLOCK"]
    for i in range(9):
        bad = list(ins)
        bad[i] = None
        assert fwd(ins_=bad) == E["BPT_ERR_NULL"], i
        bad[i] = ins[i] + 8
        assert fwd(ins_=bad) == E["BPT_ERR_ALIGN"], i
    assert fwd(out_=None) == E["BPT_ERR_NULL"]
    assert fwd(ws_=None) == E["BPT_ERR_NULL"]
    assert fwd(out_=out + 4) == E["BPT_ERR_ALIGN"]
    assert fwd(nbytes=need - 256) == E["BPT_ERR_WORKSPACE"]
    assert fwd(out_=ins[0]) == E["BPT_ERR_ALIAS"]       # out over x
    assert fwd(out_=ins[3] + 256) == E["BPT_ERR_ALIAS"]  # out inside Wo
    assert fwd(out_=ws + 4096) == E["BPT_ERR_ALIAS"]    # out inside the workspace
    assert fwd(ws_=ins[5]) == E["BPT_ERR_ALIAS"]        # workspace over W1

    grads = [base + (11 + i) * step for i in range(10)]  # dout, dx, 8 gradients

    def bwd(grads_=grads, p=0.1, shape=sh, nbytes=need):
        return L.bpt_layer_bwd_from_fwd(B.ctypes.byref(shape), *ins, 64, 64, 1, 0, p, 7, *grads_,
                                        ws, nbytes, None)
    assert bwd(p=1.0) == E["BPT_ERR_DROPOUT"]
    assert bwd(shape=B.make_shape(1, 256, 128, 2, 256, "f32")) == E["BPT_ERR_DTYPE"]
    assert bwd(nbytes=need - 256) == E["BPT_ERR_WORKSPACE"]
    bad = list(grads)
    bad[1] = ins[0]  # dx over x
    assert bwd(grads_=bad) == E["BPT_ERR_ALIAS"]
    bad = list(grads)
    bad[4] = None
    assert bwd(grads_=bad) == E["BPT_ERR_NULL"]


def test_backward_workspace_is_linear_in_seq_with_no_seq_times_ffn_term(L):
    """The backward's workspace grows by the same bytes per token at every
    length (no seq² term), and that slope does not depend on f (no seq × f
    array: the FFN's hidden activations, their gradient and their column-sum
    partials exist for one group of rows at a time). From 32768 tokens on,
    where the per-token column-sum partials outgrow one group's at every f
    tested (below, the larger of the two is a constant)."""
    def ws(s, h, nh, f):
        return B.bpt_layer_bwd_workspace_bytes(B.make_shape(1, s, h, nh, f, "bf16"), 1024, 512, True)
    for h, nh in ((2048, 16), (4096, 32)):
        slopes = set()
        for f in (h, 4 * h, 8 * h):
            w = [ws(s, h, nh, f) for s in (32768, 65536, 131072, 262144)]
            d = [(w[i + 1] - w[i]) / (32768 << i) for i in range(3)]
            assert d[0] == d[1] == d[2], (h, f, d)
            slopes.add(d[0])
        assert len(slopes) == 1, (h, slopes)


def test_noalloc_scratch_size_matches_the_header():
    import re
    text = open(HEADER).read()
    m = re.search(r"#define\s+BPT_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m, "BPT_NOALLOC_SCRATCH_BYTES not found in bpt.h"
    assert B.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    assert B.STATUS_NAMES[12] == "BPT_ERR_SCRATCH"
    assert b"scratch" in B.lib().bpt_status_string(12)


def test_attention_tile_follows_the_block_sizes():
    """rows = the largest of 256..16 dividing B_q; keys = the largest of
    64, 32, 16 dividing B_kv (host-side plan, no GPU)."""
    sh = B.make_shape(1, 24576, 2048, 16, 8192, "bf16")  # 3·8192: every block below divides it
    cases = {(16, 16): (16, 16), (32, 32): (32, 32), (64, 64): (64, 64), (128, 128): (128, 64),
             (256, 256): (256, 64), (512, 512): (256, 64), (4096, 4096): (256, 64),
             (48, 48): (16, 16), (384, 96): (128, 32), (1024, 512): (256, 64),
             (2048, 1024): (256, 64), (512, 256): (256, 64)}
    for (bq, bkv), want in cases.items():
        assert B.bpt_layer_attention_tile(sh, bq, bkv) == want, (bq, bkv)
    with pytest.raises(B.BptError):
        B.bpt_layer_attention_tile(sh, 24, 16)
    # the fp32 path runs one fixed tile whatever the block sizes
    sh32 = B.make_shape(1, 256, 64, 2, 256, "f32")
    for bq, bkv in [(16, 16), (64, 64), (256, 128)]:
        assert B.bpt_layer_attention_tile(sh32, bq, bkv) == (64, 32)


def test_one_hip_runtime_per_process():
    """Loading the library through the binding, before anything else imports
    torch, leaves one HIP runtime in the process: torch's (the library binds
    to it by SONAME). A second runtime (the system's, pulled in by loading
    the library first) would not know torch's streams or state."""
    import subprocess
    import sys
    code = ("from blockwise_attention_ffn_amd import binding\n"
            "binding.lib()\n"
            "import torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps), sorted(maps))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr
    n = int(r.stdout.split()[0])
    assert n == 1, r.stdout


def test_header_is_plain_c_and_cpp(tmp_path):
    """include/bpt.h is the boundary for C callers too: it must compile as
    ISO C99 (pedantic, warnings as errors) and as C++17, with every declared
    entry point referenced."""
    import shutil
    import subprocess
    names = re.findall(r"^\w[\w\s\*]*?\b(bpt_\w+)\s*\(", open(HEADER).read(), re.M)
    assert "bpt_layer_fwd" in names and "bpt_layer_bwd_from_fwd" in names
    src = tmp_path / "use.c"
    src.write_text('#include "bpt.h"\nint main(void) {\n  unsigned long n = 0;\n' +
                   "".join(f"  n += sizeof(&{n});\n" for n in sorted(set(names))) +
                   "  return n == 0;\n}\n")
    inc = os.path.dirname(HEADER)
    for cc, std in (("gcc", ["-std=c99", "-pedantic"]), ("g++", ["-std=c++17", "-x", "c++"])):
        if not shutil.which(cc):
            pytest.skip(f"{cc} not installed")
        r = subprocess.run([cc, *std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", inc,
                            str(src)], capture_output=True, text=True)
        assert r.returncode == 0, (cc, r.stderr)
