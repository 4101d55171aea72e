"""Host-side pieces of bench.py, on the CPU: the attention-code hash that
decides whether the committed counter record still describes the kernel."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_tokens_ignore_comments_and_layout():
    b = _bench()
    a = "int x = 1; // one\n/* block\n comment */ int  y=2;\n"
    c = "int x = 1;\n\n   int  y=2; // two\n"
    assert b.code_tokens(a) == b.code_tokens(c) == "int x = 1; int y=2;"
    assert b.code_tokens(a) != b.code_tokens(a.replace("y=2", "y=3"))


def test_committed_traffic_record_matches_the_attention_code():
    b = _bench()
    assert b.measured_traffic("c3_bf16_s32k_h2048") is not None, \
        "profiles/attn_fwd_c3_traffic.txt was taken for other attention code: re-take the counters"
    assert b.measured_traffic("c2_bf16_b2_s8k_h2048") is None


def test_attention_roofline_prices_each_dtype_on_its_own_peak():
    b = _bench()
    from blockwise_attention_ffn_amd import inputs
    r = b.attention_roofline(inputs.WORKLOADS["c3_bf16_s32k_h2048"], 1250.0, 256, 64)
    assert (r["bound"], r["peak"], r["kernel"]) == ("mfma", 2500.0, "attn_fwd_bf16_kernel<128, false, 8, 64>")
    assert abs(r["frac"] - 0.5) < 1e-12
    r = b.attention_roofline(inputs.WORKLOADS["c1_fp32_s256_h64"], 1.0, 64, 32)
    assert (r["bound"], r["peak"], r["kernel"]) == ("alu", 157.3, "attn_f32_kernel<32>")


def test_more_than_one_gpu_is_refused_before_any_device_work():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and r.stdout == ""


def test_keep_without_backward_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--keep"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--backward" in r.stderr and r.stdout == ""
