#!/usr/bin/env python3
"""Benchmark of the MI355X BPT layer forward.

Default: one GPU, the 32K-token workload (batch 1, seq 32768, hidden 2048,
16 heads x 128, FFN 8192, ReLU, causal, bf16 storage / fp32 accumulation,
synthetic N(0,1) activations and N(0, 0.02) weights). A step is one full
layer forward (QKV projection, blockwise attention, output projection,
residual, FFN, residual) on inputs already resident in HBM. W warm-up steps,
then K timed steps between a synchronize on each side, timed with HIP events
on the stream the library launches on. Prints ONE JSON line.

Also reported in that line:
  step_ms       median, minimum and maximum of the timed steps' own
                durations (an event after each step; value and ms_per_step
                are the mean over the timed region);
  roofline      the dominant kernel (blockwise attention) timed alone with
                HIP events over the same number of launches, against the
                bf16 dense MFMA peak;
  cpu_baseline  the fp64 CPU oracle on a bounded row sample of the same
                workload, extrapolated to the full layer (labelled as such),
                with its rate in fp64 GFLOP/s of the layer's algorithmic
                FLOPs, the BLAS library and the host's memory.

Extra modes (each prints its own JSON lines, never the default line):
  --sweep     block-size sweep at the 32K shape
  --memory    peak device memory against sequence length
  --stack     the 4-layer, 131072-token stack
  --dropout p the training-mode forward next to the inference forward
  --backward  a training step (forward + backward); with --dropout p, the
              training-mode forward and its backward; with --keep, the forward
              that keeps its activations for the backward and the backward
              from them (no recomputed forward)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BPT layer fwd tokens/sec and % bf16 MFMA peak at seq 32K, h=2048 (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X published fp32 vector peak
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c3_bf16_s32k_h2048")
    p.add_argument("--B_q", type=int, default=None)
    p.add_argument("--B_kv", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=4096,
                   help="query rows of the oracle's CPU sample")
    p.add_argument("--sweep", action="store_true")
    p.add_argument("--memory", action="store_true")
    p.add_argument("--stack", action="store_true")
    p.add_argument("--backward", action="store_true",
                   help="time the layer backward next to the forward (training step)")
    p.add_argument("--keep", action="store_true",
                   help="with --backward: bpt_layer_fwd_for_bwd + bpt_layer_bwd_from_fwd")
    p.add_argument("--dropout", type=float, default=0.0,
                   help="time the training-mode forward (bpt_layer_fwd_train) with this "
                        "dropout rate instead, next to the inference forward")
    p.add_argument("--out", default=None, help="also append the JSON line(s) to this file")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB first (a known-size "
                        "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def emit(obj, path=None):
    line = json.dumps(obj)
    print(line, flush=True)
    if path:
        with open(path, "a") as fh:
            fh.write(line + "\n")


# ----------------------------------------------------------------------------
class Setup:
    """Inputs resident on the device, shape, workspace."""

    def __init__(self, w, B_q, B_kv, seq=None, ffn_rows=0):
        import torch
        from blockwise_attention_ffn_amd import inputs
        from blockwise_attention_ffn_amd import layer as L
        self.w = w
        self.B_q, self.B_kv = B_q, B_kv
        t0 = time.time()
        x, layers = inputs.make_inputs(w, seq=seq)
        self.x_host, self.layers_host = x, layers
        self.x = L.upload(x, w.dtype)
        self.wts = [L.upload_weights(lw, w.dtype) for lw in layers]
        self.shape = L.shape_for(self.x, w.heads, w.ffn, w.dtype)
        from blockwise_attention_ffn_amd import binding as B
        self.ffn_rows = ffn_rows
        nbytes = B.bpt_layer_workspace_bytes_ex(self.shape, B_q, B_kv, w.causal, ffn_rows)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.out = torch.empty_like(self.x)
        # a second activation buffer only for stacks of layers (ping-pong)
        self.out2 = torch.empty_like(self.x) if len(self.wts) > 1 else None
        torch.cuda.synchronize()
        log(f"inputs ready in {time.time() - t0:.1f}s: {self.shape}")

    def step(self, stream):
        from blockwise_attention_ffn_amd import binding as B
        cur = self.x
        bufs = (self.out, self.out2)
        for i, wd in enumerate(self.wts):
            dst = bufs[i % 2]
            B.bpt_layer_fwd_ex(self.shape, cur, *wd.as_tuple(), self.B_q, self.B_kv, self.w.causal,
                               self.ffn_rows, dst, self.ws, stream)
            cur = dst


def time_steps(fn, steps, warmup, stream, per_step=None):
    """Mean ms per step over ``steps`` timed steps after ``warmup`` untimed
    ones. With a list as ``per_step``, an event after every step also
    records each step's own duration there (events on the same stream,
    inside the one timed region)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True)
          for _ in range(steps + 1 if per_step is not None else 2)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        if per_step is not None:
            ev[i + 1].record(stream)
    ev[-1].record(stream)
    torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / steps  # ms


ATTN_SOURCES = ("attn_bf16.h", "attn_bf16_d128.hip", "lds_dma.h")


def code_tokens(text):
    """C++ source with comments removed and whitespace runs collapsed, so
    that edits to comments or layout leave the hash of the code unchanged
    (string literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def attention_source_hash():
    """sha256 (16 hex digits) of the code (comments and layout aside) of the
    sources the head-dim-128 attention kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "blockwise_attention_ffn_amd", "csrc", name)) as fh:
            h.update(code_tokens(fh.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    record, or None when there is none for this workload or the kernel source
    has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_c3_traffic.txt")
    if workload_name != "c3_bf16_s32k_h2048" or not os.path.exists(path):
        return None
    text = open(path).read()
    rec = json.loads(text[text.index("{"):])
    if attention_source_hash() != rec.get("attn_source_sha256_16"):
        return None
    return rec["traffic_bytes_per_launch"]


def attention_kernel_name(head_dim, rows, keys, dtype="bf16"):
    """The kernel instance a (rows, keys) tile runs (bf16 template arguments:
    head dim, log-sum-exp output, waves per workgroup, keys per stage; the
    fp32 path has one kernel per head dim, on the vector ALUs)."""
    if dtype != "bf16":
        return f"attn_f32_kernel<{head_dim}>"
    return f"attn_fwd_bf16_kernel<{head_dim}, false, {max(1, rows // 32)}, {keys}>"


def attention_roofline(w, a_tflops, t_rows, t_keys):
    """bound, kernel, peak and fraction of the attention kernel: bf16 on the
    MFMA peak, fp32 (FMA on the vector ALUs, no fp32 MFMA) on the fp32 vector
    peak."""
    if w.dtype == "bf16":
        bound, peak = "mfma", PEAK_BF16_TFLOPS
    else:
        bound, peak = "alu", PEAK_FP32_VECTOR_TFLOPS
    return {"bound": bound, "kernel": attention_kernel_name(w.head_dim, t_rows, t_keys, w.dtype),
            "achieved": a_tflops, "peak": peak, "unit": "TFLOP/s", "frac": a_tflops / peak}


def attention_flops(w, seq=None):
    b, s, h = w.batch, (seq or w.seq), w.hidden
    return 2.0 * b * h * s * (s + 1) if w.causal else 4.0 * b * s * s * h


# ----------------------------------------------------------------------------
def cpu_baseline(w, rows_n):
    """The fp64 oracle, unmodified, on a bounded sample: K and V are
    projected for every token and ``rows_n`` query rows are evaluated
    against their full key ranges. The full layer's time is extrapolated as
    T_projection + T_rows * (s / rows_n)."""
    import oracle
    from blockwise_attention_ffn_amd import inputs
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in infos] or [1])
        if infos:
            blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in infos}))
    except Exception:  # pragma: no cover
        threads = None
    ram = None
    try:
        with open("/proc/meminfo") as fh:
            for ln in fh:
                if ln.startswith("MemTotal:"):
                    ram = int(ln.split()[1]) * 1024
    except OSError:  # pragma: no cover
        pass
    x, (lw,) = inputs.make_inputs(w)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(w.seq, size=rows_n, replace=False))
    tm = {}
    t0 = time.perf_counter()
    oracle.layer_forward(x, *lw.as_tuple(), heads=w.heads, causal=w.causal, rows=rows, timings=tm)
    wall = time.perf_counter() - t0
    t_full = tm["projection"] + tm["rows"] * (w.seq / rows_n)
    toks = w.batch * w.seq / t_full
    flops = (6 + 2) * w.batch * w.seq * w.hidden ** 2 + 4 * w.batch * w.seq * w.hidden * w.ffn \
        + attention_flops(w)
    return {
        "value": toks,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle; K/V projected for all {w.seq} tokens "
                   f"({tm['projection']:.2f}s) plus {rows_n} random query rows with full key "
                   f"ranges ({tm['rows']:.2f}s); full layer extrapolated as projection + rows "
                   f"x s/{rows_n} = {t_full:.1f}s; sample wall {wall:.1f}s; host affinity "
                   f"{len(os.sched_getaffinity(0))} cpus"),
        "extrapolated": True,
        "gflops_fp64": flops / t_full / 1e9,
        "blas": blas,
        "host_ram_bytes": ram,
    }


# ----------------------------------------------------------------------------
def main_bench(args):
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    B_q = args.B_q or w.B_q
    B_kv = args.B_kv or w.B_kv
    S = Setup(w, B_q, B_kv)
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    step_ms = []
    ms = time_steps(lambda: S.step(stream), args.steps, args.warmup, stream, per_step=step_ms)
    flops = B.bpt_layer_algorithmic_flops(S.shape, w.causal) * w.layers
    tokens = w.batch * w.seq
    tflops = flops / (ms * 1e-3) / 1e12

    # dominant kernel alone: blockwise attention on the Q/K/V already in the workspace
    A = torch.empty_like(S.x)
    wd = S.wts[0]
    B.bpt_debug_attention(S.shape, S.x, wd.Wqkv, wd.bqkv, B_q, B_kv, w.causal, True, A, S.ws, stream)

    def attn():
        B.bpt_debug_attention(S.shape, S.x, wd.Wqkv, wd.bqkv, B_q, B_kv, w.causal, False, A, S.ws,
                              stream)
    attn_ms = time_steps(attn, args.steps, args.warmup, stream)
    a_flops = attention_flops(w)
    a_tflops = a_flops / (attn_ms * 1e-3) / 1e12
    rows = B.bpt_layer_epilogue_rows(S.shape, B_q)
    t_rows, t_keys = B.bpt_layer_attention_tile(S.shape, B_q, B_kv)
    line = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "heads": w.heads, "head_dim": w.head_dim, "ffn": w.ffn, "causal": w.causal,
                   "layers": w.layers, "B_q": B_q, "B_kv": B_kv, "epilogue_rows": rows,
                   "attention_tile": {"query_rows_per_workgroup": t_rows,
                                      "keys_per_stage": t_keys}},
        "tflops": tflops,
        "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "algorithmic_flops_per_step": flops,
        "step_ms": {"median": float(np.median(step_ms)), "min": min(step_ms),
                    "max": max(step_ms)},
        "roofline": {**attention_roofline(w, a_tflops, t_rows, t_keys),
                     "traffic": measured_traffic(w.name),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "attention_source_sha256_16": attention_source_hash(),
                     "ms_per_launch": attn_ms, "flops_per_launch": a_flops},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    emit(line, args.out)


def main_train(args):
    """Training-mode forward (dropout on both residual branches) at the
    workload, timed next to the inference forward on the same inputs."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    B_q = args.B_q or w.B_q
    B_kv = args.B_kv or w.B_kv
    S = Setup(w, B_q, B_kv)
    stream = torch.cuda.current_stream()
    wd = S.wts[0]

    def train():
        B.bpt_layer_fwd_train(S.shape, S.x, *wd.as_tuple(), B_q, B_kv, w.causal, 0, args.dropout,
                              12345, S.out, S.ws, stream)
    ms_inf = time_steps(lambda: S.step(stream), args.steps, args.warmup, stream)
    ms = time_steps(train, args.steps, args.warmup, stream)
    flops = B.bpt_layer_algorithmic_flops(S.shape, w.causal)
    tokens = w.batch * w.seq
    tflops = flops / (ms * 1e-3) / 1e12
    emit({
        "metric": f"BPT layer training-mode fwd (dropout {args.dropout:g} on both residual "
                  f"branches) tokens/sec and % bf16 MFMA peak",
        "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "heads": w.heads, "ffn": w.ffn, "causal": w.causal, "B_q": B_q,
                   "B_kv": B_kv, "dropout": args.dropout},
        "tflops": tflops, "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "inference_ms_per_step": ms_inf,
    }, args.out)


def main_backward(args):
    """Training step at the workload: the inference forward and the layer
    backward (bpt_layer_bwd, which recomputes the forward block by block),
    each timed on its own over the same inputs. With --dropout p: the
    training-mode forward and its backward (bpt_layer_bwd_train)."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    B_q = args.B_q or w.B_q
    B_kv = args.B_kv or w.B_kv
    if w.dtype != "bf16":
        raise SystemExit("the backward is bf16 only")
    S = Setup(w, B_q, B_kv)
    stream = torch.cuda.current_stream()
    wd = S.wts[0]
    h, f = w.hidden, w.ffn
    g = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn(S.x.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dx = torch.empty_like(S.x)
    grads = [torch.empty(sh, dtype=torch.float32, device="cuda") for sh in
             [(3 * h, h), (3 * h,), (h, h), (h,), (f, h), (f,), (h, f), (h,)]]
    wsb = torch.empty(B.bpt_layer_bwd_workspace_bytes(S.shape, B_q, B_kv, w.causal),
                      dtype=torch.uint8, device="cuda")

    p = args.dropout
    if args.keep:
        return backward_kept(args, w, S, B_q, B_kv, wd, dout, dx, grads, wsb, stream)

    def bwd():
        if p > 0:
            B.bpt_layer_bwd_train(S.shape, S.x, *wd.as_tuple(), B_q, B_kv, w.causal, 0, p, 17, dout,
                                  dx, *grads, wsb, stream)
        else:
            B.bpt_layer_bwd(S.shape, S.x, *wd.as_tuple(), B_q, B_kv, w.causal, 0, dout, dx, *grads,
                            wsb, stream)

    def fwd_step():
        if p > 0:
            B.bpt_layer_fwd_train(S.shape, S.x, *wd.as_tuple(), B_q, B_kv, w.causal, 0, p, 17, S.out,
                                  S.ws, stream)
        else:
            S.step(stream)
    ms_fwd = time_steps(fwd_step, args.steps, args.warmup, stream)
    ms_bwd = time_steps(bwd, args.steps, args.warmup, stream)
    fwd = B.bpt_layer_algorithmic_flops(S.shape, w.causal)
    attn = attention_flops(w)
    dense = fwd - attn
    T = w.batch * w.seq
    # model FLOPs of the backward: each forward product has two (dX and dW for
    # the dense ones; dV, dP, dK, dQ for the two attention ones)
    bwd_model = 2.0 * fwd
    # executed by bpt_layer_bwd: the recomputed forward up to H (every dense
    # product but W2, and the attention), the gradient products (twice the
    # dense forward), and the attention backward's 8 products of attn / 2 each
    # (dV: scores, dV; dK: scores, dP, dK; dQ: scores, dP, dQ)
    bwd_exec = (dense - 2.0 * T * h * f) + attn + 2.0 * dense + 4.0 * attn
    step_ms = ms_fwd + ms_bwd
    tflops = (fwd + bwd_model) / (step_ms * 1e-3) / 1e12
    emit({
        "metric": "BPT layer training step (fwd + bwd with blockwise recomputation"
                  + (f", dropout {p:g} on both residual branches" if p > 0 else "")
                  + ") tokens/sec and % bf16 MFMA peak (model FLOPs)",
        "value": T / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq": w.seq, "hidden": h,
                   "heads": w.heads, "ffn": f, "causal": w.causal, "B_q": B_q, "B_kv": B_kv,
                   "dropout": p},
        "tflops": tflops, "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "fwd_ms": ms_fwd, "bwd_ms": ms_bwd,
        "bwd_model_tflops": bwd_model / (ms_bwd * 1e-3) / 1e12,
        "bwd_executed_tflops": bwd_exec / (ms_bwd * 1e-3) / 1e12,
        "bwd_workspace_bytes": wsb.numel(),
    }, args.out)


def backward_kept(args, w, S, B_q, B_kv, wd, dout, dx, grads, wsb, stream):
    """--backward --keep: the training step as bpt_layer_fwd_for_bwd (the
    forward, leaving Q, K, V^T, A, the log-sum-exp and y in the backward's
    workspace) followed by bpt_layer_bwd_from_fwd (the backward from them, no
    recomputed forward). The backward consumes what the forward kept, so
    steps are timed as pairs; the forward is also timed alone."""
    from blockwise_attention_ffn_amd import binding as B
    p, h = args.dropout, w.hidden

    def fwd():
        B.bpt_layer_fwd_for_bwd(S.shape, S.x, *wd.as_tuple(), B_q, B_kv, w.causal, 0, p, 17, S.out,
                                wsb, stream)

    def pair():
        fwd()
        B.bpt_layer_bwd_from_fwd(S.shape, S.x, *wd.as_tuple(), B_q, B_kv, w.causal, 0, p, 17, dout,
                                 dx, *grads, wsb, stream)
    ms_fwd = time_steps(fwd, args.steps, args.warmup, stream)
    step_ms = time_steps(pair, args.steps, args.warmup, stream)
    ms_bwd = step_ms - ms_fwd
    fwd_fl = B.bpt_layer_algorithmic_flops(S.shape, w.causal)
    attn = attention_flops(w)
    dense = fwd_fl - attn
    T = w.batch * w.seq
    bwd_model = 2.0 * fwd_fl
    # executed by the backward from kept activations: H per group (W1), the
    # gradient products, and the attention backward's 8 products of attn / 2
    bwd_exec = 2.0 * T * h * w.ffn + 2.0 * dense + 4.0 * attn
    tflops = (fwd_fl + bwd_model) / (step_ms * 1e-3) / 1e12
    emit({
        "metric": "BPT layer training step (fwd keeping its activations + bwd from them"
                  + (f", dropout {p:g} on both residual branches" if p > 0 else "")
                  + ") tokens/sec and % bf16 MFMA peak (model FLOPs)",
        "value": T / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq": w.seq, "hidden": h,
                   "heads": w.heads, "ffn": w.ffn, "causal": w.causal, "B_q": B_q, "B_kv": B_kv,
                   "dropout": p, "kept_activations": True},
        "tflops": tflops, "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "fwd_ms": ms_fwd, "bwd_ms": ms_bwd,
        "bwd_model_tflops": bwd_model / (ms_bwd * 1e-3) / 1e12,
        "bwd_executed_tflops": bwd_exec / (ms_bwd * 1e-3) / 1e12,
        "bwd_workspace_bytes": wsb.numel(),
    }, args.out)


def main_sweep(args):
    """Block sizes at the 32K shape: the 9-point grid of the workload, then
    B_q = B_kv over the pages' grid {16, 64, 128, 256, 512, 1024, 2048, 4096}.
    Per point: the layer (args.steps timed steps) and the attention kernel
    alone (on the Q/K/V of that point's projection), the attention tile the
    block sizes select, and the FFN group."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import inputs
    from blockwise_attention_ffn_amd import layer as L
    w = inputs.WORKLOADS["c3_bf16_s32k_h2048"]
    pts = [(q, k) for q in w.sweep_q for k in w.sweep_kv]
    pts += [(b, b) for b in (16, 64, 128, 256, 512, 1024, 2048, 4096) if (b, b) not in pts]
    if args.B_q and args.B_kv:
        pts = [(args.B_q, args.B_kv)]
    S = Setup(w, w.B_q, w.B_kv)
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flops = B.bpt_layer_algorithmic_flops(S.shape, True)
    a_flops = attention_flops(w)
    A = torch.empty_like(S.x)
    wd = S.wts[0]
    for q, k in pts:
        S.B_q, S.B_kv = q, k
        S.ws = L.alloc_workspace(S.shape, q, k, True)
        ms = time_steps(lambda: S.step(stream), args.steps, args.warmup, stream)
        B.bpt_debug_attention(S.shape, S.x, wd.Wqkv, wd.bqkv, q, k, True, True, A, S.ws, stream)
        attn_ms = time_steps(lambda: B.bpt_debug_attention(S.shape, S.x, wd.Wqkv, wd.bqkv, q, k,
                                                           True, False, A, S.ws, stream),
                             args.steps, args.warmup, stream)
        tr, tk = B.bpt_layer_attention_tile(S.shape, q, k)
        tf = flops / (ms * 1e-3) / 1e12
        emit({"sweep": "block", "workload": w.name, "B_q": q, "B_kv": k,
              "attention_tile": {"query_rows_per_workgroup": tr, "keys_per_stage": tk},
              "attention_kernel": attention_kernel_name(w.head_dim, tr, tk, w.dtype),
              "epilogue_rows": B.bpt_layer_epilogue_rows(S.shape, q), "ms": ms,
              "tokens_per_s": w.seq / (ms * 1e-3), "tflops": tf,
              "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS, "attention_ms": attn_ms,
              "attention_tflops": a_flops / (attn_ms * 1e-3) / 1e12}, args.out)
        del S.ws
        torch.cuda.empty_cache()


def main_memory(args):
    """Peak device memory of one layer call against the sequence length, for
    the blockwise FFN (groups of query blocks, the default) and for the FFN
    over the whole sequence at once (the comparator the BPT review's memory
    analysis measures against). Buffers: x, out, weights, workspace."""
    import torch
    from blockwise_attention_ffn_amd import binding as B
    from blockwise_attention_ffn_amd import inputs
    w = inputs.WORKLOADS["c5_bf16_s128k_h2048_x4"].replace(layers=1)
    for mode in ("blockwise_ffn", "whole_sequence_ffn"):
        for s in (8192, 16384, 32768, 65536, 131072):
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            base = torch.cuda.memory_allocated()
            free0, _ = torch.cuda.mem_get_info()
            ffn_rows = 0 if mode == "blockwise_ffn" else s
            try:
                S = Setup(w, 2048, 1024, seq=s, ffn_rows=ffn_rows)
                stream = torch.cuda.current_stream()
                ms = time_steps(lambda: S.step(stream), 3, 1, stream)
            except torch.OutOfMemoryError:
                emit({"sweep": "memory", "mode": mode, "seq": s, "oom": True}, args.out)
                continue
            peak = torch.cuda.max_memory_allocated() - base
            free1, _ = torch.cuda.mem_get_info()
            ws = B.bpt_layer_workspace_bytes_ex(S.shape, 2048, 1024, True, ffn_rows)
            rows = ffn_rows or B.bpt_layer_epilogue_rows(S.shape, 2048)
            emit({"sweep": "memory", "mode": mode, "seq": s, "peak_bytes": peak,
                  "workspace_bytes": ws, "hipMemGetInfo_delta": free0 - free1, "ms": ms,
                  "ffn_group_rows": rows}, args.out)
            del S
    torch.cuda.empty_cache()


def main():
    args = parse()
    if args.keep and not args.backward:
        print("--keep times the training step with kept activations: use it with --backward",
              file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the layer runs "
              "on a single device, and how it would shard across GPUs is described, not "
              "implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    from blockwise_attention_ffn_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from blockwise_attention_ffn_amd import build
        build.build()
    binding.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.backward:
        return main_backward(args)
    if args.dropout > 0:
        main_train(args)
    elif args.sweep:
        main_sweep(args)
    elif args.memory:
        main_memory(args)
    elif args.stack:
        args.workload = "c5_bf16_s128k_h2048_x4"
        args.no_cpu_baseline = True
        main_bench(args)
    else:
        main_bench(args)


if __name__ == "__main__":
    main()
