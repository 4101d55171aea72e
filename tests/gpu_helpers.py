"""Shared helpers of the GPU parity tests (inputs, runs, error metrics)."""
from __future__ import annotations

import sys

import numpy as np

from blockwise_attention_ffn_amd import inputs
from blockwise_attention_ffn_amd import layer as L

# Parity bars: max |gpu - oracle| / max |oracle| (the infinity-norm relative
# error) on each checked tensor. fp32: 1e-4; bf16 storage with fp32
# accumulation: 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_inf(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / max(den, 1e-30)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def device_inputs(x, lw, dtype):
    xd = L.upload(x, dtype)
    wd = L.upload_weights(lw, dtype)
    return xd, wd


def run_gpu(x, lw, heads, ffn, dtype, causal, B_q, B_kv, debug=True):
    """Run one layer on the GPU through the C ABI. Returns host float64
    arrays (out, A, y); A and y are None unless ``debug``."""
    import torch
    xd, wd = device_inputs(x, lw, dtype)
    sh = L.shape_for(xd, heads, ffn, dtype)
    if debug:
        out, A, y = L.layer_forward_debug(sh, xd, wd, B_q, B_kv, causal)
        torch.cuda.synchronize()
        return L.to_f64(out), L.to_f64(A), L.to_f64(y)
    out = L.layer_forward(sh, xd, wd, B_q, B_kv, causal)
    torch.cuda.synchronize()
    return L.to_f64(out), None, None


def check_against_oracle(tag, gpu, ref, dtype, rows=None):
    """gpu = (out, A, y) full-size host arrays; ref = oracle dict (possibly on
    a row sample). Asserts the parity bar on out and A, reports the rest."""
    out, A, y = gpu
    sel = (lambda t: t) if rows is None else (lambda t: t[:, rows, :])
    tol = TOL[dtype]
    e_out = rel_inf(sel(out), ref["out"])
    msg = [f"{tag}: out {e_out:.2e} (l2 {rel_l2(sel(out), ref['out']):.2e})"]
    errs = {"out": e_out}
    if A is not None:
        errs["A"] = rel_inf(sel(A), ref["A"])
        errs["y"] = rel_inf(sel(y), ref["y"])
        # the FFN's contribution alone (out - y), reported only: it is the
        # difference of two rounded outputs, so its relative error is large
        # whenever the FFN term is small next to the residual stream
        errs["ffn_part"] = rel_inf(sel(out) - sel(y), ref["out"] - ref["y"])
        msg.append(f"A {errs['A']:.2e} y {errs['y']:.2e} out-y {errs['ffn_part']:.2e}")
    say(" ".join(msg))
    assert e_out <= tol, f"{tag}: out error {e_out:.3e} > {tol}"
    if A is not None:
        assert errs["A"] <= tol, f"{tag}: A error {errs['A']:.3e} > {tol}"
        assert errs["y"] <= tol, f"{tag}: y error {errs['y']:.3e} > {tol}"
    return errs


def make(wname, **over):
    w = inputs.WORKLOADS[wname]
    seq = over.pop("seq", None)
    batch = over.pop("batch", None)
    if over:
        w = w.replace(**over)
    x, layers = inputs.make_inputs(w, seq=seq, batch=batch)
    return w, x, layers
