"""Conveniences over the binding: uploading host arrays and running a layer.

Only plumbing: device allocation through torch (so torch's memory
statistics see every buffer) and calls into the C ABI.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from . import binding as B

_KEYS = ("Wqkv", "bqkv", "Wo", "bo", "W1", "b1", "W2", "b2")


def torch_dtype(dtype: str):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def upload(a: np.ndarray, dtype: str, device="cuda"):
    """float32 host array -> device tensor of the call dtype. For bf16 the
    values must already be bf16-exact (the input generator guarantees it), so
    the conversion is exact."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=torch_dtype(dtype)).contiguous()


@dataclass
class DeviceWeights:
    Wqkv: object
    bqkv: object
    Wo: object
    bo: object
    W1: object
    b1: object
    W2: object
    b2: object

    def as_tuple(self):
        return tuple(getattr(self, k) for k in _KEYS)


def upload_weights(lw, dtype: str, device="cuda") -> DeviceWeights:
    """Host weights in the formulas' [in, out] form (x·W) -> device weights
    in the library's [out, in] layout (x·Wᵀ, nn.Linear's). The transpose is a
    one-time layout change at upload; biases are uploaded as they are."""
    return DeviceWeights(*(upload(np.ascontiguousarray(a.T) if a.ndim == 2 else a, dtype, device)
                           for a in lw.as_tuple()))


def shape_for(x, heads: int, ffn: int, dtype: str) -> B.BptShape:
    b, s, h = x.shape
    return B.make_shape(b, s, h, heads, ffn, dtype)


def alloc_workspace(shape: B.BptShape, B_q: int, B_kv: int, causal: bool, device="cuda"):
    import torch
    n = B.bpt_layer_workspace_bytes(shape, B_q, B_kv, causal)
    return torch.empty(n, dtype=torch.uint8, device=device)


def layer_forward(shape, x, w: DeviceWeights, B_q: int, B_kv: int, causal: bool, out=None,
                  workspace=None, stream=None):
    import torch
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(shape, B_q, B_kv, causal, x.device)
    B.bpt_layer_fwd(shape, x, *w.as_tuple(), B_q, B_kv, causal, out, workspace, stream)
    return out


def last_group_rows(shape, B_q: int, ffn_rows: int = 0) -> int:
    """Rows of the last FFN group (what bpt_debug_intermediates' H_out holds)."""
    T = shape.batch * shape.seq
    G = ffn_rows or B.bpt_layer_epilogue_rows(shape, B_q)
    return T - G * ((T - 1) // G)


def layer_forward_debug(shape, x, w: DeviceWeights, B_q: int, B_kv: int, causal: bool,
                        workspace=None, stream=None, ffn_rows: int = 0, want_H: bool = False):
    """Returns (out, A, y) device tensors, from the same kernels as the layer;
    with ``want_H`` also the last FFN group's hidden activations [n, ffn]."""
    import torch
    out = torch.empty_like(x)
    A = torch.empty_like(x)
    y = torch.empty_like(x)
    H = None
    if want_H:
        H = torch.empty((last_group_rows(shape, B_q, ffn_rows), shape.ffn), dtype=x.dtype,
                        device=x.device)
    if workspace is None:
        n = B.bpt_layer_workspace_bytes_ex(shape, B_q, B_kv, causal, ffn_rows)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    B.bpt_debug_intermediates(shape, x, *w.as_tuple(), B_q, B_kv, causal, ffn_rows, out, A, y, H,
                              workspace, stream)
    return (out, A, y, H) if want_H else (out, A, y)


def stack_forward(shape, x, layers: Sequence[DeviceWeights], B_q: int, B_kv: int, causal: bool,
                  workspace=None, keep_all: bool = False, stream=None):
    """Apply layers in turn, ping-ponging two activation buffers and reusing
    one workspace. Returns the final output (and every layer's output if
    ``keep_all``)."""
    import torch
    if workspace is None:
        workspace = alloc_workspace(shape, B_q, B_kv, causal, x.device)
    outs: List = []
    bufs = [torch.empty_like(x), torch.empty_like(x)]
    cur = x
    for i, w in enumerate(layers):
        dst = bufs[i % 2] if not keep_all else torch.empty_like(x)
        B.bpt_layer_fwd(shape, cur, *w.as_tuple(), B_q, B_kv, causal, dst, workspace, stream)
        if keep_all:
            outs.append(dst)
        cur = dst
    return (cur, outs) if keep_all else cur


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(device="cpu", dtype=torch.float64).numpy()
