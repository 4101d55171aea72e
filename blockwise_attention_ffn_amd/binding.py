"""ctypes binding of the C ABI in include/bpt.h (argument marshalling only).

Every function here has the name of the C entry point it calls and takes
torch tensors (device memory) in place of raw pointers. All computation
happens in the HIP kernels behind the C ABI; there is no fallback: if the
shared library is missing or fails to load, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbpt.so")

BPT_F32 = 0
BPT_BF16 = 1

STATUS_NAMES = {
    0: "BPT_OK", 1: "BPT_ERR_NULL", 2: "BPT_ERR_SHAPE", 3: "BPT_ERR_BLOCK", 4: "BPT_ERR_DTYPE",
    5: "BPT_ERR_ALIGN", 6: "BPT_ERR_ALIAS", 7: "BPT_ERR_WORKSPACE", 8: "BPT_ERR_DEVICE",
    9: "BPT_ERR_HIP", 10: "BPT_ERR_SIZE", 11: "BPT_ERR_DROPOUT", 12: "BPT_ERR_SCRATCH",
}

# bpt_layer_fwd_noalloc's fixed scratch per GPU (BPT_NOALLOC_SCRATCH_BYTES in bpt.h)
NOALLOC_SCRATCH_BYTES = 96 << 20

EXPORTED = [
    "bpt_layer_workspace_bytes", "bpt_layer_epilogue_rows", "bpt_layer_fwd",
    "bpt_layer_workspace_bytes_ex", "bpt_layer_fwd_ex", "bpt_layer_fwd_train",
    "bpt_debug_dropout_keep", "bpt_layer_bwd_workspace_bytes", "bpt_layer_bwd",
    "bpt_debug_intermediates", "bpt_debug_attention", "bpt_layer_algorithmic_flops",
    "bpt_status_string", "bpt_version", "bpt_layer_fwd_noalloc", "bpt_layer_attention_tile",
    "bpt_layer_bwd_train", "bpt_layer_fwd_for_bwd", "bpt_layer_bwd_from_fwd",
]


class BptShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("ffn", ctypes.c_int64), ("dtype", ctypes.c_int32)]

    def __repr__(self):
        return (f"BptShape(b={self.batch}, s={self.seq}, h={self.hidden}, heads={self.heads}, "
                f"f={self.ffn}, dtype={'bf16' if self.dtype == BPT_BF16 else 'f32'})")


class BptError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.name = STATUS_NAMES.get(code, str(code))
        super().__init__(f"{where}: {self.name} ({bpt_status_string(code)})")


_lib = None


def lib():
    """Load libbpt.so once; raise ImportError if it is not built.

    torch is imported first. Its wheel ships its own HIP runtime
    (libamdhip64, SONAME libamdhip64.so.7), and libbpt.so needs a library of
    that SONAME: loaded after torch, it binds to torch's runtime, so the
    process has one HIP runtime and the device pointers and streams torch
    hands over belong to it. Loaded first, libbpt.so would pull in the
    system's runtime and torch would then load its own beside it: two
    runtimes in one process, each blind to the other's streams and state."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m blockwise_attention_ffn_amd.build` (hipcc, gfx950)")
    import torch  # noqa: F401  (before the library: see above)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    SP = ctypes.POINTER(BptShape)
    L.bpt_layer_workspace_bytes.argtypes = [SP, I64, I64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.bpt_layer_workspace_bytes.restype = ctypes.c_int
    L.bpt_layer_epilogue_rows.argtypes = [SP, I64, ctypes.POINTER(I64)]
    L.bpt_layer_epilogue_rows.restype = ctypes.c_int
    L.bpt_layer_fwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int, P, P,
                                ctypes.c_size_t, P]
    L.bpt_layer_fwd.restype = ctypes.c_int
    L.bpt_layer_workspace_bytes_ex.argtypes = [SP, I64, I64, ctypes.c_int, I64,
                                               ctypes.POINTER(ctypes.c_size_t)]
    L.bpt_layer_workspace_bytes_ex.restype = ctypes.c_int
    L.bpt_layer_fwd_ex.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int, I64, P, P,
                                   ctypes.c_size_t, P]
    L.bpt_layer_fwd_ex.restype = ctypes.c_int
    L.bpt_debug_intermediates.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int,
                                          I64, P, P, P, P, P, ctypes.c_size_t, P]
    L.bpt_debug_intermediates.restype = ctypes.c_int
    L.bpt_debug_attention.argtypes = [SP, P, P, P, I64, I64, ctypes.c_int, ctypes.c_int, P, P,
                                      ctypes.c_size_t, P]
    L.bpt_debug_attention.restype = ctypes.c_int
    L.bpt_layer_fwd_train.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int, I64,
                                      ctypes.c_double, ctypes.c_uint64, P, P, ctypes.c_size_t, P]
    L.bpt_layer_fwd_train.restype = ctypes.c_int
    L.bpt_debug_dropout_keep.argtypes = [I64, I64, I64, ctypes.c_double, ctypes.c_uint64,
                                         ctypes.c_int, P, P]
    L.bpt_debug_dropout_keep.restype = ctypes.c_int
    L.bpt_layer_bwd_workspace_bytes.argtypes = [SP, I64, I64, ctypes.c_int, I64,
                                                ctypes.POINTER(ctypes.c_size_t)]
    L.bpt_layer_bwd_workspace_bytes.restype = ctypes.c_int
    L.bpt_layer_bwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int, I64, P, P,
                                P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.bpt_layer_bwd.restype = ctypes.c_int
    L.bpt_layer_bwd_train.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int, I64,
                                      ctypes.c_double, ctypes.c_uint64, P, P, P, P, P, P, P, P, P,
                                      P, P, ctypes.c_size_t, P]
    L.bpt_layer_bwd_train.restype = ctypes.c_int
    L.bpt_layer_fwd_for_bwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int, I64,
                                        ctypes.c_double, ctypes.c_uint64, P, P, ctypes.c_size_t, P]
    L.bpt_layer_fwd_for_bwd.restype = ctypes.c_int
    L.bpt_layer_bwd_from_fwd.argtypes = L.bpt_layer_bwd_train.argtypes
    L.bpt_layer_bwd_from_fwd.restype = ctypes.c_int
    L.bpt_layer_algorithmic_flops.argtypes = [SP, ctypes.c_int]
    L.bpt_layer_algorithmic_flops.restype = ctypes.c_double
    L.bpt_status_string.argtypes = [ctypes.c_int]
    L.bpt_status_string.restype = ctypes.c_char_p
    L.bpt_version.argtypes = []
    L.bpt_version.restype = ctypes.c_char_p
    L.bpt_layer_fwd_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_int, I64,
                                        P, P]
    L.bpt_layer_fwd_noalloc.restype = ctypes.c_int
    L.bpt_layer_attention_tile.argtypes = [SP, I64, I64, ctypes.POINTER(I64), ctypes.POINTER(I64)]
    L.bpt_layer_attention_tile.restype = ctypes.c_int
    _lib = L
    return L


# ----------------------------------------------------------------------------
def make_shape(batch, seq, hidden, heads, ffn, dtype) -> BptShape:
    if isinstance(dtype, str):
        dtype = {"bf16": BPT_BF16, "f32": BPT_F32}[dtype]
    return BptShape(int(batch), int(seq), int(hidden), int(heads), int(ffn), int(dtype))


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the BPT library must be contiguous")
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def bpt_status_string(code: int) -> str:
    return lib().bpt_status_string(int(code)).decode()


def bpt_version() -> str:
    return lib().bpt_version().decode()


def bpt_layer_workspace_bytes(shape: BptShape, B_q: int, B_kv: int, causal: bool) -> int:
    out = ctypes.c_size_t(0)
    st = lib().bpt_layer_workspace_bytes(ctypes.byref(shape), B_q, B_kv, int(bool(causal)),
                                         ctypes.byref(out))
    if st:
        raise BptError(st, "bpt_layer_workspace_bytes")
    return out.value


def bpt_layer_attention_tile(shape: BptShape, B_q: int, B_kv: int):
    """(query rows per workgroup, keys per stage) of the bf16 attention."""
    rows, keys = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib().bpt_layer_attention_tile(ctypes.byref(shape), B_q, B_kv, ctypes.byref(rows),
                                        ctypes.byref(keys))
    if st:
        raise BptError(st, "bpt_layer_attention_tile")
    return rows.value, keys.value


def bpt_layer_epilogue_rows(shape: BptShape, B_q: int) -> int:
    out = ctypes.c_int64(0)
    st = lib().bpt_layer_epilogue_rows(ctypes.byref(shape), B_q, ctypes.byref(out))
    if st:
        raise BptError(st, "bpt_layer_epilogue_rows")
    return out.value


def bpt_layer_algorithmic_flops(shape: BptShape, causal: bool) -> float:
    return float(lib().bpt_layer_algorithmic_flops(ctypes.byref(shape), int(bool(causal))))


def bpt_layer_fwd(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int, B_kv: int,
                  causal: bool, out, workspace, stream=None, check: bool = True) -> int:
    st = lib().bpt_layer_fwd(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv), _ptr(Wo),
                             _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), B_q, B_kv,
                             int(bool(causal)), _ptr(out), _ptr(workspace),
                             _nbytes(workspace) if workspace is not None and not isinstance(workspace, int) else 0,
                             _stream(stream))
    if st and check:
        raise BptError(st, "bpt_layer_fwd")
    return st


def bpt_layer_workspace_bytes_ex(shape: BptShape, B_q: int, B_kv: int, causal: bool,
                                 ffn_rows: int) -> int:
    out = ctypes.c_size_t(0)
    st = lib().bpt_layer_workspace_bytes_ex(ctypes.byref(shape), B_q, B_kv, int(bool(causal)),
                                            ffn_rows, ctypes.byref(out))
    if st:
        raise BptError(st, "bpt_layer_workspace_bytes_ex")
    return out.value


def bpt_layer_fwd_ex(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int, B_kv: int,
                     causal: bool, ffn_rows: int, out, workspace, stream=None) -> None:
    st = lib().bpt_layer_fwd_ex(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv), _ptr(Wo),
                                _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), B_q, B_kv,
                                int(bool(causal)), ffn_rows, _ptr(out), _ptr(workspace),
                                _nbytes(workspace), _stream(stream))
    if st:
        raise BptError(st, "bpt_layer_fwd_ex")


def bpt_layer_fwd_noalloc(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int,
                          B_kv: int, causal: bool, ffn_rows: int, out, stream=None) -> None:
    st = lib().bpt_layer_fwd_noalloc(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv),
                                     _ptr(Wo), _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                     B_q, B_kv, int(bool(causal)), int(ffn_rows), _ptr(out),
                                     _stream(stream))
    if st:
        raise BptError(st, "bpt_layer_fwd_noalloc")


def bpt_layer_fwd_train(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int,
                        B_kv: int, causal: bool, ffn_rows: int, dropout_p: float, seed: int, out,
                        workspace, stream=None) -> None:
    st = lib().bpt_layer_fwd_train(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv),
                                   _ptr(Wo), _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                   B_q, B_kv, int(bool(causal)), ffn_rows, float(dropout_p),
                                   int(seed), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream))
    if st:
        raise BptError(st, "bpt_layer_fwd_train")


def bpt_layer_bwd_workspace_bytes(shape: BptShape, B_q: int, B_kv: int, causal: bool,
                                  ffn_rows: int = 0) -> int:
    out = ctypes.c_size_t(0)
    st = lib().bpt_layer_bwd_workspace_bytes(ctypes.byref(shape), B_q, B_kv, int(bool(causal)),
                                             ffn_rows, ctypes.byref(out))
    if st:
        raise BptError(st, "bpt_layer_bwd_workspace_bytes")
    return out.value


def bpt_layer_bwd(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int, B_kv: int,
                  causal: bool, ffn_rows: int, dout, dx, dWqkv, dbqkv, dWo, dbo, dW1, db1, dW2,
                  db2, workspace, stream=None) -> None:
    st = lib().bpt_layer_bwd(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv), _ptr(Wo),
                             _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), B_q, B_kv,
                             int(bool(causal)), ffn_rows, _ptr(dout), _ptr(dx), _ptr(dWqkv), _ptr(dbqkv),
                             _ptr(dWo), _ptr(dbo), _ptr(dW1), _ptr(db1), _ptr(dW2), _ptr(db2),
                             _ptr(workspace), _nbytes(workspace), _stream(stream))
    if st:
        raise BptError(st, "bpt_layer_bwd")


def bpt_layer_bwd_train(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int,
                        B_kv: int, causal: bool, ffn_rows: int, dropout_p: float, seed: int, dout,
                        dx, dWqkv, dbqkv, dWo, dbo, dW1, db1, dW2, db2, workspace,
                        stream=None) -> None:
    st = lib().bpt_layer_bwd_train(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv), _ptr(Wo),
                                   _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), B_q, B_kv,
                                   int(bool(causal)), ffn_rows, float(dropout_p), int(seed),
                                   _ptr(dout), _ptr(dx), _ptr(dWqkv), _ptr(dbqkv), _ptr(dWo),
                                   _ptr(dbo), _ptr(dW1), _ptr(db1), _ptr(dW2), _ptr(db2),
                                   _ptr(workspace), _nbytes(workspace), _stream(stream))
    if st:
        raise BptError(st, "bpt_layer_bwd_train")


def bpt_layer_fwd_for_bwd(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int,
                          B_kv: int, causal: bool, ffn_rows: int, dropout_p: float, seed: int,
                          out, workspace, stream=None) -> None:
    st = lib().bpt_layer_fwd_for_bwd(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv),
                                     _ptr(Wo), _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                     B_q, B_kv, int(bool(causal)), ffn_rows, float(dropout_p),
                                     int(seed), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                     _stream(stream))
    if st:
        raise BptError(st, "bpt_layer_fwd_for_bwd")


def bpt_layer_bwd_from_fwd(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int,
                           B_kv: int, causal: bool, ffn_rows: int, dropout_p: float, seed: int,
                           dout, dx, dWqkv, dbqkv, dWo, dbo, dW1, db1, dW2, db2, workspace,
                           stream=None) -> None:
    st = lib().bpt_layer_bwd_from_fwd(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv),
                                      _ptr(Wo), _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                      B_q, B_kv, int(bool(causal)), ffn_rows, float(dropout_p),
                                      int(seed), _ptr(dout), _ptr(dx), _ptr(dWqkv), _ptr(dbqkv),
                                      _ptr(dWo), _ptr(dbo), _ptr(dW1), _ptr(db1), _ptr(dW2),
                                      _ptr(db2), _ptr(workspace), _nbytes(workspace),
                                      _stream(stream))
    if st:
        raise BptError(st, "bpt_layer_bwd_from_fwd")


def bpt_debug_dropout_keep(tokens: int, channels: int, token0: int, dropout_p: float, seed: int,
                           site: int, keep, stream=None) -> None:
    st = lib().bpt_debug_dropout_keep(tokens, channels, token0, float(dropout_p), int(seed),
                                      int(site), _ptr(keep), _stream(stream))
    if st:
        raise BptError(st, "bpt_debug_dropout_keep")


def bpt_debug_intermediates(shape: BptShape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q: int,
                            B_kv: int, causal: bool, ffn_rows: int, out, A_out, y_out, H_out,
                            workspace, stream=None) -> None:
    st = lib().bpt_debug_intermediates(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv),
                                       _ptr(Wo), _ptr(bo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                       B_q, B_kv, int(bool(causal)), int(ffn_rows), _ptr(out),
                                       _ptr(A_out), _ptr(y_out), _ptr(H_out), _ptr(workspace),
                                       _nbytes(workspace), _stream(stream))
    if st:
        raise BptError(st, "bpt_debug_intermediates")


def bpt_debug_attention(shape: BptShape, x, Wqkv, bqkv, B_q: int, B_kv: int, causal: bool,
                        run_qkv: bool, A_out, workspace, stream=None) -> None:
    st = lib().bpt_debug_attention(ctypes.byref(shape), _ptr(x), _ptr(Wqkv), _ptr(bqkv), B_q,
                                   B_kv, int(bool(causal)), int(bool(run_qkv)), _ptr(A_out),
                                   _ptr(workspace), _nbytes(workspace), _stream(stream))
    if st:
        raise BptError(st, "bpt_debug_attention")


def bpt_layer_fwd_raw(shape: BptShape, ptrs, B_q, B_kv, causal, out_ptr, ws_ptr, ws_bytes,
                      stream_ptr) -> int:
    """Raw-pointer form used by the host-only validation tests (no tensors):
    ``ptrs`` = (x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2) as ints or None."""
    return lib().bpt_layer_fwd(ctypes.byref(shape), *ptrs, B_q, B_kv, int(bool(causal)), out_ptr,
                               ws_ptr, ws_bytes, stream_ptr)
