"""Seeded synthetic inputs for the BPT layer forward.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, so both the GPU path and the fp64
CPU oracle can consume the same arrays without sharing any computation.

Recipe (the same for every workload):
  * generator: numpy PCG64 (``numpy.random.default_rng``), float32 standard
    normal draws, scaled by the stated standard deviation in float32;
  * bf16 workloads round every value once to bf16 with round-to-nearest-even
    (integer arithmetic on the float32 bit pattern, below); the float32 array
    returned then holds exactly the bf16 values;
  * draw order within one layer: x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2; a
    bias whose standard deviation is 0 is all zeros and consumes no draws;
  * single-layer workloads draw everything from ``default_rng(seed)``; a
    stack draws x from ``default_rng(seed)`` and layer l's weights from
    ``default_rng([seed, l])``.

Weight layout is [in, out] (the ``x @ W`` convention of the position-wise FFN
formula on the BPT paper-review page, section "核心公式"); the fused QKV
weight is [h, 3h] with column blocks [Q | K | V] and head n of each block at
columns n*d .. n*d+d-1.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np


# --------------------------------------------------------------------------
# bf16 rounding (storage only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, returning the 16-bit patterns (uint16).

    Round-to-nearest, ties-to-even on the discarded 16 low bits. Finite
    inputs only (the generators never produce inf or nan).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the float32 values they denote."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array holding the nearest bf16 values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    causal: bool
    B_q: int
    B_kv: int
    weight_std: float
    bias_std: float
    seed: int
    layers: int = 1
    sweep_q: tuple = ()
    sweep_kv: tuple = ()

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a small fp32 one, and four bf16 ones (bf16 storage,
# fp32 accumulation). Biases: zero where stated, N(0, 0.01) where stated,
# zero where the workload does not mention them.
WORKLOADS: Dict[str, Workload] = {
    "c1_fp32_s256_h64": Workload("c1_fp32_s256_h64", "f32", 1, 256, 64, 2, 256, False,
                                 64, 64, 0.02, 0.0, 0),
    "c2_bf16_b2_s8k_h2048": Workload("c2_bf16_b2_s8k_h2048", "bf16", 2, 8192, 2048, 16, 8192,
                                     True, 512, 512, 0.02, 0.01, 1),
    "c3_bf16_s32k_h2048": Workload("c3_bf16_s32k_h2048", "bf16", 1, 32768, 2048, 16, 8192,
                                   True, 1024, 512, 0.02, 0.0, 2,
                                   sweep_q=(512, 1024, 2048), sweep_kv=(256, 512, 1024)),
    "c4_bf16_s16k_h4096": Workload("c4_bf16_s16k_h4096", "bf16", 1, 16384, 4096, 32, 16384,
                                   True, 1024, 512, 0.02, 0.0, 3),
    "c5_bf16_s128k_h2048_x4": Workload("c5_bf16_s128k_h2048_x4", "bf16", 1, 131072, 2048, 16,
                                       8192, True, 2048, 1024, 0.02, 0.0, 4, layers=4),
}
WORKLOAD_ORDER: List[str] = list(WORKLOADS)


@dataclasses.dataclass
class LayerWeights:
    """One layer's parameters as float32 arrays (bf16-exact for bf16)."""
    Wqkv: np.ndarray  # [h, 3h]
    bqkv: np.ndarray  # [3h]
    Wo: np.ndarray    # [h, h]
    bo: np.ndarray    # [h]
    W1: np.ndarray    # [h, f]
    b1: np.ndarray    # [f]
    W2: np.ndarray    # [f, h]
    b2: np.ndarray    # [h]

    def as_tuple(self):
        return (self.Wqkv, self.bqkv, self.Wo, self.bo, self.W1, self.b1, self.W2, self.b2)


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    if std == 0.0:
        return np.zeros(shape, dtype=np.float32)
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "bf16":
        a = round_to_bf16(a)
    return a


def draw_weights(rng: np.random.Generator, hidden: int, ffn: int, weight_std: float,
                 bias_std: float, dtype: str) -> LayerWeights:
    h, f = hidden, ffn
    Wqkv = _draw(rng, (h, 3 * h), weight_std, dtype)
    bqkv = _draw(rng, (3 * h,), bias_std, dtype)
    Wo = _draw(rng, (h, h), weight_std, dtype)
    bo = _draw(rng, (h,), bias_std, dtype)
    W1 = _draw(rng, (h, f), weight_std, dtype)
    b1 = _draw(rng, (f,), bias_std, dtype)
    W2 = _draw(rng, (f, h), weight_std, dtype)
    b2 = _draw(rng, (h,), bias_std, dtype)
    return LayerWeights(Wqkv, bqkv, Wo, bo, W1, b1, W2, b2)


def make_inputs(w: Workload, seq: Optional[int] = None, batch: Optional[int] = None):
    """Return (x [b, s, h] float32, [LayerWeights per layer]).

    ``seq``/``batch`` override the workload's sizes (same recipe, same seed);
    tests use this to run a workload's structure at a size the oracle
    finishes quickly.
    """
    b = w.batch if batch is None else batch
    s = w.seq if seq is None else seq
    rng = np.random.default_rng(w.seed)
    x = _draw(rng, (b, s, w.hidden), 1.0, w.dtype)
    layers = []
    if w.layers == 1:
        layers.append(draw_weights(rng, w.hidden, w.ffn, w.weight_std, w.bias_std, w.dtype))
    else:
        for l in range(w.layers):
            lr = np.random.default_rng([w.seed, l])
            layers.append(draw_weights(lr, w.hidden, w.ffn, w.weight_std, w.bias_std, w.dtype))
    return x, layers


def sample_rows(seq: int, B_q: int, n_random: int, seed: int = 1234) -> np.ndarray:
    """Query rows to check at sizes where the oracle cannot do every row.

    Includes rows 0, 1, s-1, both sides of every query-block boundary and
    ``n_random`` seeded random rows; sorted and unique.
    """
    rows = {0, min(1, seq - 1), seq - 1}
    for st in range(0, seq, B_q):
        rows.add(st)
        rows.add(min(st + B_q - 1, seq - 1))
    rng = np.random.default_rng(seed)
    if n_random > 0:
        rows.update(int(r) for r in rng.integers(0, seq, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)
