"""The backward's small-shape GPU cases reach every tail path of the
attention-backward loops (CPU only: shape arithmetic, no GPU call).

The dV/dK workgroup of key tile y walks the query blocks of 32 from 128·y
(causal) or from 0 to s; the dQ workgroup of query tile y walks the key blocks
of 32 up to min(128·y + 128, s) (causal) or s. Both kernels run block 0, then
four blocks per loop iteration, so (blocks − 1) mod 4 of them are left for
the tail, whose four cases are separate code paths. Each case must be reached
by some GPU parity case at each head dim.
"""
import math

from tests.test_gpu_backward import SMALL_SHAPES


def _tails(s, d, causal):
    out = {"dkv": set(), "dq": set()}
    for y in range(math.ceil(s / 128)):
        first = 128 * y if causal else 0
        out["dkv"].add((math.ceil((s - first) / 32) - 1) % 4)
        end = min(128 * y + 128, s) if causal else s
        out["dq"].add((math.ceil(end / 32) - 1) % 4)
    return out


def test_small_shapes_reach_every_tail_path():
    seen = {(k, d): set() for k in ("dkv", "dq") for d in (32, 64, 128)}
    for b, s, h, nh, f, causal, B_q, B_kv, ffn_rows in SMALL_SHAPES:
        for k, v in _tails(s, h // nh, causal).items():
            seen[(k, h // nh)] |= v
    missing = {k: sorted({0, 1, 2, 3} - v) for k, v in seen.items() if v != {0, 1, 2, 3}}
    assert not missing, f"tail paths no GPU case reaches: {missing}"


def test_tail_arithmetic_on_hand_worked_cases():
    # s = 176, causal: key tile 0 walks 6 query blocks (tail 1), tile 1 walks
    # 2 (tail 1); query tile 0 walks 4 key blocks (tail 3), tile 1 walks 6
    assert _tails(176, 128, True) == {"dkv": {1}, "dq": {1, 3}}
    # s = 208, not causal: 7 blocks everywhere
    assert _tails(208, 128, False) == {"dkv": {2}, "dq": {2}}
