"""The hand-counted waits of the LDS rings, checked on the CPU.

tests/lds_schedule.py writes out the issue / wait / barrier / read sequence
of every wave of a workgroup for the GEMM, the attention forward (every
instance the library builds) and the two attention-backward kernels, over
trip counts that cover the prologue, the bulk loop (odd and even lengths),
the tail steps, causal tiles whose waves stop at different stages, partial
last tiles and a single short stage. Every LDS read must see the stage it
expects, with no load of another stage racing it.

Three more kinds of test:
* planted miscounts (a wait one stage too lax, a load one stage too far
  ahead, a missing barrier) must be reported, so the model is not vacuous;
* vector-memory operations the compiler may add anywhere (spill reloads,
  stores completing in any order) must not break any count;
* the waits the model issues while loads into LDS are outstanding must be
  exactly the vmcnt values the compiled kernels carry (the assembly of the
  library sources, compiled for gfx950), so the model and the code it
  describes cannot drift apart unnoticed.
"""
import re

import pytest

from blockwise_attention_ffn_amd import asm_check as C

from tests.lds_schedule import (Ev, attn_bwd_dkv_programs, attn_bwd_dq_programs, attn_fwd_programs,
                                attn_geometry, attn_workgroups, check, gemm_programs)

GEMM_KT = list(range(1, 14)) + [64, 256]   # K = 32·KT: 32 .. 416, 2048, 8192
ATTN_CONFIGS = [(D, WQ, KB) for D in (32, 64, 128) for WQ in (1, 2, 4, 8) for KB in (16, 32, 64)]
BWD_S = [1, 31, 32, 33, 96, 100, 128, 129, 224, 300, 515]  # every tail of the block walk (0-3 steps)


def _rows(WQ):
    return (16, 32) if WQ == 1 else (32 * WQ,)


def _attn_cases(D, WQ, KB):
    for rows in _rows(WQ):
        for s in sorted({1, KB - 1, KB, 2 * KB + 5, 3 * KB, rows + 7, 2 * rows, 5 * KB + 3,
                         13 * KB, 2 * rows + 3 * KB + 1}):
            if s < 1:
                continue
            for causal in (False, True):
                for tiles in attn_workgroups(s, rows, causal):
                    yield rows, s, causal, tiles


def _no_errors(errs, what):
    assert errs == [], f"{what}:\n" + "\n".join(errs)


# ---------------------------------------------------------------- the kernels as built
def gemm_waits():
    waits = set()
    for KT in GEMM_KT:
        errs, w = check(gemm_programs(KT))
        _no_errors(errs, f"GEMM, K = {32 * KT}")
        waits |= {v for _, v in w}
    return waits


def attn_waits(D, WQ, KB):
    waits = set()
    for rows, s, causal, tiles in _attn_cases(D, WQ, KB):
        errs, w = check(attn_fwd_programs(D, WQ, KB, s, causal, tiles, rows))
        _no_errors(errs, f"attention d={D} waves={WQ} keys={KB} rows={rows} s={s} "
                         f"causal={causal} tiles {tiles}")
        waits |= {v for _, v in w}
    return waits


def bwd_waits(kind, D):
    waits = set()
    for s in BWD_S:
        n_y = (s + 127) // 128
        for causal in (False, True):
            for y in range(n_y):
                if kind == "dq":
                    progs = attn_bwd_dq_programs(D, s, causal, y, n_y)
                else:
                    progs = attn_bwd_dkv_programs(D, kind == "dk", s, causal, y)
                errs, w = check(progs)
                _no_errors(errs, f"backward {kind} d={D} s={s} causal={causal} workgroup {y}")
                waits |= {v for _, v in w}
    return waits


def test_gemm_every_read_sees_its_stage():
    assert gemm_waits() == {16, 8, 0}


@pytest.mark.parametrize("D,WQ,KB", ATTN_CONFIGS)
def test_attention_every_read_sees_its_stage(D, WQ, KB):
    _, LOADS = attn_geometry(D, WQ, KB)
    assert attn_waits(D, WQ, KB) == {0, LOADS, 2 * LOADS}


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("kind", ["dv", "dk", "dq"])
def test_backward_every_read_sees_its_stage(kind, D):
    assert bwd_waits(kind, D)


def test_attention_workgroups_cover_every_tile_once():
    for s in (1, 15, 16, 17, 255, 256, 257, 1000, 4096):
        for rows in (16, 32, 64, 128, 256):
            n_qt = (s + rows - 1) // rows
            for causal in (False, True):
                wgs = attn_workgroups(s, rows, causal)
                assert sorted(t for w in wgs for t in w) == list(range(n_qt))
                if rows > 32 and causal and n_qt > 1:
                    # equal stage counts, one workgroup short by a tile when n_qt is odd
                    assert len({sum(t + 1 for t in w) for w in wgs if len(w) == 2}) == 1


def test_attention_geometry_has_no_partial_wave():
    """The step waits count LOADS loads per operand for every wave; a wave
    that issued some but fewer would leave older stages in flight. K and V^T
    stages are whole KiB blocks, NBLK = KB·D/512, and both NBLK and the wave
    count are powers of two, so each wave issues LOADS loads or none."""
    for D, WQ, KB in ATTN_CONFIGS:
        NBLK, LOADS = attn_geometry(D, WQ, KB)
        per_wave = {sum(1 for i in range(LOADS) if w + WQ * i < NBLK) for w in range(WQ)}
        assert per_wave <= {0, LOADS}, (D, WQ, KB, per_wave)


# ---------------------------------------------------------------- planted mistakes
def test_gemm_wait_one_stage_too_lax_is_caught():
    errs, _ = check(gemm_programs(8, wait_prev=16))
    assert any("follows no wait covering" in e for e in errs)


def test_gemm_load_one_stage_too_far_ahead_is_caught():
    # AHEAD = 4 with 4 buffers: step kt refills the buffer of stage kt, whose
    # fragments the step's MFMAs are still consuming
    errs, _ = check(gemm_programs(9, ahead=4, nstage=4, wait_prev=8))
    assert any("may see" in e or "unordered" in e for e in errs)


def test_attention_wait_one_load_too_lax_is_caught():
    errs, _ = check(attn_fwd_programs(128, 8, 64, 4096, False, 0, 256, step_wait_extra=1))
    assert any("follows no wait covering" in e for e in errs)


def test_attention_missing_barrier_is_caught():
    errs, _ = check(attn_fwd_programs(64, 4, 32, 1024, True, [7, 0], 128, drop_step_barrier=True))
    assert errs


def test_attention_one_wave_needs_no_barrier():
    # a single wave orders its own loads and reads by its waits alone, which is
    # why the compiler may drop the barriers of the 1-wave instances
    _no_errors(check(attn_fwd_programs(64, 1, 32, 700, True, [21], 32, drop_step_barrier=True))[0],
               "1-wave attention without barriers")


def test_backward_uneven_barriers_are_caught():
    progs = attn_bwd_dq_programs(64, 300, False, 0, 3)
    progs[1] = [e for e in progs[1] if e.kind != "barrier"][:] + [Ev("barrier")]
    errs, _ = check(progs)
    assert any("different numbers of barriers" in e for e in errs)


# ---------------------------------------------------------------- compiler-added operations
def _compiler_ops(w, step):
    # a spill store and reload, and a plain load, in every step window
    return [Ev("vstore"), Ev("vload"), Ev("vstore"), Ev("vload")]


def test_counts_survive_compiler_memory_operations():
    """Loads complete in order, so a load into LDS that is still outstanding
    has every younger load outstanding too: a wait for at most n outstanding
    operations, with n the loads into LDS issued after it, cannot return
    early whatever the compiler adds. Stores are let complete first, the case
    that leaves the most loads in flight."""
    for KT in (5, 8, 64):
        _no_errors(check(gemm_programs(KT, extra=_compiler_ops))[0], f"GEMM K = {32 * KT}")
    for D, WQ, KB, rows, s, causal, tiles in [(128, 8, 64, 256, 2000, True, [7, 0]),
                                              (64, 2, 16, 64, 333, False, [2]),
                                              (32, 1, 32, 16, 129, True, [8])]:
        _no_errors(check(attn_fwd_programs(D, WQ, KB, s, causal, tiles, rows, extra=_compiler_ops))[0],
                   f"attention d={D} waves={WQ} keys={KB}")


# ---------------------------------------------------------------- the compiled code
_GEMM = re.compile(r"gemm_bf16_kernelILi(\d+)ELb([01])ELb([01])E")
_FWD = re.compile(r"attn_fwd_bf16_kernelILi(\d+)ELb([01])ELi(\d+)ELi(\d+)E")
_DKV = re.compile(r"attn_bwd_dkv_kernelILi(\d+)ELb([01])E")
_DQ = re.compile(r"attn_bwd_dq_kernelILi(\d+)E")


def _asm_kernels(library_asm):
    for src, (_, _, asm) in library_asm.items():
        for name, body in C.parse_functions(asm).items():
            waits = C.pending_vmcnt_waits(body)
            if waits:
                yield src, name, {v for _, v in waits}


def test_compiled_waits_match_the_model(library_asm):
    """Each kernel's assembly waits, while loads into LDS may be outstanding,
    for exactly the vmcnt values the model of its loop uses: a count the
    compiler changed or dropped, or a kernel edited without its model, shows
    up here."""
    seen = {"gemm": 0, "fwd": 0, "dkv": 0, "dq": 0}
    cache = {}
    for src, name, asm_waits in _asm_kernels(library_asm):
        if _GEMM.search(name):
            key = ("gemm",)
            seen["gemm"] += 1
        elif m := _FWD.search(name):
            D, _, WQ, KB = (int(x) for x in m.groups())
            key = ("fwd", D, WQ, KB)
            seen["fwd"] += 1
        elif m := _DKV.search(name):
            key = ("dk" if m.group(2) == "1" else "dv", int(m.group(1)))
            seen["dkv"] += 1
        elif m := _DQ.search(name):
            key = ("dq", int(m.group(1)))
            seen["dq"] += 1
        else:
            pytest.fail(f"{src}: kernel {name} loads into LDS but has no model")
        if key not in cache:
            if key[0] == "gemm":
                cache[key] = gemm_waits()
            elif key[0] == "fwd":
                cache[key] = attn_waits(*key[1:])
            else:
                cache[key] = bwd_waits(*key)
        assert asm_waits == cache[key], f"{src}: {name}: assembly waits {sorted(asm_waits)}, " \
                                        f"model {sorted(cache[key])}"
    # every GEMM epilogue kind, every attention instance (+ the log-sum-exp
    # ones), dV and dK, dQ at three head dims
    assert seen["gemm"] >= 8 and seen["fwd"] == 36 + 3 and seen["dkv"] == 6 and seen["dq"] == 3, seen
