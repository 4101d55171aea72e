"""A CPU model of the pipelined loops that load memory straight into LDS.

The GEMM (csrc/gemm_bf16.hip), the attention forward (csrc/attn_bf16.h) and
the two attention-backward kernels (csrc/attn_bwd.hip) fill rings of LDS
buffers with ``buffer_load_dword[x4] ... lds`` and order every read of a
filled buffer with hand-counted ``s_waitcnt vmcnt(n)`` and ``s_barrier``.
Each generator below writes out, per wave, the sequence one wave of one
workgroup executes: every load into LDS (which LDS bytes, which stage of
which operand), every wait (its vmcnt and whether it also waits for LDS
operations), every barrier, and every LDS read of a ring buffer, with the
stage the read expects to find there. The generators follow the kernels'
control flow step for step (prologue, bulk and tail steps, the conditions on
each load and wait) with the kernels' own constants.

``check`` then executes the waves' programs against the hardware's ordering
rules and reports every read that could see anything but the stage it
expects:

* a wave's vector-memory loads complete in issue order, and ``vmcnt(n)``
  returns once at most n of the wave's vector-memory operations are
  outstanding; so after it every load except the youngest n loads is
  complete. Stores may complete in any order: the model lets them complete
  at once, which leaves the most loads in flight (the worst case);
* an LDS read is complete at the next wait for LDS operations in its wave,
  or at the point where its value is used;
* ``s_barrier``: whatever a wave completed before it happens before whatever
  any wave starts after it.

An access A happens before an access B when A's completion precedes B's start
in one wave's program order, or, in two waves, when a barrier lies between
them. Every read must see its stage: some load of that stage into each
256-byte LDS cell it reads happens before it, and every load of another stage
into that cell either happens before one of those loads or after the read.
Loads of different stages into one cell must be ordered. Every load must be
complete when the program ends, and every wave must take the same number of
barriers.
"""
from __future__ import annotations

from collections import defaultdict
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

CELL = 256  # bytes: LDS is tracked in cells of this size


@dataclass
class Ev:
    kind: str                      # load | vload | vstore | wait | barrier | read | use | write
    lo: int = 0                    # LDS byte range [lo, hi) (load, read, write)
    hi: int = 0
    tag: object = None             # stage written (load) or expected (read); None: value unused
    vm: Optional[int] = None       # wait: vmcnt, or None for no vector-memory wait
    lgkm: bool = False             # wait: also wait for every LDS operation
    key: object = None             # read / use: identifies the reads a `use` completes


def load(lo, nbytes, tag):
    return Ev("load", lo, lo + nbytes, tag)


def read(lo, nbytes, tag, key=None):
    return Ev("read", lo, lo + nbytes, tag, key=key)


def use(key):
    return Ev("use", key=key)


def wait(vm=None, lgkm=False):
    if vm is not None and not 0 <= vm <= 63:
        raise ValueError(f"vmcnt({vm}) does not fit the 6-bit field")
    return Ev("wait", vm=vm, lgkm=lgkm)


BARRIER = Ev("barrier")


@dataclass
class Access:
    wave: int
    kind: str                      # L (load into LDS), R (read), W (write)
    cells: range
    tag: object
    start: Tuple[int, int]         # (phase, index) in the wave's program
    end: Optional[Tuple[int, int]] = None
    text: str = ""
    key: object = None


def _hb(a: Access, b: Access) -> bool:
    """a completes before b starts."""
    if a.end is None:
        return False
    if a.wave == b.wave:
        return a.end[1] < b.start[1]
    return a.end[0] < b.start[0]


def run(programs: Sequence[Sequence[Ev]]):
    """Execute the waves' programs; returns (accesses, errors, waits) where
    waits lists (wave, vmcnt) of every wait with a vmcnt issued while a load
    into LDS may be outstanding (issued since the wave's last vmcnt(0))."""
    errs: List[str] = []
    accs: List[Access] = []
    waits: List[Tuple[int, int]] = []
    nbar = [sum(1 for e in p if e.kind == "barrier") for p in programs]
    if len(set(nbar)) > 1:
        errs.append(f"waves take different numbers of barriers {nbar}: the workgroup hangs")
    for w, prog in enumerate(programs):
        phase = 0
        loads: List[Access] = []     # outstanding loads (into LDS or not), issue order
        stores = 0
        pending: List[Access] = []   # LDS reads and writes not yet complete
        dma_since_zero = False
        for i, e in enumerate(prog):
            pos = (phase, i)
            if e.kind == "load":
                a = Access(w, "L", range(e.lo // CELL, (e.hi + CELL - 1) // CELL), e.tag, pos,
                           text=f"wave {w} load of {e.tag} at {e.lo}")
                accs.append(a)
                loads.append(a)
                dma_since_zero = True
            elif e.kind == "vload":
                loads.append(Access(w, "V", range(0), None, pos))
            elif e.kind == "vstore":
                stores += 1
            elif e.kind == "wait":
                if e.vm is not None:
                    if dma_since_zero:
                        waits.append((w, e.vm))
                    stores = 0  # worst case: every store completed first
                    while len(loads) > e.vm:
                        loads.pop(0).end = pos
                    if e.vm == 0:
                        dma_since_zero = False
                if e.lgkm:
                    for a in pending:
                        a.end = pos
                    pending = []
            elif e.kind == "barrier":
                phase += 1
            elif e.kind in ("read", "write"):
                a = Access(w, "R" if e.kind == "read" else "W",
                           range(e.lo // CELL, (e.hi + CELL - 1) // CELL), e.tag, pos,
                           text=f"wave {w} {e.kind} of {e.tag} at {e.lo} (event {i}, phase {phase})",
                           key=e.key)
                accs.append(a)
                pending.append(a)
            elif e.kind == "use":
                keep = []
                for a in pending:
                    if a.kind == "R" and a.key == e.key:
                        a.end = pos
                    else:
                        keep.append(a)
                pending = keep
            else:
                raise ValueError(e.kind)
        if any(a.kind == "L" for a in loads):
            errs.append(f"wave {w}: {sum(a.kind == 'L' for a in loads)} load(s) into LDS still "
                        f"outstanding when the program ends")
        for a in pending:
            a.end = (phase, len(prog))
    return accs, errs, waits


def check(programs: Sequence[Sequence[Ev]], limit: int = 20):
    """Errors of the programs (empty when every read sees its stage), and the
    (wave, vmcnt) waits issued while loads into LDS may be outstanding."""
    accs, errs, waits = run(programs)
    by_cell: Dict[int, List[Access]] = defaultdict(list)
    for a in accs:
        for c in a.cells:
            by_cell[c].append(a)
    for c, lst in sorted(by_cell.items()):
        writes = [a for a in lst if a.kind in ("L", "W")]
        for r in (a for a in lst if a.kind == "R" and a.tag is not None):
            mine = [x for x in writes if x.tag == r.tag and _hb(x, r)]
            if not mine:
                late = [x for x in writes if x.tag == r.tag]
                errs.append(f"cell {c}: {r.text} follows no wait covering a load of its stage"
                            + (f" ({late[0].text} is not ordered before it)" if late else
                               " (no load of that stage)"))
                continue
            for x in writes:
                if x.tag == r.tag:
                    continue
                if not (any(_hb(x, m) for m in mine) or _hb(r, x)):
                    errs.append(f"cell {c}: {r.text} may see {x.text}")
        for i, a in enumerate(writes):
            for b in writes[i + 1:]:
                if a.tag != b.tag and not (_hb(a, b) or _hb(b, a)):
                    errs.append(f"cell {c}: {a.text} and {b.text} are unordered")
        if len(errs) > limit:
            break
    return errs[:limit], waits


# ---------------------------------------------------------------- GEMM
GEMM_AHEAD, GEMM_TK = 3, 32
GEMM_TILE = 256 * GEMM_TK * 2          # bytes of one operand tile of one stage
GEMM_NLOAD = 8                         # loads per wave per stage: 4 KiB of A, 4 of B


def gemm_programs(KT: int, ahead: int = GEMM_AHEAD, nstage: Optional[int] = None,
                  wait_prev: Optional[int] = None, extra=None) -> List[List[Ev]]:
    """The 4 waves of one gemm_bf16_kernel workgroup over KT = K / 32 steps,
    with the kernel's ring of ``nstage`` = AHEAD + 1 buffers loaded ``ahead``
    steps ahead. ``wait_prev`` replaces the loading steps' wait for the
    stages after the one they need ((AHEAD - 2)·8 loads), and a smaller
    ``nstage`` shrinks the ring: both only to plant mistakes. ``extra(wave,
    kt)`` may return events to insert after a step's loads (compiler-issued
    memory operations)."""
    nstage = ahead + 1 if nstage is None else nstage
    steady = (ahead - 2) * GEMM_NLOAD if wait_prev is None else wait_prev
    progs = []
    for w in range(4):
        p: List[Ev] = []

        def stage_one(kt, buf, i):
            base = buf * 2 * GEMM_TILE + (0 if i < 4 else GEMM_TILE)
            p.append(load(base + (w * 4 + i % 4) * 1024, 1024, kt))

        def read_step(kt):
            buf = kt % nstage
            # every fragment of step kt: both operand tiles of its buffer
            # (after the last step the kernel reads a stale buffer it never uses)
            p.append(read(buf * 2 * GEMM_TILE, 2 * GEMM_TILE, kt if kt < KT else None, key=kt))

        def body(kt, load_, wait_):
            p.append(wait(wait_, lgkm=False))   # barrier_vm_only: LDS reads stay in flight
            p.append(BARRIER)
            read_step(kt + 1)                  # 16 fragment reads of step kt+1, spread over the slots
            if load_:
                for q in range(32):
                    if q & 3 == 1:
                        stage_one(kt + ahead, (kt + ahead) % nstage, q >> 2)
            if extra:
                p.extend(extra(w, kt))
            p.append(use(kt))                  # the step's MFMAs consume the fragments of step kt

        for s in range(ahead):
            for i in range(GEMM_NLOAD):
                stage_one(min(s, KT - 1), s % nstage, i)
        p.append(wait((ahead - 1) * GEMM_NLOAD, lgkm=True))
        p.append(BARRIER)
        read_step(0)
        KL = KT - ahead
        kt = 0
        while kt + 1 < KL:
            body(kt, True, steady)
            body(kt + 1, True, steady)
            kt += 2
        if kt < KL:
            body(kt, True, steady)
            kt += 1
            p.append(use(kt))                  # f0 = f1: register moves of step kt's fragments
        # the last AHEAD steps load nothing; at step kt + t the stages after
        # kt+t+1 (at most AHEAD-2-t) may still be loading
        for t in range(ahead):
            if t == 0 or kt + t < KT:
                body(kt + t, False, steady if t == 0 else max(ahead - 2 - t, 0) * GEMM_NLOAD)
        p.append(wait(0, lgkm=True))           # wait_vm<0>
        p.append(wait(None, lgkm=True))        # __syncthreads, then the epilogue
        p.append(BARRIER)                      # stages the tile through the ring's LDS
        p.append(Ev("write", 0, 128 * 1024, "epilogue"))
        progs.append(p)
    return progs


# ---------------------------------------------------------------- attention forward
ATTN_NSTAGE = 4


def attn_geometry(D: int, WQ: int, KB: int):
    NBLK = KB * D * 2 // 1024          # KiB blocks per K (and per V^T) stage
    LOADS = (NBLK + WQ - 1) // WQ
    return NBLK, LOADS


def attn_workgroups(s: int, rows: int, causal: bool) -> List[List[int]]:
    """The query tiles each workgroup of one (batch, head) takes, in order:
    causal with more than one wave (rows > 32), tiles n_qt-1-p and p (one
    tile when they coincide); else tile n_qt-1-p."""
    n_qt = (s + rows - 1) // rows
    if not (rows > 32 and causal and n_qt > 1):
        return [[n_qt - 1 - p] for p in range(n_qt)]
    return [[n_qt - 1 - p] + ([p] if 2 * p + 1 != n_qt else []) for p in range((n_qt + 1) // 2)]


def attn_fwd_programs(D: int, WQ: int, KB: int, s: int, causal: bool, tiles, rows: int,
                      step_wait_extra: int = 0, drop_step_barrier: bool = False,
                      extra=None) -> List[List[Ev]]:
    """The WQ waves of an attn_fwd_bf16_kernel workgroup that takes the query
    tiles ``tiles`` in turn (tile qt: rows query rows from qt·rows) of one
    (batch, head) with s keys. ``step_wait_extra`` and ``drop_step_barrier``
    plant mistakes. A stage's tag names its tile's position in ``tiles``."""
    if isinstance(tiles, int):
        tiles = [tiles]
    progs = [[] for _ in range(WQ)]
    for part, qt in enumerate(tiles):
        for w, prog in enumerate(_attn_tile(D, WQ, KB, s, causal, qt, rows, part,
                                            step_wait_extra, drop_step_barrier, extra)):
            progs[w].extend(prog)
    return progs


def _attn_tile(D, WQ, KB, s, causal, qt, rows, part, step_wait_extra, drop_step_barrier, extra):
    NBLK, LOADS = attn_geometry(D, WQ, KB)
    stage_bytes = KB * D * 2
    VBASE = ATTN_NSTAGE * stage_bytes
    q0 = qt * rows
    row_end = min(s, q0 + rows)
    kv_end = row_end if causal else s
    n_st = (kv_end + KB - 1) // KB
    progs = []
    for w in range(WQ):
        p: List[Ev] = []
        qw0 = q0 + w * 32
        wq_last = min(qw0 + 31, row_end - 1)
        nw = 0 if wq_last < qw0 else (min(n_st, wq_last // KB + 1) if causal else n_st)
        n_um = min(nw, min((qw0 + 1) // KB if causal else s // KB, s // KB))

        def issue(op, st, i):
            blk = w + WQ * i
            if blk < NBLK:
                base = (0 if op == "K" else VBASE) + (st % ATTN_NSTAGE) * stage_bytes
                p.append(load(base + blk * 1024, 1024, (part, op, st)))

        def issue_all(op, st):
            for i in range(LOADS):
                issue(op, st, i)

        def rd(op, st):
            base = (0 if op == "K" else VBASE) + (st % ATTN_NSTAGE) * stage_bytes
            p.append(read(base, stage_bytes, (part, op, st)))

        def barrier(vm):
            p.append(wait(vm + step_wait_extra if vm else vm, lgkm=True))
            if not drop_step_barrier:
                p.append(BARRIER)

        def step_bulk(st):
            rd("K", st + 1)                    # scores of stage st+1 (ring reads run ahead)
            rd("V", st)                        # P·V of stage st
            # the loads, spread over the issue slots in order: K(st+3), then V(st+2)
            for i in range(LOADS):
                issue("K", st + 3, i)
            for i in range(LOADS):
                issue("V", st + 2, i)
            if extra:
                p.extend(extra(w, st))
            barrier(2 * LOADS)

        def step(st):
            if st + 3 < n_st:
                issue_all("K", st + 3)
            if st + 2 < n_st:
                issue_all("V", st + 2)
            if st < nw:
                if st + 1 < nw:
                    rd("K", st + 1)
                rd("V", st)
            if extra:
                p.extend(extra(w, st))
            if st + 3 < n_st:
                barrier(2 * LOADS)
            elif st + 2 < n_st:
                barrier(LOADS)
            else:
                barrier(0)

        issue_all("K", 0)
        issue_all("V", 0)
        if n_st > 1:
            issue_all("K", 1)
            issue_all("V", 1)
        if n_st > 2:
            issue_all("K", 2)
        p.append(wait(0, lgkm=True))
        p.append(BARRIER)
        rd("K", 0)
        st = 0
        while st + 2 < n_um:
            step_bulk(st)
            step_bulk(st + 1)
            st += 2
        while st < n_st:
            step(st)
            if st + 1 < n_st:
                step(st + 1)
            st += 2
        p.append(wait(0, lgkm=True))
        progs.append(p)
    return progs


# ---------------------------------------------------------------- attention backward
BW_NST, BW_AHEAD = 4, 2


def _bw_sync(p, t, nblk, NL, stage):
    p.append(wait(NL * (BW_AHEAD - 1) if (BW_AHEAD > 1 and t + BW_AHEAD - 1 < nblk) else 0, lgkm=True))
    p.append(BARRIER)
    if t + BW_AHEAD < nblk:
        stage(t + BW_AHEAD)


def _bw_walk(p, nblk, NL, stage, rd_score, rd_grad):
    """Blocks 1 .. nblk-1 as the kernels walk them: four per loop iteration
    (block t in ring slot t % 4), then the 0 to 3 left, then the last block's
    gradient reads."""
    def step(t):
        _bw_sync(p, t, nblk, NL, stage)
        rd_score(t)
        rd_grad(t - 1)

    t = 1
    while t + 3 < nblk:
        for tt in range(t, t + 4):
            step(tt)
        t += 4
    for tt in range(t, nblk):      # the tail: 0 to 3 steps
        step(tt)
    rd_grad(nblk - 1)


def attn_bwd_dkv_programs(D: int, DK: bool, s: int, causal: bool, y: int) -> List[List[Ev]]:
    """The 4 waves of attn_bwd_dkv_kernel's workgroup y (keys 128y ..) of one
    (batch, head) with s tokens; DK selects the dK kernel, else dV."""
    BLKB = 32 * D * 2                  # bytes of one operand block
    NOP, NPC = 2, D // 16
    NLO = (NOP * NPC + 3) // 4
    NL = NLO + 1
    STG = NOP * BLKB + 512             # + log-sum-exps and D values, 64 floats each
    K0 = 128 * y
    qfirst = K0 if causal else 0
    nblk = (s - qfirst + 31) // 32
    progs = []
    for w in range(4):
        p: List[Ev] = []
        st_d = DK and (w & 1)

        def stage(j):
            S = (j % BW_NST) * STG
            for t in range(NLO):
                i = t * 4 + w
                if i >= NOP * NPC:
                    i = w % (NOP * NPC)
                o, pc = divmod(i, NPC)
                p.append(load(S + o * BLKB + pc * 1024, 1024, j))
            p.append(load(S + NOP * BLKB + (256 if st_d else 0), 256, j))

        def rd_score(j):
            S = (j % BW_NST) * STG
            if DK:
                p.append(read(S, 2 * BLKB, j))            # Qs and dO rows
                p.append(read(S + NOP * BLKB, 512, j))    # lse and D
            else:
                p.append(read(S, BLKB, j))                # Qs rows
                p.append(read(S + NOP * BLKB, 128, j))    # lse

        def rd_grad(j):
            S = (j % BW_NST) * STG
            p.append(read(S if DK else S + BLKB, BLKB, j))  # Qs read transposed / dO^T

        p.append(wait(0, lgkm=True))   # the K and V fragments, before any load into LDS
        for j in range(BW_AHEAD):
            if j < nblk:
                stage(j)
        _bw_sync(p, 0, nblk, NL, stage)
        rd_score(0)
        _bw_walk(p, nblk, NL, stage, rd_score, rd_grad)
        p.append(wait(0, lgkm=True))
        progs.append(p)
    return progs


def attn_bwd_dq_programs(D: int, s: int, causal: bool, y: int, n_y: int) -> List[List[Ev]]:
    """The 4 waves of attn_bwd_dq_kernel's workgroup y of n_y (queries
    128·y' .., where y' = n_y - 1 - y when causal) with s tokens."""
    BLKB = 32 * D * 2
    NPC = D // 16
    NL = (2 * NPC + 3) // 4
    STG = 2 * BLKB
    Q0 = (n_y - 1 - y if causal else y) * 128
    kend = min(Q0 + 128, s) if causal else s
    nblk = (kend + 31) // 32
    progs = []
    for w in range(4):
        p: List[Ev] = []

        def stage(j):
            S = (j % BW_NST) * STG
            for t in range(NL):
                i = t * 4 + w
                if i >= 2 * NPC:
                    i = w % (2 * NPC)
                o, pc = divmod(i, NPC)
                p.append(load(S + o * BLKB + pc * 1024, 1024, j))

        def rd_score(j):
            p.append(read((j % BW_NST) * STG, 2 * BLKB, j))   # K and V rows

        def rd_grad(j):
            p.append(read((j % BW_NST) * STG, BLKB, j))       # K read transposed

        p.append(wait(0, lgkm=True))
        for j in range(BW_AHEAD):
            if j < nblk:
                stage(j)
        _bw_sync(p, 0, nblk, NL, stage)
        rd_score(0)
        _bw_walk(p, nblk, NL, stage, rd_score, rd_grad)
        p.append(wait(0, lgkm=True))
        progs.append(p)
    return progs
