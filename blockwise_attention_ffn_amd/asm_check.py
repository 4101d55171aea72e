"""Static checks of the generated gfx950 code of kernels that load memory
straight into LDS.

The attention and GEMM kernels issue ``buffer_load_dword[x4] ... lds`` from
inline asm and order every LDS read of a loaded buffer with their own
``s_waitcnt vmcnt(n)`` + ``s_barrier`` (csrc/lds_dma.h). Those counts are
exact only under three conditions that the compiler, not the source,
decides. ``check_kernel_asm`` proves each one on the assembly of every kernel
that contains such a load, and the build fails when one does not hold:

1. No scratch memory and no out-of-line calls: spills, reloads and call
   stacks are vector-memory operations the hand counts do not model.
2. While a load into LDS may still be outstanding (from its issue until an
   ``s_waitcnt vmcnt(0)``, followed along every control-flow path), the only
   vector-memory instructions are loads into LDS. A store there could
   complete before an older load and satisfy a ``vmcnt(n)`` wait while that
   load is still in flight; any other load would shift what the counts mean.
3. Wait states the hazard recogniser does not insert for inline asm: an
   SGPR written by a VALU instruction (``v_readfirstlane``, a carry-out, a
   compare) needs 5 wait states before a vector-memory instruction reads it
   (the buffer descriptor, the offset), and an SALU write of M0 needs 1
   before a load into LDS reads it. Both are checked backwards from every
   such load along every path into it.

The parser handles the LLVM AMDGPU assembly printer's output (``hipcc -S``):
functions delimited by ``.type name,@function`` labels and ``.Lfunc_end``,
basic blocks at ``.LBB`` labels and ``; %bb.N:`` markers, and the scalar
branch instructions as block terminators.
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Set, Tuple

VMEM_PREFIXES = ("buffer_", "global_", "flat_", "scratch_", "tbuffer_")
VALU_SGPR_TO_VMEM_WAIT = 5
SALU_M0_TO_LDS_DMA_WAIT = 1


@dataclass
class Instr:
    line: int
    mnemonic: str
    operands: List[str]
    text: str

    @property
    def is_vmem(self) -> bool:
        return self.mnemonic.startswith(VMEM_PREFIXES)

    @property
    def is_lds_dma(self) -> bool:
        return self.mnemonic.startswith("buffer_load") and "lds" in self.operands

    @property
    def wait_states(self) -> int:
        if self.mnemonic == "s_nop":
            try:
                return int(self.operands[0], 0) + 1
            except (IndexError, ValueError):
                return 1
        return 1


@dataclass
class Block:
    label: str
    instrs: List[Instr] = field(default_factory=list)
    succs: List[int] = field(default_factory=list)
    preds: List[int] = field(default_factory=list)


_REG = re.compile(r"^(s|v|a)(?:(\d+)|\[(\d+):(\d+)\])$")


def _split_operands(s: str) -> List[str]:
    out, depth, cur = [], 0, ""
    for ch in s:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            out.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        out.append(cur.strip())
    # trailing modifiers written without commas ("0 offen lds") become items
    flat = []
    for o in out:
        flat.extend(o.split()) if " " in o and "[" not in o else flat.append(o)
    return flat


def sgprs(op: str) -> Set[str]:
    """Scalar registers named by one operand ('s7', 's[4:7]', 'vcc', 'm0')."""
    op = op.strip()
    if op in ("vcc",):
        return {"vcc_lo", "vcc_hi"}
    if op in ("vcc_lo", "vcc_hi", "m0", "exec_lo", "exec_hi"):
        return {op}
    if op == "exec":
        return {"exec_lo", "exec_hi"}
    m = _REG.match(op)
    if not m or m.group(1) != "s":
        return set()
    if m.group(2) is not None:
        return {f"s{m.group(2)}"}
    return {f"s{i}" for i in range(int(m.group(3)), int(m.group(4)) + 1)}


def sgprs_written_by_valu(ins: Instr) -> Set[str]:
    """Scalar registers a VALU instruction writes (empty for others)."""
    mn, ops = ins.mnemonic, ins.operands
    if not mn.startswith("v_") or not ops:
        return set()
    if mn.startswith(("v_readfirstlane", "v_readlane")):
        return sgprs(ops[0])
    if mn.startswith(("v_cmp", "v_cmpx")):
        w = sgprs(ops[0])
        return w | ({"exec_lo", "exec_hi"} if mn.startswith("v_cmpx") else set())
    carry = ("_co_", "v_addc", "v_subb", "v_mad_u64_u32", "v_mad_i64_i32", "v_div_scale")
    if any(c in mn for c in carry) and len(ops) > 1:
        return sgprs(ops[1])
    return set()


def sgprs_written_by_salu(ins: Instr) -> Set[str]:
    if not ins.mnemonic.startswith("s_") or not ins.operands:
        return set()
    if ins.mnemonic.startswith(("s_waitcnt", "s_nop", "s_barrier", "s_branch", "s_cbranch",
                                "s_endpgm", "s_setprio", "s_sleep", "s_store", "s_sendmsg")):
        return set()
    return sgprs(ins.operands[0])


def sgprs_read_by_vmem(ins: Instr) -> Set[str]:
    """Scalar registers a buffer instruction reads: descriptor, soffset, and
    M0 for a load into LDS."""
    regs: Set[str] = set()
    if ins.mnemonic.startswith(("buffer_", "tbuffer_")):
        for o in ins.operands[1:]:
            regs |= sgprs(o)
        if ins.is_lds_dma:
            regs.add("m0")
    elif ins.mnemonic.startswith(("global_", "scratch_")):
        for o in ins.operands[1:]:
            regs |= sgprs(o)
    return regs


def vmcnt_zero(ins: Instr) -> bool:
    """True for an s_waitcnt that waits for every vector-memory operation."""
    if ins.mnemonic != "s_waitcnt":
        return False
    ops = " ".join(ins.operands)
    if re.fullmatch(r"\s*0\s*", ops):
        return True
    m = re.search(r"vmcnt\((\d+)\)", ops)
    return bool(m) and int(m.group(1)) == 0


def parse_functions(asm: str) -> Dict[str, List[Tuple[int, str]]]:
    """name -> [(line number, line)] of every function body in the file."""
    names = set(re.findall(r"^\s*\.type\s+([^,\s]+),@function", asm, flags=re.M))
    funcs: Dict[str, List[Tuple[int, str]]] = {}
    cur: Optional[str] = None
    for i, line in enumerate(asm.splitlines(), 1):
        m = re.match(r"^([^\s:;]+):", line)
        if m and m.group(1) in names:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        if re.match(r"^\.Lfunc_end\d+:", line):
            cur = None
            continue
        funcs[cur].append((i, line))
    return funcs


def build_cfg(body: List[Tuple[int, str]]) -> List[Block]:
    blocks: List[Block] = [Block("<entry>")]
    label_of: Dict[str, int] = {}
    ended = False  # the current block ended with a terminator

    def new_block(label: str):
        nonlocal ended
        if blocks[-1].instrs or blocks[-1].label != "<entry>" or len(blocks) > 1:
            blocks.append(Block(label))
        else:
            blocks[-1].label = label
        ended = False

    for ln, raw in body:
        s = raw.strip()
        mb = re.match(r"^;\s*%bb\.\d+:", s)
        if mb:
            new_block(s)
            continue
        code = raw.split(";", 1)[0].strip()
        if not code or code.startswith("."):
            if code.startswith(".LBB") and code.endswith(":"):
                new_block(code[:-1])
                label_of[code[:-1]] = len(blocks) - 1
            continue
        m = re.match(r"^([^\s:;]+):$", code)
        if m:
            new_block(m.group(1))
            label_of[m.group(1)] = len(blocks) - 1
            continue
        parts = code.split(None, 1)
        ins = Instr(ln, parts[0], _split_operands(parts[1]) if len(parts) > 1 else [], code)
        if ended:
            new_block(f"<after {ln}>")
        blocks[-1].instrs.append(ins)
        if ins.mnemonic.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            ended = True
    # edges
    for i, b in enumerate(blocks):
        last = b.instrs[-1] if b.instrs else None
        fall = [i + 1] if i + 1 < len(blocks) else []
        if last is None:
            b.succs = fall
        elif last.mnemonic == "s_branch":
            b.succs = [label_of[last.operands[0]]]
        elif last.mnemonic.startswith("s_cbranch"):
            b.succs = [label_of[last.operands[0]]] + fall
        elif last.mnemonic.startswith(("s_endpgm", "s_setpc")):
            b.succs = []
        else:
            b.succs = fall
    for i, b in enumerate(blocks):
        for j in b.succs:
            blocks[j].preds.append(i)
    return blocks


def _dma_pending_out(blocks: List[Block]) -> List[bool]:
    """Per block: whether a load into LDS may be outstanding at its end (issued
    on some path with no ``s_waitcnt vmcnt(0)`` after it)."""
    out = [False] * len(blocks)
    changed = True
    while changed:
        changed = False
        for i, b in enumerate(blocks):
            pend = any(out[p] for p in b.preds)
            for ins in b.instrs:
                if ins.is_lds_dma:
                    pend = True
                elif vmcnt_zero(ins):
                    pend = False
            if pend != out[i]:
                out[i] = pend
                changed = True
    return out


def vmcnt_of(ins: Instr) -> Optional[int]:
    """The vmcnt an s_waitcnt waits for (None when it has no vmcnt field)."""
    if ins.mnemonic != "s_waitcnt":
        return None
    ops = " ".join(ins.operands)
    if re.fullmatch(r"\s*0\s*", ops):
        return 0
    m = re.search(r"vmcnt\((\d+)\)", ops)
    return int(m.group(1)) if m else None


def pending_vmcnt_waits(body: List[Tuple[int, str]]) -> List[Tuple[int, int]]:
    """(line, vmcnt) of every s_waitcnt with a vmcnt below 63 that a wave can
    reach while a load into LDS may be outstanding: the waits that order the
    reads of loaded buffers."""
    blocks = build_cfg(body)
    out = _dma_pending_out(blocks)
    found = []
    for b in blocks:
        pend = any(out[p] for p in b.preds)
        for ins in b.instrs:
            if ins.is_lds_dma:
                pend = True
                continue
            v = vmcnt_of(ins)
            if v is None or v >= 63:
                continue
            if pend:
                found.append((ins.line, v))
            if v == 0:
                pend = False
    return found


def check_kernel_asm(name: str, body: List[Tuple[int, str]]) -> List[str]:
    """Violations of conditions 1-3 in one function (empty when it holds
    them, or when it issues no load into LDS)."""
    blocks = build_cfg(body)
    all_ins = [ins for b in blocks for ins in b.instrs]
    if not any(ins.is_lds_dma for ins in all_ins):
        return []
    errs: List[str] = []
    short = name if len(name) < 90 else name[:87] + "..."
    # 1. scratch and calls
    for ins in all_ins:
        if ins.mnemonic.startswith("scratch_") or (
                ins.mnemonic.startswith("buffer_") and not ins.is_lds_dma and "off" in ins.operands
                and any(o.startswith("s[0:3]") for o in ins.operands)):
            errs.append(f"{short}: line {ins.line}: scratch access `{ins.text}`")
        if ins.mnemonic.startswith(("s_swappc", "s_setpc", "s_call")):
            errs.append(f"{short}: line {ins.line}: out-of-line call `{ins.text}`")
    # 2. may-be-outstanding loads into LDS, forward over the CFG
    out = _dma_pending_out(blocks)
    for i, b in enumerate(blocks):
        pend = any(out[p] for p in b.preds)
        for ins in b.instrs:
            if ins.is_lds_dma:
                pend = True
            elif vmcnt_zero(ins):
                pend = False
            elif pend and ins.is_vmem:
                errs.append(f"{short}: line {ins.line}: vector-memory instruction while a load "
                            f"into LDS may be outstanding `{ins.text}`")
    # 3. wait states before each vector-memory read of an SGPR / M0
    def hazards(bi: int, idx: int, regs: Set[str]) -> List[str]:
        found: List[str] = []
        seen: Set[Tuple[int, int]] = set()

        def walk(bj: int, k: int, ws: int):
            # k: index of the instruction just before the range still to scan
            while k >= 0:
                ins = blocks[bj].instrs[k]
                v = sgprs_written_by_valu(ins) & regs
                if v and ws < VALU_SGPR_TO_VMEM_WAIT:
                    found.append(f"VALU write of {sorted(v)} at line {ins.line} only {ws} wait "
                                 f"state(s) before")
                if "m0" in regs and "m0" in sgprs_written_by_salu(ins) and ws < SALU_M0_TO_LDS_DMA_WAIT:
                    found.append(f"SALU write of m0 at line {ins.line} only {ws} wait state(s) before")
                ws += ins.wait_states
                if ws >= VALU_SGPR_TO_VMEM_WAIT:
                    return
                k -= 1
            for p in blocks[bj].preds:
                if (p, ws) not in seen:
                    seen.add((p, ws))
                    walk(p, len(blocks[p].instrs) - 1, ws)

        walk(bi, idx - 1, 0)
        return found

    for bi, b in enumerate(blocks):
        for k, ins in enumerate(b.instrs):
            if not ins.is_vmem:
                continue
            regs = sgprs_read_by_vmem(ins)
            if not regs:
                continue
            for h in hazards(bi, k, regs):
                errs.append(f"{short}: line {ins.line} `{ins.text}`: {h}")
    return errs


def check_asm_text(asm: str) -> Tuple[List[str], List[str]]:
    """(checked function names, violations) for one assembly file."""
    checked, errs = [], []
    for name, body in parse_functions(asm).items():
        if any(re.search(r"\bbuffer_load_\w+\b.*\blds\b", l.split(";", 1)[0]) for _, l in body):
            checked.append(name)
            errs.extend(check_kernel_asm(name, body))
    return checked, errs


# ---------------------------------------------------------------- resources
_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|SGPRs Spill|VGPRs Spill|"
                     r"Dynamic Stack):\s*(\S+)")


def parse_resource_remarks(text: str) -> Dict[str, Dict[str, str]]:
    """Per-function fields of the compiler's kernel-resource-usage remarks."""
    out: Dict[str, Dict[str, str]] = {}
    cur = None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = val
            out[cur] = {}
        elif cur is not None:
            out[cur][key] = val
    return out


def resource_violations(remarks: Dict[str, Dict[str, str]], names) -> List[str]:
    """Non-zero scratch, spills or a dynamic stack in the named functions."""
    errs = []
    for n in names:
        r = remarks.get(n)
        if r is None:
            errs.append(f"{n}: no resource-usage remark")
            continue
        if r.get("ScratchSize [bytes/lane]", "0") != "0":
            errs.append(f"{n}: scratch {r['ScratchSize [bytes/lane]']} bytes per lane")
        for k in ("SGPRs Spill", "VGPRs Spill"):
            if r.get(k, "0") != "0":
                errs.append(f"{n}: {k} {r[k]}")
        if r.get("Dynamic Stack", "False") != "False":
            errs.append(f"{n}: dynamic stack")
    return errs
