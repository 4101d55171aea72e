"""The static checks of kernels that load memory straight into LDS
(blockwise_attention_ffn_amd/asm_check.py), on the CPU.

Synthetic assembly in the LLVM AMDGPU printer's format plants one violation
at a time (a store or a plain load while a load into LDS may be outstanding,
also across a loop's back edge; scratch access; an out-of-line call; a VALU
write of a descriptor SGPR or an SALU write of M0 too close before the load)
and the checker must report each; the clean variants must pass. Then the
library's real sources are compiled to assembly and must pass every check.
"""
import pytest

from blockwise_attention_ffn_amd import asm_check as C
from blockwise_attention_ffn_amd import build as B

HEAD = """\t.text
\t.type\tk,@function
k:
; %bb.0:
\ts_load_dwordx4 s[4:7], s[0:1], 0x0
\tv_readfirstlane_b32 s20, v1
\ts_mov_b32 s21, 0
\ts_mov_b32 s22, 0x1000
\ts_mov_b32 s23, 0x20000
\tv_mov_b32 v2, 0
\tv_mov_b32 v3, 0
\tv_mov_b32 v4, 0
\tv_mov_b32 v5, 0
"""
DMA = """\ts_mov_b32 m0, s8
\t;;#ASMSTART
\ts_nop 0
\tbuffer_load_dwordx4 v15, s[20:23], 0 offen lds
\t;;#ASMEND
"""
TAIL = """\ts_waitcnt vmcnt(0)
\tglobal_store_dword v[0:1], v2, off
\ts_endpgm
.Lfunc_end0:
"""


def errs_of(body):
    return C.check_asm_text(HEAD + body + TAIL)[1]


def test_clean_kernel_passes():
    assert errs_of(DMA + "\ts_waitcnt vmcnt(0)\n\ts_barrier\n\tds_read_b128 v[4:7], v3\n") == []


def test_store_while_load_outstanding():
    e = errs_of(DMA + "\tglobal_store_dword v[0:1], v2, off\n")
    assert len(e) == 1 and "may be outstanding" in e[0]


def test_plain_load_while_load_outstanding():
    e = errs_of(DMA + "\ts_waitcnt vmcnt(1)\n\tglobal_load_dword v9, v[0:1], off\n")
    assert len(e) == 1 and "may be outstanding" in e[0]


def test_waitcnt_zero_clears_the_window():
    assert errs_of(DMA + "\ts_waitcnt vmcnt(0) lgkmcnt(0)\n\tglobal_load_dword v9, v[0:1], off\n") == []


def test_window_follows_the_back_edge():
    # the load into LDS at the end of the loop body is outstanding at the
    # loop header, where a store sits before any wait
    body = (".LBB0_1:\n\tglobal_store_dword v[0:1], v2, off\n" + DMA +
            "\ts_cmp_lg_u32 s9, 0\n\ts_cbranch_scc1 .LBB0_1\n; %bb.2:\n")
    e = errs_of(body)
    assert len(e) == 1 and "may be outstanding" in e[0]


def test_window_across_an_out_of_line_block():
    # a cold block laid out after the wait at the end, reached from inside the window
    body = (DMA + "\ts_cbranch_vccnz .LBB0_9\n; %bb.1:\n\ts_waitcnt vmcnt(0)\n\ts_branch .LBB0_8\n"
            ".LBB0_9:\n\tglobal_store_dword v[0:1], v2, off\n\ts_waitcnt vmcnt(0)\n"
            ".LBB0_8:\n")
    e = errs_of(body)
    assert len(e) == 1 and "may be outstanding" in e[0]


def test_scratch_and_calls():
    e = errs_of("\tscratch_store_dwordx2 off, v[2:3], off\n" + DMA +
                "\ts_waitcnt vmcnt(0)\n\ts_swappc_b64 s[30:31], s[16:17]\n")
    assert any("scratch access" in x for x in e)
    assert any("out-of-line call" in x for x in e)


def test_valu_write_of_descriptor_too_close():
    e = errs_of("\tv_readfirstlane_b32 s22, v7\n" + DMA + "\ts_waitcnt vmcnt(0)\n")
    assert len(e) == 1 and "VALU write of ['s22']" in e[0]
    # five wait states in between are enough
    ok = "\tv_readfirstlane_b32 s22, v7\n\ts_nop 4\n" + DMA + "\ts_waitcnt vmcnt(0)\n"
    assert errs_of(ok) == []


def test_valu_carry_out_counts_as_an_sgpr_write():
    e = errs_of("\tv_mad_u64_u32 v[4:5], s[20:21], v3, s4, v[2:3]\n" + DMA + "\ts_waitcnt vmcnt(0)\n")
    assert len(e) == 1 and "s20" in e[0]


def test_valu_write_reaches_through_a_predecessor():
    body = ("\tv_readfirstlane_b32 s21, v7\n\ts_branch .LBB0_3\n.LBB0_3:\n" + DMA +
            "\ts_waitcnt vmcnt(0)\n")
    e = errs_of(body)
    assert len(e) == 1 and "s21" in e[0]


def test_salu_m0_write_needs_one_wait_state():
    bad = ("\ts_mov_b32 m0, s8\n\t;;#ASMSTART\n\tbuffer_load_dwordx4 v15, s[20:23], 0 offen lds\n"
           "\t;;#ASMEND\n\ts_waitcnt vmcnt(0)\n")
    e = errs_of(bad)
    assert len(e) == 1 and "m0" in e[0]
    assert errs_of(DMA + "\ts_waitcnt vmcnt(0)\n") == []


def test_resource_remarks():
    text = "\n".join([
        "x.hip:1:1: remark: Function Name: k1 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark: Function Name: k2 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]",
    ])
    r = C.parse_resource_remarks(text)
    assert C.resource_violations(r, ["k1"]) == []
    e = C.resource_violations(r, ["k2", "k3"])
    assert any("scratch 16" in x for x in e) and any("VGPRs Spill 2" in x for x in e)
    assert any("k3: no resource-usage remark" in x for x in e)


@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip") and B.uses_lds_dma(s)])
def test_library_sources_pass(src, library_asm):
    checked, errs, _ = library_asm[src]
    assert checked, f"no kernel with loads into LDS found in {src}"
    assert errs == [], "\n".join(errs)
