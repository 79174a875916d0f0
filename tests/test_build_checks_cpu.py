"""The build's scan of the generated gfx950 code for LDS DMA hazards: a
buffer_load ... lds written as inline assembly is invisible to the compiler's
hazard recognizer, so the build itself rejects one that reads an SGPR fewer
than five wait states after a VALU instruction wrote it (gfx9 hazard rule for
vector memory instructions reading SGPRs)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from newton_schulz_muon_amd import build  # noqa: E402

DMA = "\tbuffer_load_dwordx4 v166, s[64:67], s15 offen lds\n"


def _asm(*body):
    # the entry label is followed by enough wait states not to count as a
    # branch target within reach of the DMA
    return "k:\n\ts_nop 7\n" + "\t; comment\n" + "".join("\t" + b + "\n" for b in body)


def test_valu_soffset_write_is_flagged():
    asm = _asm("s_mov_b32 m0, s8", "v_readfirstlane_b32 s15, v3", "v_add_u32_e32 v1, v2, v3", ";;#ASMSTART") + DMA
    found = build.dma_sgpr_hazards(asm)
    assert len(found) == 1 and "1 wait states after v_readfirstlane_b32 s15" in found[0], found


def test_five_wait_states_clear_it():
    asm = _asm("v_readfirstlane_b32 s15, v3", "s_nop 4") + DMA
    assert build.dma_sgpr_hazards(asm) == []
    asm = _asm("v_readfirstlane_b32 s15, v3", "s_nop 3") + DMA
    assert len(build.dma_sgpr_hazards(asm)) == 1
    asm = _asm("v_readfirstlane_b32 s15, v3", *["s_add_u32 s1, s2, s3"] * 5) + DMA
    assert build.dma_sgpr_hazards(asm) == []


def test_spill_restore_into_descriptor_is_flagged():
    asm = _asm("v_readlane_b32 s64, v234, 35", "v_readlane_b32 s65, v234, 36", "v_readlane_b32 s66, v234, 37",
               "v_readlane_b32 s67, v234, 38") + DMA
    assert len(build.dma_sgpr_hazards(asm)) == 4


def test_scalar_writes_and_other_sgprs_pass():
    asm = _asm("v_readfirstlane_b32 s14, v3", "s_mul_i32 s15, s14, s16", "v_cmp_gt_i32_e64 s[12:13], s1, v4") + DMA
    assert build.dma_sgpr_hazards(asm) == []


def test_carry_out_and_vcc_writes_are_defs():
    asm = _asm("v_add_co_u32_e64 v1, s[14:15], v2, v3") + DMA
    assert len(build.dma_sgpr_hazards(asm)) == 1
    dma_vcc = "\tbuffer_load_dwordx4 v1, s[104:107], s15 offen lds\n"
    assert len(build.dma_sgpr_hazards(_asm("v_cmp_lt_u32_e32 vcc, v1, v2") + dma_vcc)) == 1


def test_branch_target_within_window_is_flagged():
    asm = "k:\n\tv_readfirstlane_b32 s1, v1\n\ts_nop 7\n.LBB0_1:\n\ts_nop 0\n" + DMA
    found = build.dma_sgpr_hazards(asm)
    assert len(found) == 1 and "branch target" in found[0], found
