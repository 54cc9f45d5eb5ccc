"""The build's static check for early reads of inline MFMA results (CPU only)."""

import os

import pytest

from long_context_prefix_amd import build
from long_context_prefix_amd.isa_check import inline_mfma_hazards

MFMA = "v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0"


def _asm(*after):
    return "\n".join(["_Zk:", ";;#ASMSTART", MFMA, ";;#ASMEND", *after])


def test_early_valu_read_is_found():
    assert len(inline_mfma_hazards(_asm("v_add_f32 v1, v2, v3", "v_mov_b32 v40, v12"))) == 1


def test_early_store_is_found():
    assert len(inline_mfma_hazards(_asm("global_store_dwordx4 v[0:1], v[22:25], off"))) == 1


def test_guarded_read_is_clean():
    # 16 wait states of s_nop plus 8 instructions: the read comes after 24 wait states
    asm = _asm("s_nop 7", "s_nop 7", *(["v_add_f32 v1, v2, v3"] * 8), "v_mov_b32 v40, v12")
    assert inline_mfma_hazards(asm) == []
    # one instruction fewer is one wait state short
    asm = _asm("s_nop 7", "s_nop 7", *(["v_add_f32 v1, v2, v3"] * 7), "v_mov_b32 v40, v12")
    assert len(inline_mfma_hazards(asm)) == 1


def test_accumulation_chain_and_unrelated_reads_are_clean():
    asm = _asm(";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], v[10:25]", ";;#ASMEND",
               "v_add_f32 v1, v2, v3", "v_mov_b32 v40, v9")
    # the second MFMA is itself inline: its own readers are checked too (none here)
    assert inline_mfma_hazards(asm) == []


def test_built_library_assembly_is_clean():
    if not os.path.exists(build.ASM):
        pytest.skip("library not built here")
    text = open(build.ASM).read()
    assert "v_mfma_f32_32x32x16_bf16 v[" in text  # the inline score MFMAs are present
    assert inline_mfma_hazards(text) == []


AGPR_MFMA = "v_mfma_f32_32x32x16_bf16 a[16:31], v[2:5], v[6:9], a[16:31]"


def _asm_a(*after, before=()):
    return "\n".join(["_Zk:", *before, ";;#ASMSTART", AGPR_MFMA, ";;#ASMEND", *after])


def test_early_accvgpr_read_of_an_agpr_result_is_found():
    assert len(inline_mfma_hazards(_asm_a("v_accvgpr_read_b32 v40, a20"))) == 1
    # an AGPR outside the result is fine
    assert inline_mfma_hazards(_asm_a("v_accvgpr_read_b32 v40, a40")) == []


def test_early_spill_of_an_agpr_result_is_found():
    assert len(inline_mfma_hazards(_asm_a("scratch_store_dwordx4 off, a[16:19], off"))) == 1


def test_early_overwrite_of_a_result_is_found():
    assert len(inline_mfma_hazards(_asm_a("v_accvgpr_write_b32 a17, v3"))) == 1
    assert len(inline_mfma_hazards(_asm("v_mov_b32 v12, 0"))) == 1  # VGPR result overwritten by VALU
    assert len(inline_mfma_hazards(_asm("ds_read_b128 v[10:13], v1"))) == 1  # ... or by a load


def test_guarded_agpr_read_is_clean():
    asm = _asm_a("s_nop 7", "s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v40, a20")
    assert inline_mfma_hazards(asm) == []


def test_operand_written_just_before_an_inline_mfma_is_found():
    # a VALU write of the B operand right before the MFMA
    assert len(inline_mfma_hazards(_asm_a(before=("v_cvt_pk_bf16_f32 v7, v40, v41",)))) == 1
    # of the accumulator (an AGPR) through v_accvgpr_write
    assert len(inline_mfma_hazards(_asm_a(before=("v_accvgpr_write_b32 a16, v3",)))) == 1
    # four wait states in between are enough
    asm = _asm_a(before=("v_cvt_pk_bf16_f32 v7, v40, v41", "s_nop 3"))
    assert inline_mfma_hazards(asm) == []
    # an unrelated write is fine
    assert inline_mfma_hazards(_asm_a(before=("v_cvt_pk_bf16_f32 v70, v40, v41",))) == []


def test_scratch_use_of_forward_kernels_is_found():
    from long_context_prefix_amd.isa_check import private_segment_sizes, scratch_findings

    def desc(name, n):
        return f"\t.amdhsa_kernel {name}\n\t\t.amdhsa_group_segment_fixed_size 0\n" \
               f"\t\t.amdhsa_private_segment_fixed_size {n}\n\t.end_amdhsa_kernel\n"

    fwd = "_ZN3lcp15attn_fwd_kernelINS_7Bf16DmaILi128EEELi128ELb1ELi2ELb1ELb0EEEvNS_7FwdArgsE"
    wide = "_ZN3lcp20attn_fwd_wide_kernelILi256ELb0ELb0EEEvNS_7FwdArgsE"
    f32 = "_ZN3lcp15attn_fwd_kernelINS_7F32PathILi256EEELi256ELb0ELi1ELb0ELb0EEEvNS_7FwdArgsE"
    bwd = "_ZN3lcp20bwd_dkdv_slot_kernelILi256ELi1EEEvNS_7BwdArgsE"
    asm = desc(fwd, 36) + desc(wide, 0) + desc(f32, 844) + desc(bwd, 8)
    assert private_segment_sizes(asm) == {fwd: 36, wide: 0, f32: 844, bwd: 8}
    found = scratch_findings(asm)
    assert len(found) == 1 and fwd in found[0]  # the fp32 path and the backward are not covered
    assert scratch_findings(desc(fwd, 0) + desc(wide, 0)) == []
    assert len(scratch_findings(desc(wide, 4))) == 1


def test_built_forward_kernels_use_no_scratch():
    from long_context_prefix_amd.isa_check import private_segment_sizes, scratch_findings

    if not os.path.exists(build.ASM):
        pytest.skip("library not built here")
    text = open(build.ASM).read()
    sizes = private_segment_sizes(text)
    assert any("Bf16DmaILi128" in k for k in sizes)  # the D = 128 forward kernels are in the build
    assert scratch_findings(text) == []


def test_a_block_the_common_path_branches_over_is_no_distance():
    # the read after the label is reached by the branch after two instructions, not 40
    asm = _asm("s_nop 7", "s_cbranch_scc1 .LBB0_2", *(["v_add_f32 v1, v2, v3"] * 40), ".LBB0_2:",
               "v_mov_b32 v40, v12")
    assert len(inline_mfma_hazards(asm)) == 1
    # a jump skips the instructions after it as well
    asm = _asm("s_branch .LBB0_3", *(["v_add_f32 v1, v2, v3"] * 40), ".LBB0_3:", "v_mov_b32 v40, v12")
    assert len(inline_mfma_hazards(asm)) == 1
    # enough distance on the branch path too: clean
    asm = _asm("s_nop 7", "s_nop 7", "s_nop 7", "s_cbranch_scc1 .LBB0_4", "v_add_f32 v1, v2, v3", ".LBB0_4:",
               "v_mov_b32 v40, v12")
    assert inline_mfma_hazards(asm) == []


def test_an_operand_written_at_the_end_of_a_loop_is_found():
    # the loop's back edge brings the VALU write right before the MFMA at the loop head
    asm = "\n".join(["_Zk:", "s_mov_b32 s0, 0", ".LBB0_1:", ";;#ASMSTART", AGPR_MFMA, ";;#ASMEND",
                     *(["v_add_f32 v1, v2, v3"] * 30), "v_cvt_pk_bf16_f32 v7, v40, v41", "s_cbranch_scc1 .LBB0_1"])
    assert len(inline_mfma_hazards(asm)) == 1
