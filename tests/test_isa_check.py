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
