"""The build-time MFMA wait-state check (transformer_exact_attention_amd.asm_check)."""
import os

import pytest

from transformer_exact_attention_amd import asm_check

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"


def block(*lines):
    return "\n".join(["\t" + x for x in lines])


def asm_mfma():
    return block(";;#ASMSTART", MFMA, ";;#ASMEND")


def test_clean_sequence_passes():
    text = block("v_cvt_pk_bf16_f32 v8, v1, v2", "v_add_f32_e32 v20, v21, v22", "s_nop 0") + "\n" + asm_mfma()
    assert asm_check.check(text) == []
    assert asm_check.count_asm_mfma(text) == 1


def test_vector_write_to_operand_right_before_is_flagged():
    text = block("v_accvgpr_read_b32 v9, a40") + "\n" + asm_mfma()
    assert len(asm_check.check(text)) == 1


def test_write_two_instructions_before_is_flagged_but_three_is_not():
    two = block("v_mov_b32_e32 v5, 0", "s_mov_b32 m0, s2") + "\n" + asm_mfma()
    three = block("v_mov_b32_e32 v5, 0", "s_mov_b32 m0, s2", "s_add_i32 s3, s3, 1") + "\n" + asm_mfma()
    assert len(asm_check.check(two)) == 1
    assert asm_check.check(three) == []


def test_nop_counts_its_wait_states():
    assert asm_check.check(block("v_mov_b32_e32 v10, 0", "s_nop 1") + "\n" + asm_mfma()) == []
    assert len(asm_check.check(block("v_mov_b32_e32 v10, 0", "s_nop 0") + "\n" + asm_mfma())) == 1


def test_label_inside_window_is_flagged():
    text = block("v_add_f32_e32 v30, v31, v32") + "\n.LBB0_3:\n" + asm_mfma()
    assert len(asm_check.check(text)) == 1


def test_mfma_outside_asm_blocks_is_ignored():
    assert asm_check.check(block("v_mov_b32_e32 v5, 0", MFMA)) == []


def test_built_prefill_assembly_if_present():
    path = os.path.join(ROOT, "_build", "prefill_bf16.hip.s")
    if not os.path.exists(path):
        pytest.skip("library not built in this tree")
    text = open(path).read()
    assert asm_check.count_asm_mfma(text) > 0
    assert asm_check.check(text) == []
