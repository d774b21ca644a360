"""The build-time MFMA wait-state check (transformer_exact_attention_amd.asm_check)."""
import os

import pytest

from transformer_exact_attention_amd import asm_check

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"
MFMA_V = "v_mfma_f32_32x32x16_bf16 v[40:55], v[4:7], a[8:11], v[40:55]"


def block(*lines):
    return "\n".join(["\t" + x for x in lines])


def asm(mfma=MFMA):
    return block(";;#ASMSTART", mfma, ";;#ASMEND")


def join(*parts):
    return "\n".join(parts)


# ---- sources written too soon before an asm MFMA ----------------------------

def test_clean_sequence_passes():
    text = join(block("v_cvt_pk_bf16_f32 v8, v1, v2", "v_add_f32_e32 v20, v21, v22", "s_nop 0"), asm())
    assert asm_check.check_all(text) == []
    assert asm_check.count_asm_mfma(text) == 1


def test_vector_write_to_operand_right_before_is_flagged():
    assert len(asm_check.check(join(block("v_accvgpr_read_b32 v9, a40"), asm()))) == 1


def test_write_two_instructions_before_is_flagged_but_three_is_not():
    two = join(block("v_mov_b32_e32 v5, 0", "s_mov_b32 m0, s2"), asm())
    three = join(block("v_mov_b32_e32 v5, 0", "s_mov_b32 m0, s2", "s_add_i32 s3, s3, 1"), asm())
    assert len(asm_check.check(two)) == 1
    assert asm_check.check(three) == []


def test_nop_counts_its_wait_states():
    assert asm_check.check(join(block("v_mov_b32_e32 v10, 0", "s_nop 1"), asm())) == []
    assert len(asm_check.check(join(block("v_mov_b32_e32 v10, 0", "s_nop 0"), asm()))) == 1


def test_write_on_a_branch_into_the_label_is_flagged():
    text = join(block("v_mov_b32_e32 v6, 1", "s_cbranch_scc1 .LBB0_3", "s_add_i32 s3, s3, 1",
                      "s_add_i32 s3, s3, 1"), ".LBB0_3:", asm())
    assert len(asm_check.check(text)) == 1
    safe = join(block("v_mov_b32_e32 v6, 1", "s_nop 1", "s_cbranch_scc1 .LBB0_3", "s_add_i32 s3, s3, 1",
                      "s_add_i32 s3, s3, 1"), ".LBB0_3:", asm())
    assert asm_check.check(safe) == []


def test_mfma_outside_asm_blocks_is_ignored():
    assert asm_check.check_all(block("v_mov_b32_e32 v5, 0", MFMA)) == []


# ---- results used too soon after an asm MFMA ---------------------------------

def test_result_read_soon_after_is_flagged():
    assert len(asm_check.check_results(join(asm(MFMA_V), block("v_add_f32_e32 v1, v41, v2")))) == 1


def test_result_read_after_enough_wait_states_passes():
    text = join(asm(MFMA_V), block("s_nop 7", "s_nop 7", "s_nop 7", "v_add_f32_e32 v1, v41, v2"))
    assert asm_check.check_results(text) == []


def test_accumulating_mfma_needs_no_wait_states():
    assert asm_check.check_results(join(asm(MFMA_V), asm(MFMA_V))) == []


def test_result_read_on_a_branch_target_is_flagged():
    text = join(asm(MFMA_V), block("s_cbranch_vccz .LBB0_7", "s_nop 7", "s_nop 7", "s_nop 7"),
                ".LBB0_7:", block("v_mul_f32_e32 v45, v45, v3"))
    assert len(asm_check.check_results(text)) == 1


def test_built_prefill_assembly_if_present():
    path = os.path.join(ROOT, "_build", "prefill_bf16.hip.s")
    if not os.path.exists(path):
        pytest.skip("library not built in this tree")
    text = open(path).read()
    assert asm_check.count_asm_mfma(text) > 0
    assert asm_check.check_all(text) == []
