"""The build's check that no VALU result reaches an inline-assembly MFMA operand
with fewer than two wait states (the compiler's hazard recognizer does not see
assembly MFMAs), on synthetic assembly."""

import pytest

from paged_mla_decode_04_amd import build

MFMA = "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[180:183], v[4:7], v[0:15]\n"


def check(tmp_path, text):
    p = tmp_path / "k.s"
    p.write_text(text)
    build.check_mfma_operand_hazards(str(p), "k")


def test_write_right_before_the_mfma_is_caught(tmp_path):
    with pytest.raises(RuntimeError):
        check(tmp_path, "\tv_mov_b32 v5, 0\n" + MFMA)


def test_two_wait_states_are_enough(tmp_path):
    check(tmp_path, "\tv_mov_b32 v5, 0\n\ts_nop 1\n" + MFMA)
    check(tmp_path, "\tv_mov_b32 v5, 0\n\ts_add_i32 s0, s0, 1\n\ts_add_i32 s1, s1, 1\n" + MFMA)


def test_unrelated_registers_pass(tmp_path):
    check(tmp_path, "\tv_mov_b32 v20, 0\n" + MFMA)  # outside v[0:15], v[4:7], v[180:183]


def test_accumulator_source_counts(tmp_path):
    with pytest.raises(RuntimeError):
        check(tmp_path, "\tv_add_f32_e32 v3, v1, v2\n" + MFMA)


def test_paths_through_a_branch_are_followed(tmp_path):
    text = ("\tv_mov_b32 v5, 0\n\ts_cbranch_scc1 .LBB0_2\n\tv_add_f32_e32 v9, v1, v2\n"
            "\ts_nop 3\n.LBB0_2:\n" + MFMA)
    with pytest.raises(RuntimeError):
        check(tmp_path, text)


def test_fall_through_after_an_unconditional_branch_is_not_a_path(tmp_path):
    text = ("\tv_mov_b32 v5, 0\n\ts_branch .LBB0_3\n.LBB0_2:\n\ts_nop 1\n" + MFMA +
            ".LBB0_3:\n\ts_endpgm\n")
    check(tmp_path, text)
