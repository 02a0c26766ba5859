"""The build's checks on synthetic assembly: no VALU result reaches an
inline-assembly MFMA operand with fewer than two wait states, no LDS-direct
load directly follows a write of M0 (the compiler's hazard recognizer does not
see through inline assembly in either case), no kernel uses scratch
memory, and the wide kernel's common-step score product keeps its LDS reads
ahead (no full LDS wait before any but its last MFMA)."""

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


LDS_LOAD = "\tbuffer_load_dwordx4 v204, s[24:27], 0 offen offset:0x80 lds\n"


def check_dma(tmp_path, text):
    p = tmp_path / "d.s"
    p.write_text(text)
    build.check_lds_dma_m0_hazards(str(p), "d")


def test_lds_load_right_after_an_m0_write_is_caught(tmp_path):
    with pytest.raises(RuntimeError):
        check_dma(tmp_path, "\ts_add_i32 m0, s14, s44\n" + LDS_LOAD)
    with pytest.raises(RuntimeError):
        check_dma(tmp_path, "\ts_mov_b32 m0, s6\n" + LDS_LOAD)


def test_one_wait_state_after_the_m0_write_is_enough(tmp_path):
    check_dma(tmp_path, "\ts_add_i32 m0, s14, s44\n\ts_nop 0\n" + LDS_LOAD)
    check_dma(tmp_path, "\ts_mov_b32 m0, s6\n\tv_lshlrev_b32_e32 v0, 2, v0\n" + LDS_LOAD)


def test_m0_write_before_a_branch_into_the_load_is_caught(tmp_path):
    text = ("\ts_mov_b32 m0, s6\n\ts_cbranch_scc1 .LBB0_2\n\ts_nop 0\n.LBB0_2:\n" + LDS_LOAD)
    with pytest.raises(RuntimeError):
        check_dma(tmp_path, text)


def test_the_kernels_pass_the_m0_check():
    for src in build.LDS_DMA_SOURCES:
        build.check_lds_dma(src)


SCRATCH = """\t.amdhsa_kernel k
\t\t.amdhsa_private_segment_fixed_size {size}
\t.end_amdhsa_kernel
\t.vgpr_spill_count: {spills}
"""


def test_scratch_use_without_a_spill_is_caught():
    with pytest.raises(RuntimeError, match="scratch memory"):
        build.check_no_scratch(SCRATCH.format(size=192, spills=0), "k")


def test_a_spill_is_caught():
    with pytest.raises(RuntimeError, match="spills"):
        build.check_no_scratch(SCRATCH.format(size=8, spills=2), "k")


def test_no_scratch_passes():
    build.check_no_scratch(SCRATCH.format(size=0, spills=0), "k")


def score_loop(waits):
    body = ["_ZN3mla12_GLOBAL__N_118decode_wide_kernelILb0EEEvNS_10DecodeArgsE:"]
    for w in waits:
        body += ["\tds_read_b128 v[28:31], v191 offset:4096", f"\ts_waitcnt lgkmcnt({w})",
                 "\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[28:31], v[32:35], v[0:15]", "\t;;#ASMEND"]
    body += ["\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[12:15], v[170:173], a[0:15]", "\t;;#ASMEND",
             "\t;;#ASMSTART", "\ts_nop 3", "\t;;#ASMEND"]
    return "\n".join(body) + "\n"


def test_score_reads_ahead_pass():
    import tempfile, os
    with tempfile.TemporaryDirectory() as td:
        p = os.path.join(td, "k.s")
        open(p, "w").write(score_loop([3] * 33 + [2, 1, 0]))
        build.check_score_reads_ahead(p, "k")


def test_full_lds_waits_in_the_score_loop_are_caught():
    import tempfile, os
    with tempfile.TemporaryDirectory() as td:
        p = os.path.join(td, "k.s")
        open(p, "w").write(score_loop(([0, 3, 3, 3] * 9)[:33] + [2, 1, 0]))
        with pytest.raises(RuntimeError, match="reads ahead are lost"):
            build.check_score_reads_ahead(p, "k")


def test_the_wide_kernel_keeps_its_score_reads_ahead():
    build.check_fixed_agprs("mla_decode_wide.hip")


# ---- M0 belongs to the wide kernel's chunk copies

COPY = ("\ts_add_u32 m0, s12, 0x3c00\n\ts_nop 0\n"
        "\tbuffer_load_dwordx4 v2, s[8:11], 0 offen offset:128 lds\n")


def test_copies_alone_pass_the_m0_ownership_check():
    build.check_m0_only_in_copies(COPY * 3, "k")


def test_a_compiler_use_of_m0_is_caught():
    for extra in ("\ts_mov_b32 m0, s4\n", "\tv_movrels_b32_e32 v1, v2\n\ts_mov_b32 m0, -1\n",
                  "\tds_read_b32 v1, v0\n\ts_add_u32 m0, s1, s2\n"):
        with pytest.raises(RuntimeError, match="M0 is used outside"):
            build.check_m0_only_in_copies(COPY + extra + COPY, "k")
