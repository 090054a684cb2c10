"""The build's check for accumulator accesses too soon after an inline-asm
MFMA (transformer_attn_bwd_amd/hazards.py), on small assembly snippets and
on the device assembly of the last build."""
import glob
import os

import pytest

from transformer_attn_bwd_amd.hazards import check_asm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HEAD = "_ZN4attn6kernelEv:\n"
MFMA = "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n"
WAIT = "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n"
END = "\ts_endpgm\n.Lfunc_end0:\n"


def test_read_right_after_the_mfma_is_reported():
    v = check_asm(HEAD + MFMA + "\tv_accvgpr_read_b32 v8, a3\n" + WAIT + END)
    assert len(v) == 1 and "a3" in v[0]


def test_read_after_the_wait_passes():
    assert check_asm(HEAD + MFMA + WAIT + "\tv_accvgpr_read_b32 v8, a3\n" + END) == []


def test_write_and_store_of_an_accumulator_count_too():
    asm = HEAD + MFMA + "\tv_accvgpr_write_b32 a0, 0\n\tglobal_store_dword v[2:3], a5, off\n" + END
    assert len(check_asm(asm)) == 2


def test_vgpr_mfma_results_and_plain_vgpr_code_are_not_flagged():
    asm = (HEAD + "\tv_mfma_f32_32x32x16_bf16 v[8:23], v[0:3], v[4:7], 0\n"
           "\tv_add_f32_e32 v30, v8, v9\n" + MFMA + "\tv_mul_f32_e32 v31, v30, v30\n" + END)
    assert check_asm(asm) == []


def test_a_loop_exit_reached_by_a_jump_is_checked():
    # the loop body ends in an MFMA and jumps to an exit block placed elsewhere
    asm = (HEAD + "\ts_branch .LBB0_2\n.LBB0_1:\n\tv_accvgpr_read_b32 v8, a3\n" + WAIT +
           "\ts_endpgm\n.LBB0_2:\n" + MFMA + "\ts_cbranch_scc1 .LBB0_2\n\ts_branch .LBB0_1\n"
           ".Lfunc_end0:\n")
    v = check_asm(asm)
    assert len(v) == 1 and "a3" in v[0]


def test_a_block_only_reached_before_any_mfma_is_clean():
    # zeroing of accumulators in a block that the MFMA loop never reaches
    asm = (HEAD + "\ts_cbranch_scc1 .LBB0_3\n" + MFMA + WAIT + "\ts_branch .LBB0_4\n"
           ".LBB0_3:\n\tv_accvgpr_write_b32 a0, 0\n.LBB0_4:\n" + END)
    assert check_asm(asm) == []


def test_last_build_is_clean():
    files = glob.glob(os.path.join(ROOT, "_build", "*", "*-hip-amdgcn-amd-amdhsa-gfx950.s"))
    if not files:
        pytest.skip("no device assembly in _build (run the build first)")
    found = []
    for f in files:
        with open(f) as fh:
            found += check_asm(fh.read())
    assert found == [], found[:5]


def test_operand_written_just_before_the_mfma_is_reported():
    asm = HEAD + "\tv_cvt_pk_bf16_f32 v5, v10, v11\n" + MFMA + WAIT + END
    v = check_asm(asm)
    assert len(v) == 1 and "v5" in v[0]


def test_operand_written_two_wait_states_before_passes():
    asm = HEAD + "\tv_cvt_pk_bf16_f32 v5, v10, v11\n\ts_nop 1\n" + MFMA + WAIT + END
    assert check_asm(asm) == []
    asm = HEAD + "\tv_cvt_pk_bf16_f32 v5, v10, v11\n\tv_add_f32_e32 v20, v21, v22\n" \
        "\ts_add_i32 s0, s0, 1\n" + MFMA + WAIT + END
    assert check_asm(asm) == []


def test_other_agprs_are_free_right_after_the_mfma():
    # a20 is not written by the MFMA (a value the compiler parked in an AGPR)
    asm = HEAD + MFMA + "\tv_accvgpr_read_b32 v8, a20\n\tv_accvgpr_write_b32 a16, v9\n" + WAIT + END
    assert check_asm(asm) == []
    asm = HEAD + MFMA + "\tv_accvgpr_read_b32 v8, a15\n" + WAIT + END
    assert len(check_asm(asm)) == 1
