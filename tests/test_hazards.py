"""The build-time MFMA operand hazard check (tiled_attention_16_amd/hazards.py).

A VALU write of a register needs two wait states before an MFMA reads it; the
checker must find every violation on straight-line code and across branches,
and accept code that keeps the distance.
"""
from tiled_attention_16_amd.hazards import check

HEAD = "_Z6kernelv:\n"
MFMA = "\tv_mfma_f32_32x32x16_bf16 v[0:15], a[4:7], a[0:3], v[0:15]\n"


def test_write_right_before_is_a_hazard():
    asm = HEAD + "\tv_accvgpr_write_b32 a3, v3\n" + MFMA
    assert len(check(asm)) == 1


def test_one_instruction_between_is_still_a_hazard():
    asm = HEAD + "\tv_accvgpr_write_b32 a5, v3\n\ts_mov_b32 s0, 0\n" + MFMA
    assert len(check(asm)) == 1


def test_two_wait_states_clear_it():
    assert check(HEAD + "\tv_accvgpr_write_b32 a3, v3\n\ts_nop 1\n" + MFMA) == []
    assert check(HEAD + "\tv_mov_b32 v7, v3\n\ts_mov_b32 s0, 0\n\ts_mov_b32 s1, 0\n" + MFMA) == []


def test_srcc_and_vgpr_writes_count():
    assert len(check(HEAD + "\tv_mul_f32_e32 v9, v1, v9\n" + MFMA)) == 1      # C operand
    assert check(HEAD + "\tv_mul_f32_e32 v16, v1, v16\n" + MFMA) == []         # not an operand


def test_unrelated_writes_and_mfma_chains_pass():
    asm = HEAD + "\tv_exp_f32_e32 v20, v21\n" + MFMA + MFMA   # MFMA -> MFMA is the hardware's job
    assert check(asm) == []


def test_hazard_through_a_branch():
    asm = (HEAD + "\tv_accvgpr_write_b32 a0, v3\n\ts_cbranch_scc1 .LBB0_2\n"
           "\ts_mov_b32 s0, 0\n\ts_mov_b32 s1, 0\n.LBB0_2:\n" + MFMA)
    # the fall-through path has two wait states; the branch path has only one
    assert len(check(asm)) == 1


def test_no_fall_through_after_unconditional_branch():
    asm = (HEAD + "\ts_branch .LBB0_3\n\tv_accvgpr_write_b32 a0, v3\n.LBB0_2:\n" + MFMA +
           ".LBB0_3:\n\ts_endpgm\n")
    # the write before the label is dead code reached only by falling through;
    # here it does fall through into .LBB0_2, so it is reported
    assert len(check(asm)) == 1
    asm2 = (HEAD + "\tv_accvgpr_write_b32 a0, v3\n\ts_branch .LBB0_3\n.LBB0_2:\n" + MFMA +
            ".LBB0_3:\n\ts_endpgm\n")
    assert check(asm2) == []


def test_mfma_result_read_too_soon():
    asm = HEAD + MFMA + "\tv_fma_f32 v40, s1, v3, v41\n"
    assert len(check(asm)) == 1
    padded = HEAD + MFMA + "\ts_nop 7\n\ts_nop 7\n\ts_nop 3\n\tv_fma_f32 v40, s1, v3, v41\n"
    assert check(padded) == []


def test_mfma_result_read_through_branch_and_chain():
    # the read sits behind a taken branch: still too close
    asm = HEAD + MFMA + "\ts_cbranch_scc1 .LBB0_5\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n.LBB0_5:\n\tv_add_f32_e32 v50, v2, v51\n"
    assert len(check(asm)) == 1
    # a later MFMA of the same chain takes over: only its own distance counts
    chain = HEAD + MFMA + MFMA + "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_add_f32_e32 v50, v2, v51\n"
    assert check(chain) == []
