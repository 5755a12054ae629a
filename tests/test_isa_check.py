"""The build's assembly check for LDS-DMA wait-state hazards
(block_diffusion_amd.isa_check) on small hand-written listings: a VALU
write of the DMA's SGPR base or of M0 within five wait states is reported,
five wait states (s_nop 4) in between are not; the walk follows the
fall-through path across block labels (unless an unconditional branch ends
the previous block) and every branch to a label."""
from block_diffusion_amd import isa_check

HDR = "_ZN3dbd6kernelEv:\n"


def _scan(body):
    return isa_check.scan(HDR + body)


def test_flags_valu_sgpr_write_before_dma():
    n, h = _scan("\tv_readlane_b32 s5, v255, 5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v24, s[4:5]\n")
    assert n == 1 and len(h) == 1 and h[0][3].startswith("v_readlane_b32 s5")


def test_flags_valu_m0_write():
    n, h = _scan("\tv_readfirstlane_b32 m0, v3\n\tglobal_load_lds_dwordx4 v[2:3], off\n")
    assert len(h) == 1


def test_five_wait_states_are_enough():
    n, h = _scan("\tv_readlane_b32 s5, v255, 5\n\ts_nop 4\n\tglobal_load_lds_dwordx4 v24, s[4:5]\n")
    assert n == 1 and h == []
    n, h = _scan("\tv_readlane_b32 s5, v255, 5\n\ts_nop 3\n\tglobal_load_lds_dwordx4 v24, s[4:5]\n")
    assert len(h) == 1


def test_other_registers_and_salu_writes_pass():
    body = ("\tv_readlane_b32 s6, v255, 6\n\ts_add_i32 m0, s3, 0x400\n\ts_mov_b32 s5, s9\n"
            "\t;;#ASMSTART\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v2, s[4:5]\n\t;;#ASMEND\n")
    assert _scan(body)[1] == []


def test_fall_through_across_a_label_is_followed():
    body = "\tv_readlane_b32 s5, v255, 5\n.LBB0_3:\n\tglobal_load_lds_dwordx4 v2, s[4:5]\n"
    assert len(_scan(body)[1]) == 1
    body = "\tv_readlane_b32 s5, v255, 5\n\ts_branch .LBB0_9\n.LBB0_3:\n\tglobal_load_lds_dwordx4 v2, s[4:5]\n"
    assert _scan(body)[1] == []


def test_branch_sources_are_followed():
    body = ("\tv_readlane_b32 s5, v255, 5\n\ts_cbranch_scc1 .LBB0_3\n\ts_mov_b32 s7, 0\n"
            "\ts_nop 7\n\ts_branch .LBB0_9\n.LBB0_3:\n\tglobal_load_lds_dwordx4 v2, s[4:5]\n")
    assert len(_scan(body)[1]) == 1
    body = ("\tv_readlane_b32 s5, v255, 5\n\ts_nop 4\n\ts_cbranch_scc1 .LBB0_3\n\ts_branch .LBB0_9\n"
            ".LBB0_3:\n\tglobal_load_lds_dwordx4 v2, s[4:5]\n")
    assert _scan(body)[1] == []


def test_stage_base_moved_by_scalar_arithmetic():
    # the prefill's full-stage loads: the 64-bit base advanced by scalar
    # multiply and add-with-carry (SALU writes need no wait states) ...
    body = ("\ts_mul_hi_u32 s1, s55, s22\n\ts_mul_i32 s0, s55, s22\n\ts_lshl_b64 s[0:1], s[0:1], 5\n"
            "\ts_add_u32 s0, s6, s0\n\ts_addc_u32 s1, s7, s1\n\ts_add_i32 m0, s53, s47\n"
            "\ts_nop 4\n\tglobal_load_lds_dwordx4 v120, s[0:1]\n")
    n, h = _scan(body)
    assert n == 1 and h == []
    # ... but the same base taken from a VALU lane read needs five
    body = ("\tv_readfirstlane_b32 s1, v7\n\ts_add_i32 m0, s53, s47\n"
            "\ts_nop 0\n\tglobal_load_lds_dwordx4 v120, s[0:1]\n")
    n, h = _scan(body)
    assert n == 1 and len(h) == 1 and h[0][3].startswith("v_readfirstlane_b32 s1")
