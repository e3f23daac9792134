"""The build's assembly check for global->LDS loads whose scalar base address
was written by a vector instruction without the required wait states (CPU)."""
from causal_video_diffusion_amd.build import check_dma_base_hazards


def test_vector_written_base_is_flagged():
    asm = """
\tv_readfirstlane_b32 s1, v15
\tv_readfirstlane_b32 s0, v14
\t;;#ASMSTART
\tglobal_load_lds_dwordx4 v225, s[0:1]
\t;;#ASMEND
"""
    found = check_dma_base_hazards(asm)
    assert len(found) == 1 and "v_readfirstlane_b32 s0, v14" in found[0]


def test_scalar_written_base_and_enough_wait_states_pass():
    salu = """
\ts_add_u32 s4, s50, s4
\ts_mov_b32 m0, s6
\ts_addc_u32 s5, s51, s5
\t;;#ASMSTART
\tglobal_load_lds_dwordx4 v238, s[4:5]
\t;;#ASMEND
"""
    nops = """
\tv_readfirstlane_b32 s0, v14
\ts_nop 4
\tglobal_load_lds_dwordx4 v225, s[0:1]
"""
    far = "\tv_readlane_b32 s9, v253, 3\n" + "\ts_add_i32 s20, s20, 1\n" * 5 + \
          "\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    other = "\tv_readfirstlane_b32 s2, v4\n\tglobal_load_lds_dwordx4 v1, s[0:1]\n"
    for asm in (salu, nops, far, other):
        assert check_dma_base_hazards(asm) == []


def test_too_few_wait_states_are_flagged_on_every_path_into_a_block():
    short = "\tv_readlane_b32 s9, v253, 3\n\ts_nop 2\n\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    assert len(check_dma_base_hazards(short)) == 1
    # the write reaches the load through a taken branch
    branch = """
\tv_readfirstlane_b32 s4, v1
\ts_cbranch_scc1 .LBB0_7
\ts_mov_b32 s20, 0
\ts_branch .LBB0_8
.LBB0_7:
\tglobal_load_lds_dwordx4 v1, s[4:5]
.LBB0_8:
\ts_endpgm
"""
    assert len(check_dma_base_hazards(branch)) == 1
    # ... and through a fall-through into the load's block
    fall = "\tv_readfirstlane_b32 s5, v1\n.LBB0_9:\n\tglobal_load_lds_dwordx4 v1, s[4:5]\n"
    assert len(check_dma_base_hazards(fall)) == 1
    # clean on both paths: the branch source wrote the base with a scalar op,
    # and the block is not entered by falling through
    clean = branch.replace("v_readfirstlane_b32 s4, v1", "s_mov_b32 s4, s30")
    assert check_dma_base_hazards(clean) == []
